/*
 * oracle_checks.c -- drives the float64 oracle (oracle/pa_oracle.c) over
 * seeded small problems for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitized_host.py).  Every buffer is
 * allocated at its exact size, so a read past the page pool, a page-table
 * row, a tail slot or the output is reported by the sanitizer.  The oracle
 * must return 0, give finite results (lse = -inf only for empty contexts),
 * agree with its partitioned form, and reject page ids outside the pool
 * without reading through them.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pa_oracle_decode(int B, int Hq, int Hkv, int D, int page_size, int q_dtype, const void* q,
                     int kv_dtype, const void* k_cache, const void* v_cache, int num_pages,
                     int64_t stride_page, int64_t stride_head, int64_t stride_slot,
                     const int32_t* page_table, int pt_stride, const int32_t* context_lens,
                     double scale, int window, int rotary_mode, double rope_theta,
                     double rope_scale, int threads, double* out, double* lse);
int pa_oracle_decode_split(int B, int Hq, int Hkv, int D, int page_size, int q_dtype,
                           const void* q, int kv_dtype, const void* k_cache, const void* v_cache,
                           int num_pages, int64_t stride_page, int64_t stride_head,
                           int64_t stride_slot, const int32_t* page_table, int pt_stride,
                           const int32_t* context_lens, double scale, int window,
                           int rotary_mode, double rope_theta, double rope_scale,
                           int partition_size, int threads, double* out, double* lse);

static uint64_t state = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64(void)
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return state * 2685821657736338717ull;
}
static int range(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }

/* A random element of the given dtype (0 f32, 1 f16, 2 bf16) with a normal
 * exponent near 1, written as its bit pattern. */
static void put_elt(void* base, size_t i, int dtype)
{
    uint64_t r = next_u64();
    if (dtype == 0) {
        uint32_t bits = (uint32_t)(r & 0x807FFFFFu) | ((uint32_t)(124 + (r >> 40) % 6) << 23);
        memcpy((char*)base + 4 * i, &bits, 4);
    } else if (dtype == 1) {
        uint16_t bits = (uint16_t)((r & 0x83FFu) | ((uint16_t)(12 + (r >> 40) % 6) << 10));
        memcpy((char*)base + 2 * i, &bits, 2);
    } else {
        uint16_t bits = (uint16_t)((r & 0x807Fu) | ((uint16_t)(124 + (r >> 40) % 6) << 7));
        memcpy((char*)base + 2 * i, &bits, 2);
    }
}

int main(void)
{
    int failures = 0, cases = 0;
    for (int it = 0; it < 400; ++it) {
        const int Hkv = range(1, 3), G = range(1, 4), Hq = Hkv * G;
        const int D = 2 * range(1, 12);
        const int ps = 1 << range(0, 4);
        const int dtype = range(0, 2);
        const int B = range(0, 3);
        const int rot = range(0, 1);
        const int window = range(0, 2) ? 0 : range(1, 40);
        int32_t* lens = malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
        int maxp = 1, total_pages = 0;
        for (int b = 0; b < B; ++b) {
            lens[b] = range(0, 3) ? range(1, 90) : 0;
            int pages = (lens[b] + ps - 1) / ps;
            if (pages > maxp) maxp = pages;
            total_pages += pages;
        }
        const int num_pages = total_pages + range(1, 4);
        const int pt_stride = maxp + range(0, 2);
        /* Token-major or head-major pages, slots padded sometimes. */
        const int64_t slot = D + 2 * range(0, 2);
        int64_t s_page, s_head, s_slot;
        if (range(0, 1)) {
            s_slot = slot;
            s_head = (int64_t)ps * slot;
            s_page = (int64_t)Hkv * ps * slot;
        } else {
            s_head = slot;
            s_slot = (int64_t)Hkv * slot;
            s_page = (int64_t)ps * Hkv * slot;
        }
        const size_t eb = dtype == 0 ? 4 : 2;
        const size_t kv_elts = (size_t)num_pages * (size_t)s_page;
        void* k = malloc(kv_elts * eb);
        void* v = malloc(kv_elts * eb);
        for (size_t i = 0; i < kv_elts; ++i) {
            put_elt(k, i, dtype);
            put_elt(v, i, dtype);
        }
        void* q = malloc((size_t)(B > 0 ? B : 1) * Hq * D * eb);
        for (size_t i = 0; i < (size_t)B * Hq * D; ++i) put_elt(q, i, dtype);
        /* Distinct pages per sequence from a shuffled pool. */
        int32_t* perm = malloc(sizeof(int32_t) * (size_t)num_pages);
        for (int i = 0; i < num_pages; ++i) perm[i] = i;
        for (int i = num_pages - 1; i > 0; --i) {
            int j = range(0, i), t = perm[i];
            perm[i] = perm[j];
            perm[j] = t;
        }
        int32_t* table = malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1) * pt_stride);
        int used = 0;
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < pt_stride; ++j)
                table[(size_t)b * pt_stride + j] =
                    j < (lens[b] + ps - 1) / ps ? perm[used++] : -7; /* padding: never read */
        const size_t outn = (size_t)(B > 0 ? B : 1) * Hq * D;
        double* out = malloc(sizeof(double) * outn);
        double* lse = malloc(sizeof(double) * (size_t)(B > 0 ? B : 1) * Hq);
        double* out2 = malloc(sizeof(double) * outn);
        double* lse2 = malloc(sizeof(double) * (size_t)(B > 0 ? B : 1) * Hq);
        const double scale = 1.0 / sqrt((double)D);
        int rc = pa_oracle_decode(B, Hq, Hkv, D, ps, dtype, q, dtype, k, v, num_pages, s_page, s_head,
                                  s_slot, table, pt_stride, lens, scale, window, rot, 100.0, 1.0,
                                  1, out, lse);
        if (rc != 0) {
            fprintf(stderr, "case %d: decode returned %d\n", it, rc);
            ++failures;
        }
        const int S = ps * range(1, 5);
        rc = pa_oracle_decode_split(B, Hq, Hkv, D, ps, dtype, q, dtype, k, v, num_pages, s_page,
                                    s_head, s_slot, table, pt_stride, lens, scale, window, rot,
                                    100.0, 1.0, S, 1, out2, lse2);
        if (rc != 0) {
            fprintf(stderr, "case %d: split returned %d\n", it, rc);
            ++failures;
        }
        for (int b = 0; b < B; ++b) {
            int lo = (window > 0 && lens[b] > window) ? lens[b] - window : 0;
            int empty = lens[b] - lo == 0;
            for (int h = 0; h < Hq; ++h) {
                const double l1 = lse[b * Hq + h], l2 = lse2[b * Hq + h];
                if (empty ? !(isinf(l1) && l1 < 0 && isinf(l2) && l2 < 0)
                          : !(isfinite(l1) && fabs(l1 - l2) <= 1e-12 * (1.0 + fabs(l1)))) {
                    fprintf(stderr, "case %d b %d h %d: lse %g / %g\n", it, b, h, l1, l2);
                    ++failures;
                }
                for (int d = 0; d < D; ++d) {
                    const size_t i = ((size_t)b * Hq + h) * D + d;
                    if (!isfinite(out[i]) || fabs(out[i] - out2[i]) > 1e-12 * (1.0 + fabs(out[i])) ||
                        (empty && out[i] != 0.0)) {
                        fprintf(stderr, "case %d: out %g / %g\n", it, out[i], out2[i]);
                        ++failures;
                        break;
                    }
                }
            }
        }
        /* A page id outside the pool in a row's visible part: rejected, not read. */
        if (B > 0 && lens[0] > 0) {
            int32_t keep = table[(lens[0] - 1) / ps];
            table[(lens[0] - 1) / ps] = range(0, 1) ? num_pages : -1;
            rc = pa_oracle_decode(B, Hq, Hkv, D, ps, dtype, q, dtype, k, v, num_pages, s_page,
                                  s_head, s_slot, table, pt_stride, lens, scale, window, rot,
                                  100.0, 1.0, 1, out, lse);
            if (rc >= 0) {
                fprintf(stderr, "case %d: invalid page id accepted\n", it);
                ++failures;
            }
            table[(lens[0] - 1) / ps] = keep;
        }
        ++cases;
        free(lens);
        free(k);
        free(v);
        free(q);
        free(perm);
        free(table);
        free(out);
        free(lse);
        free(out2);
        free(lse2);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle checks passed (%d cases)\n", cases);
    return 0;
}
