/*
 * pa_oracle.c -- plain CPU reference for single-query paged-KV decode attention
 * with grouped-query attention (GQA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the HIP library, and the HIP library never calls into it.
 *
 * What it computes (the plain definition, in float64):
 *   for every sequence b and query head h, with KV head g = floor(h / G),
 *   G = Hq / Hkv, and visible keys j in [lo_b, n_b):
 *     s_j      = scale * sum_d q[b,h,d] * K_b[j,g,d]
 *     out[b,h] = sum_j softmax(s)_j * V_b[j,g,:]
 *     lse[b,h] = ln sum_j exp(s_j)
 *   Sources:
 *   - "Output and LSE" checked against an f64 reference, shuffled page table,
 *     sliding window, batch > 1: TVM PR #20426 (Apache mail-archive copy),
 *     section "Correctness".
 *   - K/V gathered per page through a block table (key_cache[blk_ids]): the
 *     paged_attention_v2_pytorch.py commit page, section "KV gather".
 *   - Query head h reads KV head floor(h / G): the same commit page, the
 *     [kv_h, gqa, ...] -> [H, ...] reshape of the scores@V broadcast.
 *
 * Rotary position embedding (rotary_mode 1), applied to q and to every key
 * as they are read.  TVM PR #20426, section "Correctness", names the option
 * (`rotary_mode = 1`) without defining it; the reading taken is the rotary
 * embedding of the RoFormer paper with the rotate-half pairing that the
 * pages' models (Llama 3.x, Qwen3, Gemma 2) use:
 *   for i < D/2, the pair (x[i], x[i + D/2]) of a vector at position pos is
 *   turned by the angle pos * theta_i, theta_i = rope_theta^(-2i/D) /
 *   rope_scale:
 *     x'[i]       = x[i] cos(a) - x[i + D/2] sin(a)
 *     x'[i + D/2] = x[i + D/2] cos(a) + x[i] sin(a)
 *   Key j of a sequence sits at position j; the query is the newest token,
 *   position n_b - 1.  The score uses the rotated q and rotated key.
 *
 * pa_oracle_decode_split() computes the same result the partitioned way,
 * following the commit page's "Phase 1: Per-partition attention" (per
 * partition: max, exp-sum, normalised weighted V) and "Phase 2:
 * Cross-partition reduction" (global max, rescale = exp(m_p - max) * l_p,
 * out = sum_p rescale_p / sum(rescale) * o_p).  It is used to pin the
 * invariant that the partition size does not change the result.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - The cache already holds the current token: keys 0..n_b-1 are visible.
 *   - Sliding window W > 0 keeps the W most recent keys, [n_b - W, n_b);
 *     W <= 0 means no window.
 *   - LSE is the natural logarithm of the sum of exp(scaled scores).
 *   - n_b - lo_b == 0 (empty context): out = 0, lse = -inf.
 *   - Partitions are aligned to absolute multiples of the partition size and
 *     clipped to [lo_b, n_b).
 *   - Rotary positions are the token indices in the sequence (no offset), the
 *     whole head is rotated, and a sliding window does not renumber them.
 *
 * Layouts:
 *   q            [B, Hq, D] contiguous, dtype q_dtype
 *   k/v cache    [num_pages, Hkv, page_size, D] addressed through element
 *                strides (page, head, slot); the D axis is contiguous
 *   page_table   int32 [B, pt_stride]; entry j / page_size of row b is the
 *                physical page of token j
 *   context_lens int32 [B]
 *   out          float64 [B, Hq, D]; lse float64 [B, Hq]
 *
 * Returns 0 on success, a negative code on invalid arguments or when the page
 * table names a page outside [0, num_pages) (checked, never read).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PA_ORACLE_F32 0
#define PA_ORACLE_F16 1
#define PA_ORACLE_BF16 2

/* IEEE 754 binary16 -> float64, straight from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double pa_oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> float64: bfloat16 is the upper half of a binary32. */
double pa_oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double load_elt(const void* base, int64_t idx, int dtype)
{
    if (dtype == PA_ORACLE_F32)
        return (double)((const float*)base)[idx];
    if (dtype == PA_ORACLE_F16)
        return pa_oracle_f16_to_f64(((const uint16_t*)base)[idx]);
    return pa_oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
}

typedef struct {
    int B, Hq, Hkv, D, page_size;
    int q_dtype;
    const void* q;
    int kv_dtype;
    const void* k_cache;
    const void* v_cache;
    int num_pages;
    int64_t stride_page, stride_head, stride_slot;
    const int32_t* page_table;
    int pt_stride;
    const int32_t* context_lens;
    double scale;
    int window;
    int rotary;        /* 0: none; 1: rotary embedding of q and keys */
    double rope_theta; /* frequency base */
    double rope_scale; /* positions are divided by it */
} problem;

static int check_problem(const problem* p)
{
    if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->page_size <= 0)
        return -1;
    if (p->Hq % p->Hkv != 0)
        return -1;
    if (p->q_dtype < 0 || p->q_dtype > 2 || p->kv_dtype < 0 || p->kv_dtype > 2)
        return -1;
    if (p->rotary != 0 && p->rotary != 1)
        return -1;
    if (p->rotary && (p->D % 2 != 0 || !(p->rope_theta > 0.0) || !(p->rope_scale > 0.0)))
        return -1;
    for (int b = 0; b < p->B; ++b) {
        int n = p->context_lens[b];
        if (n < 0)
            return -1;
        int pages = (n + p->page_size - 1) / p->page_size;
        if (pages > p->pt_stride)
            return -1;
        int lo = (p->window > 0 && n > p->window) ? n - p->window : 0;
        for (int j = lo / p->page_size; j < pages; ++j) {
            int32_t pg = p->page_table[(int64_t)b * p->pt_stride + j];
            if (pg < 0 || pg >= p->num_pages)
                return -2;
        }
    }
    return 0;
}

/* Element offset of K/V[token j of sequence b, kv head g, dim 0]: a naive
 * page-table walk, page = table[b][j / page_size], slot = j % page_size. */
static int64_t kv_offset(const problem* p, int b, int j, int g)
{
    int32_t page = p->page_table[(int64_t)b * p->pt_stride + j / p->page_size];
    int slot = j % p->page_size;
    return (int64_t)page * p->stride_page + (int64_t)g * p->stride_head +
           (int64_t)slot * p->stride_slot;
}

/* Element d of the vector of D elements at `base + off`, rotated to position
 * `pos` (rotary embedding, rotate-half pairing; see the header comment). */
static double rotated_elt(const problem* p, const void* base, int64_t off, int dtype, int d,
                          double pos)
{
    int half = p->D / 2;
    int i = d < half ? d : d - half;
    double angle = pos / p->rope_scale * pow(p->rope_theta, -2.0 * i / p->D);
    double x = load_elt(base, off + d, dtype);
    if (d < half)
        return x * cos(angle) - load_elt(base, off + d + half, dtype) * sin(angle);
    return x * cos(angle) + load_elt(base, off + d - half, dtype) * sin(angle);
}

/* The query vector of (b, h) as the scores use it: q[b,h,:], rotated to
 * position n_b - 1 when rotary_mode is 1. */
static void query_vector(const problem* p, int b, int h, double* qv)
{
    int64_t qo = ((int64_t)b * p->Hq + h) * p->D;
    for (int d = 0; d < p->D; ++d)
        qv[d] = p->rotary ? rotated_elt(p, p->q, qo, p->q_dtype, d, p->context_lens[b] - 1.0)
                          : load_elt(p->q, qo + d, p->q_dtype);
}

/* Scaled score s_j = scale * qv . K[j, g, :], the key rotated to position j
 * when rotary_mode is 1. */
static double score(const problem* p, int b, int h, const double* qv, int j)
{
    int g = h / (p->Hq / p->Hkv);
    int64_t ko = kv_offset(p, b, j, g);
    double acc = 0.0;
    for (int d = 0; d < p->D; ++d)
        acc += qv[d] * (p->rotary ? rotated_elt(p, p->k_cache, ko, p->kv_dtype, d, (double)j)
                                  : load_elt(p->k_cache, ko + d, p->kv_dtype));
    return p->scale * acc;
}

static void visible_range(const problem* p, int b, int* lo, int* n)
{
    *n = p->context_lens[b];
    *lo = (p->window > 0 && *n > p->window) ? *n - p->window : 0;
}

/* Direct softmax over all visible keys of one (b, h). */
static void one_head(const problem* p, int b, int h, double* out, double* lse)
{
    int lo, n;
    visible_range(p, b, &lo, &n);
    int g = h / (p->Hq / p->Hkv);
    int D = p->D;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n - lo <= 0) {
        *lse = -INFINITY;
        return;
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)(n - lo));
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    query_vector(p, b, h, qv);
    double M = -INFINITY;
    for (int j = lo; j < n; ++j) {
        s[j - lo] = score(p, b, h, qv, j);
        if (s[j - lo] > M)
            M = s[j - lo];
    }
    double L = 0.0;
    for (int j = lo; j < n; ++j) {
        double e = exp(s[j - lo] - M);
        L += e;
        int64_t vo = kv_offset(p, b, j, g);
        for (int d = 0; d < D; ++d)
            out[d] += e * load_elt(p->v_cache, vo + d, p->kv_dtype);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= L;
    *lse = M + log(L);
    free(s);
    free(qv);
}

/* Partitioned form of one (b, h): per-partition state (m_p, l_p, o_p), then
 * the two-phase log-sum-exp merge. */
static void one_head_split(const problem* p, int b, int h, int S, double* out, double* lse)
{
    int lo, n;
    visible_range(p, b, &lo, &n);
    int g = h / (p->Hq / p->Hkv);
    int D = p->D;
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n - lo <= 0) {
        *lse = -INFINITY;
        return;
    }
    int p0 = lo / S, p1 = (n + S - 1) / S;
    int P = p1 - p0;
    double* m = (double*)malloc(sizeof(double) * (size_t)P);
    double* l = (double*)malloc(sizeof(double) * (size_t)P);
    double* o = (double*)calloc((size_t)P * (size_t)D, sizeof(double));
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    query_vector(p, b, h, qv);
    /* Phase 1: each partition on its own. */
    for (int pi = 0; pi < P; ++pi) {
        int a = (p0 + pi) * S, e = (p0 + pi + 1) * S;
        if (a < lo) a = lo;
        if (e > n) e = n;
        double mp = -INFINITY;
        for (int j = a; j < e; ++j) {
            double sj = score(p, b, h, qv, j);
            if (sj > mp) mp = sj;
        }
        double lp = 0.0;
        for (int j = a; j < e; ++j) {
            double w = exp(score(p, b, h, qv, j) - mp);
            lp += w;
            int64_t vo = kv_offset(p, b, j, g);
            for (int d = 0; d < D; ++d)
                o[(size_t)pi * D + d] += w * load_elt(p->v_cache, vo + d, p->kv_dtype);
        }
        for (int d = 0; d < D; ++d)
            o[(size_t)pi * D + d] /= lp;
        m[pi] = mp;
        l[pi] = lp;
    }
    /* Phase 2: global max, per-partition rescale, weighted sum of outputs. */
    double gmax = -INFINITY;
    for (int pi = 0; pi < P; ++pi)
        if (m[pi] > gmax) gmax = m[pi];
    double total = 0.0;
    for (int pi = 0; pi < P; ++pi) {
        l[pi] = exp(m[pi] - gmax) * l[pi]; /* rescale_p */
        total += l[pi];
    }
    for (int pi = 0; pi < P; ++pi)
        for (int d = 0; d < D; ++d)
            out[d] += (l[pi] / total) * o[(size_t)pi * D + d];
    *lse = gmax + log(total);
    free(m);
    free(l);
    free(o);
    free(qv);
}

static int run(const problem* p, int S, int threads, double* out, double* lse)
{
    int rc = check_problem(p);
    if (rc)
        return rc;
    if (S < 0)
        return -1;
    int64_t total = (int64_t)p->B * p->Hq;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < total; ++i) {
        int b = (int)(i / p->Hq), h = (int)(i % p->Hq);
        if (S == 0)
            one_head(p, b, h, out + i * p->D, lse + i);
        else
            one_head_split(p, b, h, S, out + i * p->D, lse + i);
    }
    return 0;
}

#define PROBLEM_ARGS                                                                     \
    int B, int Hq, int Hkv, int D, int page_size, int q_dtype, const void *q, int kv_dtype, \
        const void *k_cache, const void *v_cache, int num_pages, int64_t stride_page,      \
        int64_t stride_head, int64_t stride_slot, const int32_t *page_table, int pt_stride, \
        const int32_t *context_lens, double scale, int window, int rotary_mode,             \
        double rope_theta, double rope_scale

#define PROBLEM_INIT                                                                      \
    problem p = {B,        Hq,          Hkv,         D,          page_size,    q_dtype, q, \
                 kv_dtype, k_cache,     v_cache,     num_pages,  stride_page,  stride_head, \
                 stride_slot, page_table, pt_stride, context_lens, scale, window,      \
                 rotary_mode, rope_theta, rope_scale}

int pa_oracle_decode(PROBLEM_ARGS, int threads, double* out, double* lse)
{
    PROBLEM_INIT;
    return run(&p, 0, threads, out, lse);
}

int pa_oracle_decode_split(PROBLEM_ARGS, int partition_size, int threads, double* out,
                           double* lse)
{
    PROBLEM_INIT;
    if (partition_size <= 0)
        return -1;
    return run(&p, partition_size, threads, out, lse);
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int pa_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
