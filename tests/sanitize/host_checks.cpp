// host_checks.cpp -- drives the host half of the decode library (planner and
// argument validation: pure C++, no HIP call) over seeded random and extreme
// inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitized_host.py).  Every plan that comes back OK is checked
// against what the kernels rely on; a violated property exits non-zero.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "pa_decode.h"
#include "planner.h"
#include "validate.h"

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64()
{
    // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}
int pick(std::initializer_list<int> v)
{
    return *(v.begin() + size_t(next_u64() % uint64_t(v.size())));
}
int range(int lo, int hi) { return lo + int(next_u64() % uint64_t(int64_t(hi) - lo + 1)); }

int failures = 0;
#define EXPECT(cond, ...)                                              \
    do {                                                               \
        if (!(cond)) {                                                 \
            if (failures < 20) {                                       \
                std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
                std::fprintf(stderr, __VA_ARGS__);                     \
                std::fprintf(stderr, "\n");                            \
            }                                                          \
            ++failures;                                                \
        }                                                              \
    } while (0)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pa_decode_desc random_desc()
{
    pa_decode_desc d = {};
    d.num_kv_heads = pick({1, 2, 4, 8, 65535, 65536, 0});
    d.num_q_heads = int(std::min<int64_t>(INT_MAX, int64_t(d.num_kv_heads) * pick({1, 2, 3, 4, 5, 6, 8, 16, 17})));
    d.head_dim = pick({64, 96, 128, 256, 32, 0, -64});
    d.page_size = (next_u64() % 16) ? 16 : 8;
    d.dtype = pick({PA_DTYPE_F32, PA_DTYPE_F16, PA_DTYPE_BF16, 7});
    d.max_batch = pick({0, 1, 16, 64, 4096, 65535, 65536, INT_MAX});
    d.max_context_len = pick({0, 1, 4096, 100000, 1 << 20, INT_MAX});
    d.device = 0;
    d.rotary_mode = (next_u64() % 3) ? 0 : 1;
    d.rope_theta = 10000.f;
    d.rope_scale = 1.f;
    d.debug_checks = 0;
    return d;
}

// Properties of a fixed-partition plan the kernels rely on.
void check_fixed_plan(const pa_decode_desc& d, int batch, int max_ctx, int window,
                      const pa_decode_plan& p)
{
    const int S = p.partition_size, P = p.num_partitions;
    EXPECT(S > 0 && S % 16 == 0, "S %d", S);
    EXPECT(P >= 1, "P %d", P);
    EXPECT(p.split == (P > 1 ? 1 : 0), "split %d P %d", p.split, P);
    const int nw = p.waves_per_group, wpp = p.waves_per_partition;
    EXPECT(nw >= 1 && nw <= 4, "nw %d", nw);
    EXPECT(wpp >= 1 && nw % wpp == 0, "wpp %d nw %d", wpp, nw);
    EXPECT(p.block_partial == 64 * nw, "block %d", p.block_partial);
    EXPECT(int64_t(p.grid_partial[0]) * (nw / wpp) >= P, "grid x %d", p.grid_partial[0]);
    EXPECT(p.grid_partial[0] >= 1 && p.grid_partial[0] <= 65535, "grid x %d", p.grid_partial[0]);
    EXPECT(p.grid_partial[1] == d.num_kv_heads && p.grid_partial[2] == batch, "grid yz");
    // Every context length up to max_ctx needs at most P partitions.
    for (int k = 0; k < 16; ++k) {
        const int64_t n = k == 0 ? max_ctx : int64_t(next_u64() % (uint64_t(max_ctx) + 1));
        const int64_t lo = (window > 0 && n > window) ? n - window : 0;
        if (n <= lo) continue;
        const int64_t need = ceil_div(n, S) - lo / S;
        EXPECT(need <= P, "n %lld lo %lld S %d needs %lld > P %d", (long long)n, (long long)lo, S,
               (long long)need, P);
    }
    if (p.split) {
        const pa::WorkspaceLayout wl = pa::workspace_layout(d, batch, P);
        EXPECT(p.workspace_bytes == int64_t(wl.total), "workspace");
        EXPECT(wl.m_off >= size_t(batch) * d.num_q_heads * size_t(P) * d.head_dim * 4, "o region");
        EXPECT(p.grid_merge[0] >= 1 && p.block_merge == 256, "merge grid %d %d %d Hq %d B %d P %d D %d",
               p.grid_merge[0], p.grid_merge[1], p.grid_merge[2], d.num_q_heads, batch, P,
               d.head_dim);
    } else {
        EXPECT(p.workspace_bytes == 0, "unsplit workspace");
    }
    EXPECT(pa::partial_lds_bytes(d, p) <= 160 * 1024, "lds %zu", pa::partial_lds_bytes(d, p));
}

void check_balanced_plan(const pa_decode_desc& d, int batch, const pa_decode_plan& p)
{
    const int W = p.balanced_waves, nw = p.waves_per_group;
    EXPECT(W > 0 && nw >= 1 && W % nw == 0, "W %d nw %d", W, nw);
    EXPECT(int64_t(p.grid_partial[0]) * nw == W, "grid x");
    EXPECT(p.grid_partial[2] == 1 && p.waves_per_partition == 1, "grid z / wpp");
    EXPECT(p.num_partitions >= 1 && p.num_partitions <= W, "pitch %d", p.num_partitions);
    EXPECT(batch <= pa::kBalancedMaxBatch, "batch %d", batch);
    EXPECT(p.workspace_bytes == int64_t(pa::workspace_layout(d, batch, p.num_partitions, true).total),
           "workspace");
}

void plans()
{
    pa::PlanTuning tune;
    int ok = 0;
    for (int it = 0; it < 200000; ++it) {
        pa_decode_desc d = random_desc();
        if (it % 7 == 0) {
            tune.waves_per_partition = pick({0, 1, 2, 4});
            tune.waves_per_group = pick({0, 1, 2, 4});
            tune.balanced_start = range(-1, 64);
            tune.balanced_waves_per_cu = range(0, 16);
        }
        const int cus = pick({256, 1, 80, 0, -1, 304});
        const int wpc = pick({8, 1, 4, 16, 0});
        const int batch = pick({0, 1, 2, 3, 16, 64, 65, 512, 65535, -1});
        const int max_ctx = pick({0, 1, 15, 16, 17, 300, 3060, 4096, 8192, 100000,
                                               1 << 20, INT_MAX, -5});
        const int window = pick({0, -3, 1, 16, 17, 4096, 100000, INT_MAX});
        const int S = pick({0, 0, 16, 48, 512, 4096, 1 << 20, 24, -1, -7, INT_MAX});
        pa_decode_plan p;
        const int st = pa::make_plan(d, cus, wpc, tune, batch, max_ctx, window, S, &p);
        if (st == PA_DECODE_OK && batch > 0) {
            ++ok;
            if (p.balanced_waves > 0)
                check_balanced_plan(d, batch, p);
            else
                check_fixed_plan(d, batch, max_ctx, window, p);
        }
        const int nnz = pick({0, 1, 19, 192, 2048, 6250, 65536, INT_MAX, -1});
        int used = 0;
        const int st2 = pa::make_plan_csr(d, cus, wpc, tune, batch, nnz, max_ctx, window, S, &p,
                                          &used);
        if (st2 == PA_DECODE_OK && batch > 0) {
            ++ok;
            if (p.balanced_waves > 0)
                check_balanced_plan(d, batch, p);
            else
                check_fixed_plan(d, batch, used, window, p);
        }
    }
    // Valid descriptions and realistic calls (most plans come back OK).
    for (int it = 0; it < 100000; ++it) {
        pa_decode_desc d = {};
        d.num_kv_heads = pick({1, 2, 4, 8, 32});
        d.num_q_heads = d.num_kv_heads * pick({1, 2, 3, 4, 6, 8, 16});
        d.dtype = pick({PA_DTYPE_F16, PA_DTYPE_BF16, PA_DTYPE_F32});
        d.head_dim = d.dtype == PA_DTYPE_F32 ? 64 : pick({64, 96, 128, 256});
        d.page_size = 16;
        d.max_batch = 4096;
        d.max_context_len = 1 << 20;
        d.rotary_mode = int(next_u64() % 2);
        d.rope_theta = 500000.f;
        d.rope_scale = 1.f;
        pa::PlanTuning none;
        const int batch = range(1, 600);
        const int max_ctx = (next_u64() % 4) ? range(0, 8192) : range(0, 1 << 20);
        const int window = (next_u64() % 3) ? 0 : range(1, 9000);
        const int S = (next_u64() % 2) ? 0 : ((next_u64() % 8) ? 16 * range(1, 300) : -1);
        pa_decode_plan p;
        const int st = pa::make_plan(d, 256, pick({4, 8, 12}), none, batch, max_ctx, window, S, &p);
        EXPECT(st == PA_DECODE_OK || (S == -1 && batch > pa::kBalancedMaxBatch), "valid call %d", st);
        if (st == PA_DECODE_OK) {
            ++ok;
            if (p.balanced_waves > 0)
                check_balanced_plan(d, batch, p);
            else
                check_fixed_plan(d, batch, max_ctx, window, p);
        }
        const int nnz = int(next_u64() % (uint64_t(batch) * (uint64_t(max_ctx) / 16 + 1) + 1));
        int used = 0;
        const int st2 = pa::make_plan_csr(d, 256, 8, none, batch, nnz, max_ctx, window, S, &p, &used);
        if (st2 == PA_DECODE_OK) {
            ++ok;
            if (p.balanced_waves > 0)
                check_balanced_plan(d, batch, p);
            else
                check_fixed_plan(d, batch, used, window, p);
        }
    }
    std::printf("plans: %d accepted\n", ok);
}

void validation()
{
    alignas(16) static char buf[4096];
    int ok = 0;
    for (int it = 0; it < 200000; ++it) {
        pa_decode_desc d = random_desc();
        if (pa::check_desc(d) != PA_DECODE_OK) continue;
        pa_decode_args a = {};
        a.q = (next_u64() % 8) ? buf : (next_u64() % 2 ? nullptr : buf + 2);
        a.k_cache = buf;
        a.v_cache = (next_u64() % 8) ? buf + 16 : buf + 8;
        a.out = buf;
        const int64_t strides[] = {0, 8, 16, 64, 4096, -16, int64_t(1) << 40, (int64_t(1) << 40) + 16,
                                   INT64_MAX};
        a.kv_stride_page = strides[next_u64() % 9];
        a.kv_stride_head = strides[next_u64() % 9];
        a.kv_stride_slot = strides[next_u64() % 9];
        a.num_pages = pick({0, 1, 4096, INT_MAX, -1});
        a.page_table = (next_u64() % 8) ? reinterpret_cast<const int32_t*>(buf) : nullptr;
        a.pt_stride = pick({0, 1, 256, 6250, INT_MAX, -1});
        a.context_lens = reinterpret_cast<const int32_t*>(buf);
        a.batch = pick({0, 1, 16, 65535, -1});
        a.max_context_len = pick({0, 1, 4096, 100000, INT_MAX, -1});
        a.scale = (next_u64() % 16) ? 0.125f : (next_u64() % 2 ? __builtin_nanf("") : __builtin_inff());
        a.sliding_window = pick({0, 4096, -1, INT_MAX});
        a.partition_size = pick({0, 16, 24, -1, -2, 512, INT_MAX});
        const int st = pa::check_args(d, a);
        if (st == PA_DECODE_OK && a.batch > 0) {
            ++ok;
            const int eb = pa::dtype_bytes(d.dtype);
            EXPECT(a.kv_stride_slot >= d.head_dim && a.kv_stride_slot * eb < (int64_t(1) << 27),
                   "slot stride");
            EXPECT((a.kv_stride_page * eb) % 16 == 0 && (a.kv_stride_head * eb) % 16 == 0, "align");
            EXPECT(int64_t(a.num_pages) * a.kv_stride_page * eb <= (int64_t(1) << 50), "page span");
            EXPECT(int64_t(a.pt_stride) * d.page_size >= a.max_context_len, "table stride");
            EXPECT(a.batch <= d.max_batch && a.max_context_len <= d.max_context_len, "bounds");
            EXPECT(pa::aligned16(a.q) && pa::aligned16(a.v_cache), "pointers");
        }
        pa_decode_csr_args c = {};
        c.q = a.q;
        c.k_cache = a.k_cache;
        c.v_cache = a.v_cache;
        c.kv_stride_page = a.kv_stride_page;
        c.kv_stride_head = a.kv_stride_head;
        c.kv_stride_slot = a.kv_stride_slot;
        c.num_pages = a.num_pages;
        c.page_indptr = (next_u64() % 8) ? reinterpret_cast<const int32_t*>(buf) : nullptr;
        c.page_indices = (next_u64() % 8) ? reinterpret_cast<const int32_t*>(buf) : nullptr;
        c.last_page_len = reinterpret_cast<const int32_t*>(buf);
        c.nnz_pages = pick({0, 1, 6250, INT_MAX, -1});
        c.batch = a.batch;
        c.max_context_len = a.max_context_len;
        c.scale = a.scale;
        c.sliding_window = a.sliding_window;
        c.partition_size = a.partition_size;
        c.out = a.out;
        const int st2 = pa::check_csr_args(d, c);
        if (st2 == PA_DECODE_OK && c.batch > 0) {
            ++ok;
            EXPECT(c.nnz_pages >= 0 && c.page_indptr && (c.nnz_pages == 0 || c.page_indices), "csr");
        }
    }
    // Valid arguments with one field changed at a time: each change either
    // keeps the call valid or is rejected, never accepted wrongly.
    pa_decode_desc d = {};
    d.num_q_heads = 32;
    d.num_kv_heads = 8;
    d.head_dim = 128;
    d.page_size = 16;
    d.dtype = PA_DTYPE_F16;
    d.max_batch = 64;
    d.max_context_len = 1 << 20;
    int rejected = 0;
    for (int it = 0; it < 100000; ++it) {
        pa_decode_args a = {};
        a.q = buf;
        a.k_cache = buf + 16;
        a.v_cache = buf + 32;
        a.out = buf + 48;
        a.kv_stride_page = 8 * 16 * 128;
        a.kv_stride_head = 16 * 128;
        a.kv_stride_slot = 128;
        a.num_pages = 4096;
        a.page_table = reinterpret_cast<const int32_t*>(buf);
        a.pt_stride = 256;
        a.context_lens = reinterpret_cast<const int32_t*>(buf);
        a.batch = 16;
        a.max_context_len = 4096;
        a.scale = 0.088f;
        a.partition_size = 0;
        EXPECT(pa::check_args(d, a) == PA_DECODE_OK, "base call");
        switch (next_u64() % 12) {
        case 0: a.q = buf + range(1, 15); break;
        case 1: a.kv_stride_slot = range(-200, 200); break;
        case 2: a.kv_stride_page = int64_t(next_u64() >> range(1, 63)); break;
        case 3: a.num_pages = range(-5, INT_MAX - 1); break;
        case 4: a.pt_stride = range(-5, 300); break;
        case 5: a.batch = range(-5, 70); break;
        case 6: a.max_context_len = range(-5, 1 << 21); break;
        case 7: a.partition_size = range(-3, 5000); break;
        case 8: a.page_table = nullptr; break;
        case 9: a.kv_stride_head = range(-64, 2048); break;
        case 10: a.scale = (next_u64() % 2) ? __builtin_inff() : -0.5f; break;
        default: a.kv_stride_slot = int64_t(range(1, 1 << 30)) * 8; break;
        }
        const int st = pa::check_args(d, a);
        if (st != PA_DECODE_OK) {
            ++rejected;
            continue;
        }
        ++ok;
        const int eb = 2;
        EXPECT(a.kv_stride_slot >= 128 && a.kv_stride_slot * eb < (int64_t(1) << 27), "slot %lld",
               (long long)a.kv_stride_slot);
        EXPECT(a.kv_stride_page >= 0 && (a.kv_stride_page * eb) % 16 == 0, "page stride");
        EXPECT(int64_t(a.num_pages) * a.kv_stride_page * eb <= (int64_t(1) << 50), "page span");
        EXPECT(a.kv_stride_head >= 0 && (a.kv_stride_head * eb) % 16 == 0, "head stride");
        EXPECT(a.batch == 0 || (a.num_pages > 0 && pa::aligned16(a.q) && a.page_table &&
                                int64_t(a.pt_stride) * 16 >= a.max_context_len),
               "accepted call");
        EXPECT(a.partition_size == 0 || a.partition_size == -1 || a.partition_size % 16 == 0,
               "partition %d", a.partition_size);
    }
    std::printf("validation: %d accepted, %d rejected\n", ok, rejected);
}

}  // namespace

int main()
{
    plans();
    validation();
    // The environment overrides: out-of-range values are ignored.
    setenv("PA_DECODE_WAVES_PER_PARTITION", "3", 1);
    setenv("PA_DECODE_WAVES_PER_GROUP", "99999999999999999999", 1);
    setenv("PA_DECODE_BALANCED_START", "-4", 1);
    setenv("PA_DECODE_BALANCED_WAVES_PER_CU", "junk", 1);
    const pa::PlanTuning t = pa::tuning_from_env();
    EXPECT(t.waves_per_partition == 0 && t.waves_per_group == 0 && t.balanced_start == -1 &&
               t.balanced_waves_per_cu == 0,
           "tuning %d %d %d %d", t.waves_per_partition, t.waves_per_group, t.balanced_start,
           t.balanced_waves_per_cu);
    setenv("PA_DECODE_WAVES_PER_PARTITION", "2", 1);
    setenv("PA_DECODE_BALANCED_START", "12", 1);
    const pa::PlanTuning u = pa::tuning_from_env();
    EXPECT(u.waves_per_partition == 2 && u.balanced_start == 12, "tuning read");
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
