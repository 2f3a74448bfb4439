// planner.cpp -- see planner.h.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>

namespace pa {

int dtype_bytes(int dtype)
{
    switch (dtype) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_F16: return 2;
    case PA_DTYPE_BF16: return 2;
    default: return 0;
    }
}

int pages_per_block(int head_dim, int dtype)
{
    // 4 KiB of K (and of V) per block where a page allows it: two pages of
    // 128-byte rows, one of 256- or 192-byte rows, one page of 512-byte rows
    // (8 KiB).  Measured on MI355X against 8 KiB blocks, steps 1-8 % faster on
    // every head_dim 64/96/128 and f32 shape tried (half the load registers
    // and LDS per wave, 3 resident waves per SIMD instead of 2 at head_dim
    // 128, a shorter exposed last block), but 3-15 % slower for fixed
    // partitions over ragged batches, whose longest sequences' waves hold the
    // most blocks (the CSR rule gives those the balanced schedule).  Two
    // 512-byte-row pages per block (for 32-token P.V MFMAs) measured slower
    // still: the doubled load registers push the kernel to one wave per SIMD
    // with AGPR spills.
    return pages_per_block_for_row(head_dim * dtype_bytes(dtype));
}

int tile_row_slots(int head_dim, int dtype)
{
    const int ch = head_dim * dtype_bytes(dtype) / 16;
    return (ch & (ch - 1)) == 0 ? ch : ch + 1;
}

int template_group(int G)
{
    static const int built[] = {1, 2, 4, 6, 8, 16};
    for (int g : built)
        if (G <= g) return g;
    return 0;
}

int check_desc(const pa_decode_desc& d)
{
    if (d.num_q_heads <= 0 || d.num_kv_heads <= 0 || d.head_dim <= 0 || d.page_size <= 0 ||
        d.max_batch < 0 || d.max_context_len < 0 || d.device < 0)
        return PA_DECODE_INVALID_ARG;
    if (d.num_q_heads % d.num_kv_heads != 0)
        return PA_DECODE_INVALID_ARG;
    if (d.rotary_mode != 0 && d.rotary_mode != 1)
        return PA_DECODE_INVALID_ARG;
    if (d.debug_checks != 0 && d.debug_checks != 1)
        return PA_DECODE_INVALID_ARG;
    if (d.rotary_mode == 1 &&
        !(std::isfinite(d.rope_theta) && d.rope_theta > 0.f && std::isfinite(d.rope_scale) &&
          d.rope_scale > 0.f))
        return PA_DECODE_INVALID_ARG;
    if (d.dtype != PA_DTYPE_F32 && d.dtype != PA_DTYPE_F16 && d.dtype != PA_DTYPE_BF16)
        return PA_DECODE_UNSUPPORTED;
    if (d.page_size != kPageSize)
        return PA_DECODE_UNSUPPORTED;
    if (d.head_dim != 64 && d.head_dim != 96 && d.head_dim != 128 && d.head_dim != 256)
        return PA_DECODE_UNSUPPORTED;
    if (d.dtype == PA_DTYPE_F32 && d.head_dim != 64)
        return PA_DECODE_UNSUPPORTED;
    int G = d.num_q_heads / d.num_kv_heads;
    if (G > kMaxGroup || template_group(G) == 0)
        return PA_DECODE_UNSUPPORTED;
    // Sequences and KV heads index the y / z dimensions of the launch grids.
    if (d.max_batch > kMaxGridYZ || d.num_kv_heads > kMaxGridYZ)
        return PA_DECODE_UNSUPPORTED;
    return PA_DECODE_OK;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Waves per workgroup of the partial kernel: four, fewer when the K/V tiles
// or the combine buffer would pass 64 KiB of LDS, or (rotary) when the
// workgroup's tiles and tables would pass 80 KiB.
int workgroup_waves(const pa_decode_desc& d)
{
    const int ps = d.page_size;
    const int nb = pages_per_block(d.head_dim, d.dtype);
    const int G = d.num_q_heads / d.num_kv_heads;
    int nw = kMaxWavesPerGroup;
    const int Gt = template_group(G);
    const int gp4 = (Gt + 3) / 4 * 4;
    const int64_t comb = int64_t(2 * gp4 + Gt * d.head_dim) * 4;
    const int64_t tiles = int64_t(2) * nb * ps * 16 * tile_row_slots(d.head_dim, d.dtype);
    const int64_t per_wave = std::max(comb, tiles);
    while (nw > 1 && nw * per_wave > 65536) nw /= 2;
    // With rotary, also keep the workgroup (tiles, base tables, offset
    // table) within half of the compute unit's 160 KiB, so that two
    // workgroups share a compute unit.
    while (nw > 1 && nw * (tiles + rotary_table_bytes(d)) + rotary_offset_table_bytes(d) > 81920)
        nw /= 2;
    return nw;
}

WorkspaceLayout workspace_layout(const pa_decode_desc& d, int batch, int num_partitions,
                                 bool counts)
{
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
#if PA_FUSED_MERGE
    counts = true;   // comparison build: the per-(sequence, KV head) merge counters
#endif
    size_t rows = size_t(batch) * size_t(d.num_q_heads) * size_t(num_partitions);
    WorkspaceLayout w;
    w.o_off = 0;
    w.m_off = w.o_off + align(rows * size_t(d.head_dim) * sizeof(float));
    w.l_off = w.m_off + align(rows * sizeof(float));
    w.c_off = w.l_off + align(rows * sizeof(float));
    w.total = w.c_off +
              (counts ? align(size_t(batch) * size_t(d.num_q_heads) * sizeof(int32_t)) : 0);
    return w;
}

// Merge grid and block of a split plan with P state rows per (sequence,
// head); `counts` (balanced schedule): the per-wave merge whatever P.
// UNSUPPORTED when the wave count does not fit the kernels' 32-bit unit index.
static int set_merge_grid(const pa_decode_desc& d, int batch, int64_t P, pa_decode_plan* p,
                          bool counts = false)
{
    if (P <= kMergeWaveMaxPartitions || counts) {
        // one wave per (sequence, query head, 64-dim slice), four per workgroup
        const int cw = merge_slice_width(batch, d.num_q_heads, d.head_dim);
        const int64_t units = int64_t(batch) * d.num_q_heads * ((d.head_dim + cw - 1) / cw);
        if (units > INT32_MAX - 3)
            return PA_DECODE_UNSUPPORTED;
        p->grid_merge[0] = int32_t((units + 3) / 4);
        p->grid_merge[1] = 1;
        p->grid_merge[2] = 1;
    } else {
        p->grid_merge[0] = d.num_q_heads;
        p->grid_merge[1] = batch;
        p->grid_merge[2] = d.head_dim / 16;   // 16-column slices
    }
    p->block_merge = kMergeThreads;
    return PA_DECODE_OK;
}

PlanTuning tuning_from_env()
{
    PlanTuning t;
    auto read = [](const char* name, int* dst, int lo, int hi) {
        if (const char* env = std::getenv(name)) {
            char* end = nullptr;
            const long v = std::strtol(env, &end, 10);
            if (end != env && v >= lo && v <= hi) *dst = int(v);
        }
    };
    read("PA_DECODE_WAVES_PER_PARTITION", &t.waves_per_partition, 1, 4);
    read("PA_DECODE_WAVES_PER_GROUP", &t.waves_per_group, 1, 4);
    read("PA_DECODE_BALANCED_START", &t.balanced_start, 0, 64);
    read("PA_DECODE_BALANCED_WAVES_PER_CU", &t.balanced_waves_per_cu, 1, 16);
    if (t.waves_per_partition == 3) t.waves_per_partition = 0;
    if (t.waves_per_group == 3) t.waves_per_group = 0;
    return t;
}

int balanced_start_pages(const pa_decode_desc& d, const PlanTuning& tune)
{
    // Four blocks' worth, three with rotary: measured on MI355X over 2 .. 32
    // pages for batches of 16 with lengths up to 4096 at two pages per
    // block, the best charges were 8 (head_dim 128), 8 - 10 (head_dim 96)
    // and 6 - 7 (head_dim 128 with rotary, whose blocks take longer).  At one
    // page per block (4 KiB blocks) charges of 2 .. 12 pages measured within
    // 2 % of each other at head_dim 128 and 96, 3 % with rotary.
    int c = (d.rotary_mode == 1 ? 3 : 4) * pages_per_block(d.head_dim, d.dtype);
    if (tune.balanced_start >= 0) c = tune.balanced_start;
    return std::max(0, std::min(64, c));
}

// The length-balanced schedule (partition_size PA_DECODE_PARTITION_BALANCED):
// every KV head gets W waves (about four per compute unit over all heads, a
// multiple of the workgroup size), which split the batch's visible pages
// evenly in the kernel.  A (sequence, head) then has at most min(W, its
// visible pages) states.
static int make_balanced_plan(const pa_decode_desc& d, int num_cus, int waves_per_cu,
                              const PlanTuning& tune, int batch, int64_t vis_pages,
                              pa_decode_plan* plan)
{
    if (batch > kBalancedMaxBatch)
        return PA_DECODE_UNSUPPORTED;
    if (int64_t(batch) * (vis_pages + 64) >= (int64_t(1) << 31))   // charged pages fit in int32
        return PA_DECODE_UNSUPPORTED;
    const int nw = workgroup_waves(d);
    const int64_t capacity = int64_t(num_cus) * waves_per_cu;
    const int per_cu = tune.balanced_waves_per_cu > 0 ? tune.balanced_waves_per_cu : 4;
    const int64_t target = std::min<int64_t>(capacity, int64_t(num_cus) * per_cu);
    // Waves per KV head: the target shared by the heads, no more than the
    // batch's pages, a whole number of workgroups.
    int64_t W = std::min<int64_t>(target / d.num_kv_heads, int64_t(batch) * vis_pages);
    W = std::max<int64_t>(nw, W / nw * nw);
    if (W / nw > 65535)
        return PA_DECODE_UNSUPPORTED;
    const int64_t P = std::min<int64_t>(W, vis_pages);

    pa_decode_plan p = {};
    p.split = 1;
    p.partition_size = 0;
    p.num_partitions = int32_t(P);
    p.waves_per_group = nw;
    p.waves_per_partition = 1;
    p.pages_per_block = pages_per_block(d.head_dim, d.dtype);
    p.grid_partial[0] = int32_t(W / nw);
    p.grid_partial[1] = d.num_kv_heads;
    p.grid_partial[2] = 1;
    p.block_partial = nw * 64;
    if (set_merge_grid(d, batch, P, &p, true) != PA_DECODE_OK)
        return PA_DECODE_UNSUPPORTED;
    p.workspace_bytes = int64_t(workspace_layout(d, batch, int(P), true).total);
    p.num_cus = num_cus;
    p.waves_per_cu = waves_per_cu;
    p.balanced_waves = int32_t(W);
    *plan = p;
    return PA_DECODE_OK;
}

int make_plan(const pa_decode_desc& d, int num_cus, int waves_per_cu, const PlanTuning& tune,
              int batch, int max_context_len, int sliding_window, int partition_size,
              pa_decode_plan* plan)
{
    if (!plan)
        return PA_DECODE_INVALID_ARG;
    int st = check_desc(d);
    if (st != PA_DECODE_OK)
        return st;
    const bool balanced = partition_size == PA_DECODE_PARTITION_BALANCED;
    if (num_cus <= 0 || waves_per_cu <= 0 || batch < 0 || batch > d.max_batch ||
        max_context_len < 0 || max_context_len > d.max_context_len ||
        (partition_size < 0 && !balanced))
        return PA_DECODE_INVALID_ARG;
    if (partition_size > 0 && partition_size % d.page_size != 0)
        return PA_DECODE_INVALID_ARG;

    const int ps = d.page_size;
    const int nb = pages_per_block(d.head_dim, d.dtype);
    const int64_t units = int64_t(std::max(batch, 1)) * d.num_kv_heads;
    const bool windowed = sliding_window > 0 && sliding_window < max_context_len;
    const int64_t visible = windowed ? sliding_window : max_context_len;
    // Pages a visible range can touch (one more when the window edge is not
    // page aligned).
    const int64_t vis_pages = ceil_div(std::max<int64_t>(visible, 1), ps) + (windowed ? 1 : 0);
    if (balanced && batch > 0)   // (an empty batch launches nothing either way)
        return make_balanced_plan(d, num_cus, waves_per_cu, tune, batch, vis_pages, plan);
    // Waves the grid aims for: about four per compute unit (one per SIMD),
    // never more than the device holds at once.  Measured on MI355X, fewer
    // waves with more pages each stream KV faster than more, shorter waves.
    // With rotary and a batch, two waves per SIMD: a rotary block costs
    // about twice the instructions, so the waves of the longest sequences
    // set the time, and smaller partitions spread them (measured on MI355X:
    // batch 16 with lengths up to 4096, 38.7 us against 44.5; one sequence
    // gains nothing, its partitions are all full).
    const int64_t capacity = int64_t(num_cus) * waves_per_cu;
    const int per_cu = (d.rotary_mode == 1 && batch > 1) ? 8 : 4;
    const int64_t target = std::min<int64_t>(capacity, int64_t(num_cus) * per_cu);

    // The layout for partition size S: partitions, the waves sharing one
    // partition, the waves per workgroup and the grid.
    struct Layout {
        bool ok;
        int64_t S, P;
        bool split;
        int wpp, nw, slots;
        int64_t gx;
    };
    const int nw0 = workgroup_waves(d);
    auto layout = [&](int64_t S) {
        Layout L = {};
        int64_t P;
        if (max_context_len == 0) {
            P = 1;
        } else if (windowed) {
            // A window's partitions sit on multiples of S, so its visible
            // range can touch one partition more than visible / S.
            P = std::min(ceil_div(max_context_len, S), ceil_div(visible, S) + 1);
        } else {
            P = ceil_div(max_context_len, S);
        }
        P = std::max<int64_t>(P, 1);
        if (P > 65535 * int64_t(kMaxWavesPerGroup))
            return L;
        const bool split = P > 1;
        if (!split && partition_size == 0 && max_context_len > 0) {
            // The unsplit path covers the whole context with one workgroup.
            S = ceil_div(max_context_len, ps) * ps;
        }
        // Waves sharing one partition: the count (1, 2 or 4, at most one per
        // block of the partition) whose grid total is closest to `target` and
        // fits in one round of resident waves.
        const int64_t blocks = ceil_div(
            ceil_div(std::min<int64_t>(S, std::max<int64_t>(visible, 1)), ps) + (windowed ? 1 : 0), nb);
        int wpp = 1;
        {
            int64_t best = -1;
            for (int cand = 1; cand <= nw0; cand *= 2) {
                if (cand > 1 && (cand > blocks || units * P * cand > capacity)) break;
                const int64_t dist = std::abs(units * P * cand - target);
                if (best < 0 || dist < best) {
                    best = dist;
                    wpp = cand;
                }
            }
        }
        if (!split)
            wpp = int(std::min<int64_t>(nw0, std::max<int64_t>(1, blocks)));  // one partition: all waves on it
        // Experiments only: an override of the choice.
        if (tune.waves_per_partition > 0) wpp = std::min(tune.waves_per_partition, nw0);
        // A grid with fewer partitions than two per compute unit gets one
        // partition per workgroup, so that its workgroups spread over the
        // compute units instead of sharing a few.
        int nw = nw0;
        if (!split || units * P < int64_t(num_cus) * 2)
            nw = wpp;
        // head_dim 256, a grid of 4-wave partitions a little past one per
        // compute unit: two waves per partition and two partitions per
        // workgroup instead, when that fits one workgroup per unit.  The
        // doubled-up units run two waves per SIMD, and at head_dim 256 (8 KiB
        // K and V blocks) a unit streams no faster with eight waves than with
        // four; measured on MI355X with fixed partition sizes, 13-17 % faster
        // per step (batch 2 x 32k tokens, S 1008: 63.1 against 52.6 us;
        // batch 4 x 8k, S 496: 33.8 against 28.9; window 4096 at batch 8,
        // S 512: 33.8 against 29.4).  Head_dim 64 and 128 gain from the
        // second wave per SIMD and keep four waves per partition (1-6 %).
        if (d.head_dim == 256 && split && nw0 == 4 && wpp == 4 && tune.waves_per_partition <= 0 &&
            tune.waves_per_group <= 0 && units * P > num_cus && units * P < int64_t(num_cus) * 2 &&
            units * ceil_div(P, 2) <= num_cus) {
            wpp = 2;
            nw = 4;
        }
        // Experiments only: an override of the workgroup size (a multiple of
        // the waves per partition, so that the workgroup splits into whole
        // slots).
        if (tune.waves_per_group > 0 && tune.waves_per_group >= wpp && tune.waves_per_group % wpp == 0)
            nw = tune.waves_per_group;
        L.ok = true;
        L.S = S;
        L.P = P;
        L.split = split;
        L.wpp = wpp;
        L.nw = nw;
        L.slots = nw / wpp;
        L.gx = ceil_div(P, L.slots);
        return L;
    };
    Layout L;
    if (partition_size > 0) {
        L = layout(partition_size);
    } else {
        // Pages per wave so that `target` waves cover the work, a
        // workgroup's waves (nw0, fewer than four only for head_dim-256
        // rotary) sharing a partition; at least one page per wave and at
        // most 64.
        int64_t ppw = std::max<int64_t>(1, ceil_div(units * vis_pages, target));
        ppw = std::min<int64_t>(ppw, 64);
        L = layout(int64_t(nw0) * ppw * ps);
        // The partition count rounds up, so the grid can end a little past
        // one workgroup per compute unit (at one wave per SIMD), which then
        // doubles up some units: measured on MI355X, those units set the
        // kernel's end (head_dim 256 window at batch 8, 288 workgroups: 35.0
        // us per step against 29.6 at 256; head_dim 64 at 88k tokens, 264
        // workgroups: 59.4 against 46.5).  So among up to twice the pages
        // per wave (at most 256), take the layout with the least work on the
        // busiest unit: rounds of workgroups per unit (as many at once as the
        // wave target per unit allows) times pages per wave.
        const int64_t unit_waves = std::max<int64_t>(1, target / num_cus);
        auto cost = [&](const Layout& x) {
            const int64_t per_unit = std::max<int64_t>(1, unit_waves / x.nw);
            const int64_t wgs = x.gx * d.num_kv_heads * std::max(batch, 1);
            return ceil_div(wgs, int64_t(num_cus) * per_unit) * ceil_div(x.S / ps, x.wpp);
        };
        if (L.ok && L.split) {
            int64_t best = cost(L);
            const int64_t last = std::min<int64_t>(256, 2 * ppw);
            for (int64_t q = ppw + 1; q <= last; ++q) {
                const Layout c = layout(int64_t(nw0) * q * ps);
                if (!c.ok || !c.split)
                    break;
                const int64_t k = cost(c);
                if (k < best) {
                    best = k;
                    L = c;
                }
            }
        }
    }
    if (!L.ok)
        return PA_DECODE_UNSUPPORTED;
    const int64_t S = L.S, P = L.P, gx = L.gx;
    const bool split = L.split;
    const int wpp = L.wpp, nw = L.nw;
    if (gx > 65535)
        return PA_DECODE_UNSUPPORTED;

    pa_decode_plan p = {};
    p.split = split ? 1 : 0;
    p.partition_size = int32_t(S);
    p.num_partitions = int32_t(P);
    p.waves_per_group = nw;
    p.waves_per_partition = wpp;
    p.pages_per_block = nb;
    p.grid_partial[0] = int32_t(gx);
    p.grid_partial[1] = d.num_kv_heads;
    p.grid_partial[2] = batch;
    p.block_partial = nw * 64;
    if (split) {
        if (set_merge_grid(d, batch, P, &p) != PA_DECODE_OK)
            return PA_DECODE_UNSUPPORTED;
        p.workspace_bytes = int64_t(workspace_layout(d, batch, int(P)).total);
    }
    p.num_cus = num_cus;
    p.waves_per_cu = waves_per_cu;
    *plan = p;
    return PA_DECODE_OK;
}

int make_plan_csr(const pa_decode_desc& d, int num_cus, int waves_per_cu, const PlanTuning& tune,
                  int batch, int nnz_pages, int max_context_len, int sliding_window,
                  int partition_size, pa_decode_plan* plan, int* max_ctx_used)
{
    if (!plan || nnz_pages < 0 || batch < 0 || max_context_len < 0 ||
        (partition_size < 0 && partition_size != PA_DECODE_PARTITION_BALANCED))
        return PA_DECODE_INVALID_ARG;
    if (batch == 0 && nnz_pages != 0)
        return PA_DECODE_INVALID_ARG;
    const int64_t ps = d.page_size > 0 ? d.page_size : kPageSize;
    int64_t mc = max_context_len;
    if (mc == 0)
        mc = std::min<int64_t>(int64_t(nnz_pages) * ps, d.max_context_len);
    if (max_ctx_used)
        *max_ctx_used = int(mc);
    int S = partition_size;
    if (S == 0 && int64_t(nnz_pages) * ps <= int64_t(batch) * 256) {
        // Short contexts on average: a single partition covers every context.
        const int64_t cover = std::max<int64_t>(1, (std::max<int64_t>(mc, 1) + ps - 1) / ps) * ps;
        if (cover > INT32_MAX)
            return PA_DECODE_UNSUPPORTED;
        S = int(cover);
    } else if (S == 0 && batch >= kRaggedMinBatch && batch <= kBalancedMaxBatch &&
               int64_t(nnz_pages) * kRaggedDen <
                   int64_t(batch) * ((mc + ps - 1) / ps) * kRaggedNum) {
        // A ragged batch: the length-balanced schedule, when it takes these
        // sizes (else the fixed split below).
        const int st = make_plan(d, num_cus, waves_per_cu, tune, batch, int(mc), sliding_window,
                                 PA_DECODE_PARTITION_BALANCED, plan);
        if (st != PA_DECODE_UNSUPPORTED)
            return st;
    }
    return make_plan(d, num_cus, waves_per_cu, tune, batch, int(mc), sliding_window, S, plan);
}

int64_t rotary_table_bytes(const pa_decode_desc& d)
{
    // [pages per block][head_dim / 2] (cos, sin) pairs of f32
    return d.rotary_mode == 1
               ? int64_t(pages_per_block(d.head_dim, d.dtype)) * (d.head_dim / 2) * 8
               : 0;
}

int64_t rotary_offset_table_bytes(const pa_decode_desc& d)
{
    // [16 in-page offsets][head_dim + 4] f32: (cos, sin) pairs, padded rows;
    // then [head_dim / 2] f64 revolutions per position
    return d.rotary_mode == 1
               ? int64_t(kPageSize) * (d.head_dim + 4) * 4 + int64_t(d.head_dim / 2) * 8
               : 0;
}

size_t partial_lds_bytes(const pa_decode_desc& d, const pa_decode_plan& plan)
{
    const int G = template_group(d.num_q_heads / d.num_kv_heads);
    const int gp4 = (G + 3) / 4 * 4;
    const int nw = plan.waves_per_group;
    // per wave: the block's K and V tiles (4-8 KiB each)
    const size_t ktile = size_t(plan.pages_per_block) * kPageSize * 16 *
                         size_t(tile_row_slots(d.head_dim, d.dtype)) / sizeof(float);
    const size_t loop =
        size_t(nw) * (2 * ktile + size_t(rotary_table_bytes(d)) / sizeof(float)) +
        size_t(rotary_offset_table_bytes(d)) / sizeof(float);
    const size_t comb = size_t(nw) * size_t(2 * gp4 + G * d.head_dim);
#if PA_QK_VALU
    // Comparison build (scores on the vector ALUs): per wave a q copy when G
    // x (chunks / 4) > 24, and [pages per block][16][16] score floats.
    if (d.rotary_mode == 0) {
        const int ch = d.head_dim * dtype_bytes(d.dtype) / 16;
        const size_t extra = (G * (ch / 4) <= 24 ? 0 : size_t(G) * ch * 4) +
                             size_t(plan.pages_per_block) * 256;
        return std::max(loop + size_t(nw) * extra, comb) * sizeof(float);
    }
#endif
    return std::max(loop, comb) * sizeof(float);
}

}  // namespace pa
