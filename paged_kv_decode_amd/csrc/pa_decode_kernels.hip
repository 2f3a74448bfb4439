// pa_decode_kernels.hip -- gfx950 kernels of paged-KV GQA decode attention:
// instantiations of the partial kernel (partial_kernel.h) for the fixed-
// partition schedule, the merge kernels, the read probe and the host-side
// launch dispatch.
//
// Merge kernel: one workgroup per (query head, sequence): phase 1 takes the
// maximum of the partition maxima and the rescaled sum of denominators,
// phase 2 sums the partition outputs weighted by rescale_p / total, then
// lse = ln(total) + max.  The two phases follow the paged_attention_v2
// commit page, "Phase 2: Cross-partition reduction" (global max; rescale =
// exp(m_p - max) * l_p; out = sum rescale_p / sum(rescale) * o_p), and TVM
// PR #20426, section "Change", third bullet ((max, denom) first, then the
// weighted outputs).
#include "partial_kernel.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// Merge kernel for any partition count: one 256-thread workgroup per (query
// head, sequence, 16-column slice of head_dim), so that even one sequence
// spreads its reads over many compute units (the 100k workload: 24 heads x
// 16 slices = 384 workgroups).  Every wave finds the global maximum and the
// rescaled denominator sum itself (lane-strided loads, DPP and lane-swap
// reductions, no barrier).  For the outputs the 64 row groups (16 per wave,
// 4 lanes each) take rows rg, rg + 64, ...; lane c4 of a row group reads
// float4 column c4 of the slice, every load of a 256-row pass issued before
// the first use, and a row's weight comes by lane permute from the lane of
// the same wave that holds its maximum and denominator (row rg + 64 i is
// partition lane rg, k = i of the strided layout).  The row groups of a
// wave are summed with lane swaps and the four waves through LDS (one
// barrier).  Empty partitions carry max = -inf and denominator 0 and get
// weight 0; rows past P re-read row P - 1 with weight 0.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams prm)
{
    constexpr int RPT = 4;                // rows per lane per pass (64 row groups x 4 = 256)
    __shared__ f32x4 part[4][4];
    const int h = blockIdx.x, b = blockIdx.y, dsl = blockIdx.z;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int rg = 16 * wave + (lane >> 2), c4 = lane & 3;   // row group 0..63, float4 column
    const int P = prm.num_partitions;
    const size_t hrow = size_t(b) * prm.num_q_heads + h;
    const float* m = prm.ws_m + hrow * P;
    const float* l = prm.ws_l + hrow * P;
    const int col = dsl * 16 + 4 * c4;
    const char* ob = reinterpret_cast<const char*>(prm.ws_o + hrow * P * D);

    // First pass of rows, loaded before anything waits.
    f32x4 orow[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const uint32_t row = uint32_t(min(rg + 64 * i, P - 1));
        orow[i] = *reinterpret_cast<const f32x4*>(ob + (row * D + uint32_t(col)) * 4u);
    }
    // Lane-strided maxima and denominators (partition lane + 64 k) for the
    // wave's own reductions and, by lane permutes, the first pass's weights.
    float ms[4], ls[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = min(lane + kWave * k, P - 1);
        ms[k] = m[p];
        ls[k] = l[p];
    }
    pin_loads();

    // Phase 1: global max of the partition maxima (entries past P repeat
    // entry P - 1, which leaves the max unchanged).
    float mx = fmaxf(fmaxf(ms[0], ms[1]), fmaxf(ms[2], ms[3]));
    for (int p = lane + 4 * kWave; p < P; p += kWave) mx = fmaxf(mx, m[p]);
    const float M = rows4_max(row16_max(mx));
    if (M == -INFINITY) {
        // Every partition empty: out = 0, lse = -inf.
        if (threadIdx.x < 4)
            store_out4<DT>(prm.out, hrow * D + col, f32x4{0.f, 0.f, 0.f, 0.f});
        if (prm.lse && dsl == 0 && threadIdx.x == 0) prm.lse[hrow] = -INFINITY;
        return;
    }
    // Phase 2: rescale_p = 2^(m_p - M) * l_p; their sum, and the weighted
    // outputs.
    auto weight = [&](float mp, float lp) { return lp > 0.f ? fast_exp2(mp - M) * lp : 0.f; };
    float wk[4], tl = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        wk[k] = lane + kWave * k < P ? weight(ms[k], ls[k]) : 0.f;
        tl += wk[k];
    }
    for (int p = lane + 4 * kWave; p < P; p += kWave) tl += weight(m[p], l[p]);
    const float L = rows4_sum(row16_sum(tl));

    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float wr =
            __int_as_float(__builtin_amdgcn_ds_bpermute(rg * 4, __float_as_int(wk[i])));
        a += wr * orow[i];
    }
    // Further passes (more than 256 partitions).
    for (int p = rg + 64 * RPT; p < P; p += 64) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(ob + (uint32_t(p) * D + uint32_t(col)) * 4u);
        a += weight(m[p], l[p]) * o;
    }
    // Sum the 16 row groups of the wave (lanes c4, c4 + 4, ..., c4 + 60).
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = a[e];
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        a[e] = rows4_sum(x);
    }
    if (lane < 4) part[wave][c4] = a;
    __syncthreads();
    if (threadIdx.x < 4) {
        const f32x4 t = part[0][c4] + part[1][c4] + part[2][c4] + part[3][c4];
        store_out4<DT>(prm.out, hrow * D + col, t * (1.f / L));
    }
    if (prm.lse && dsl == 0 && threadIdx.x == 0) prm.lse[hrow] = (M + log2f(L)) * kLn2;
}

// Merge kernel for up to PMAX (<= 64) partitions: one wave per (sequence,
// query head, CW-column slice of head_dim; CW = 64, or 16 when the batch
// and heads give few waves).  Lane p holds partition p's max and
// denominator; the global max and the denominator sum reduce across the
// wave with DPP and lane swaps (no barrier).  For the outputs the lanes form
// 64 / (CW / 4) row groups of CW / 4 lanes; lane c4 of row group rg reads
// float4 column c4 of rows rg, rg + NRG, ..., all before the first
// reduction, takes each row's weight from the lane that holds it, and the
// row groups are summed with lane swaps at the end.  Rows past P re-read
// row P - 1 with weight 0.
template <int DT, int D, int PMAX, int CW>
__global__ __launch_bounds__(256) void merge_wave_kernel(const MergeParams prm, int units)
{
    constexpr int NS = (D + CW - 1) / CW;   // slices (the last may be partial for CW = 64)
    constexpr int LPR = CW / 4;             // lanes per row group
    constexpr int NRG = kWave / LPR;        // row groups
    constexpr int RPL = PMAX / NRG;         // rows per lane
    static_assert(RPL * NRG == PMAX && PMAX <= kWave, "rows");
    const int lane = threadIdx.x & (kWave - 1);
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) +
                                                    threadIdx.x / kWave);
    if (unit >= units)
        return;
    const int P = prm.num_partitions;
    const int slice = unit % NS;
    const size_t hrow = size_t(unit / NS);   // b * Hq + h
    const int rg = lane / LPR, c4 = lane % LPR;
    const int col = slice * CW + 4 * c4;
    const bool has_col = col < D;           // head_dim 96, CW 64: the last slice has 32 columns
    // Branch-free loads (lanes past P re-read entry P - 1), all issued
    // before the first use.
    const int pl = min(lane, P - 1);
    const float mraw = prm.ws_m[hrow * P + pl];
    const float lraw = prm.ws_l[hrow * P + pl];
    // Wave-uniform base of this head's rows; per-lane 32-bit byte offsets.
    const char* ob = reinterpret_cast<const char*>(prm.ws_o + hrow * P * D);
    f32x4 orow[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const uint32_t row = uint32_t(min(rg + NRG * i, P - 1));
        orow[i] = *reinterpret_cast<const f32x4*>(ob + (row * D + uint32_t(has_col ? col : 0)) * 4u);
    }
    pin_loads();
    const float mp = lane < P ? mraw : -INFINITY;
    const float lp = lane < P ? lraw : 0.f;

    // Phase 1: global max of the partition maxima.
    const float M = rows4_max(row16_max(mp));
    if (M == -INFINITY) {
        // Every partition empty: out = 0, lse = -inf.
        if (rg == 0 && has_col) store_out4<DT>(prm.out, hrow * D + col, f32x4{0.f, 0.f, 0.f, 0.f});
        if (prm.lse && slice == 0 && lane == 0) prm.lse[hrow] = -INFINITY;
        return;
    }
    // Phase 2: rescale each partition's denominator (rescale_p =
    // 2^(m_p - M) * l_p), sum them, and weight the partition outputs.
    const float w = lp > 0.f ? fast_exp2(mp - M) * lp : 0.f;
    const float L = rows4_sum(row16_sum(w));
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const float wr = __int_as_float(__builtin_amdgcn_ds_bpermute((rg + NRG * i) * 4, __float_as_int(w)));
        a += wr * orow[i];
    }
    // Sum the row groups: within each 16-lane row first (CW 16: lanes c4,
    // c4 + 4, c4 + 8, c4 + 12), then across the four rows.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = a[e];
        if constexpr (LPR == 4) {
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
        }
        a[e] = rows4_sum(x);
    }
    if (rg == 0 && has_col) store_out4<DT>(prm.out, hrow * D + col, a * (1.f / L));
    if (prm.lse && slice == 0 && lane == 0) prm.lse[hrow] = (M + log2f(L)) * kLn2;
}

// Merge kernel of the length-balanced schedule: (sequence b, query head h)
// has cnt = ws_cnt[b * Hq + h] state rows (at most the row pitch P), one
// wave per (b, h, CW-column slice) as in merge_wave_kernel.  No load waits
// for cnt: lane p reads the maximum and denominator of row p, and the row
// groups read their first RS rows (32 for CW 16, 16 for CW 64; clamped to
// the pitch), which covers the usual counts; rows at or past cnt are left
// out by selects (their contents are undefined), and rows from RS on are
// read once cnt is known.
template <int DT, int D, int CW>
__global__ __launch_bounds__(256) void merge_count_kernel(const MergeParams prm, int units)
{
    constexpr int NS = (D + CW - 1) / CW;   // slices (the last may be partial for CW = 64)
    constexpr int LPR = CW / 4;             // lanes per row group
    constexpr int NRG = kWave / LPR;        // row groups
    constexpr int RPL = CW == 16 ? 2 : 4;   // first-pass rows per lane
    constexpr int RS = RPL * NRG;           // first-pass rows
    static_assert(RS <= kWave, "first-pass rows have their weights in lanes");
    const int lane = threadIdx.x & (kWave - 1);
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) +
                                                    threadIdx.x / kWave);
    if (unit >= units)
        return;
    const int P = prm.num_partitions;       // row pitch
    const int slice = unit % NS;
    const size_t hrow = size_t(unit / NS);  // b * Hq + h
    const int rg = lane / LPR, c4 = lane % LPR;
    const int col = slice * CW + 4 * c4;
    const bool has_col = col < D;
    const int cnt = min(max(prm.ws_cnt[hrow], 0), P);
    const float* m = prm.ws_m + hrow * P;
    const float* l = prm.ws_l + hrow * P;
    const int pl = min(lane, P - 1);
    const float mraw = m[pl];
    const float lraw = l[pl];
    const char* ob = reinterpret_cast<const char*>(prm.ws_o + hrow * P * D);
    const uint32_t cb = uint32_t(has_col ? col : 0);
    f32x4 orow[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const uint32_t row = uint32_t(min(rg + NRG * i, P - 1));
        orow[i] = *reinterpret_cast<const f32x4*>(ob + (row * D + cb) * 4u);
    }
    pin_loads();
    auto empty = [&]() {
        if (rg == 0 && has_col) store_out4<DT>(prm.out, hrow * D + col, f32x4{0.f, 0.f, 0.f, 0.f});
        if (prm.lse && slice == 0 && lane == 0) prm.lse[hrow] = -INFINITY;
    };
    if (cnt == 0) {
        empty();
        return;
    }
    const float mp = lane < cnt ? mraw : -INFINITY;
    const float lp = lane < cnt ? lraw : 0.f;
    float mx = mp;
    for (int p = lane + kWave; p < cnt; p += kWave) mx = fmaxf(mx, m[p]);   // more than 64 rows
    const float M = rows4_max(row16_max(mx));
    if (M == -INFINITY) {
        empty();
        return;
    }
    auto weight = [&](float mq, float lq) { return lq > 0.f ? fast_exp2(mq - M) * lq : 0.f; };
    const float w = weight(mp, lp);
    float tl = w;
    for (int p = lane + kWave; p < cnt; p += kWave) tl += weight(m[p], l[p]);
    const float L = rows4_sum(row16_sum(tl));
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int row = rg + NRG * i;
        const float wr = __int_as_float(__builtin_amdgcn_ds_bpermute(row * 4, __float_as_int(w)));
        a = row < cnt ? a + wr * orow[i] : a;
    }
    // Rows from RS on, four per lane per pass with every load of a pass
    // issued before the first use (a wave-uniform loop, so that every lane
    // takes part in the lane permutes).
    constexpr int UR = 4;
    for (int base = RS; base < cnt; base += UR * NRG) {
        f32x4 o[UR];
        float mq[UR], lq[UR];
        const bool far = base + UR * NRG > kWave;   // rows past 64: weights from memory
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const uint32_t rc = uint32_t(min(base + u * NRG + rg, cnt - 1));
            o[u] = *reinterpret_cast<const f32x4*>(ob + (rc * D + cb) * 4u);
            mq[u] = far ? m[rc] : 0.f;
            lq[u] = far ? l[rc] : 0.f;
        }
        pin_loads();
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int row = base + u * NRG + rg;
            float wr = __int_as_float(
                __builtin_amdgcn_ds_bpermute((row & (kWave - 1)) * 4, __float_as_int(w)));
            wr = row < kWave ? wr : weight(mq[u], lq[u]);
            a = row < cnt ? a + wr * o[u] : a;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = a[e];
        if constexpr (LPR == 4) {
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
        }
        a[e] = rows4_sum(x);
    }
    if (rg == 0 && has_col) store_out4<DT>(prm.out, hrow * D + col, a * (1.f / L));
    if (prm.lse && slice == 0 && lane == 0) prm.lse[hrow] = (M + log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// Read probe (a measurement tool, not part of the decode step): the rate at
// which the memory system delivers a given set of KV chunks to the same
// streaming load the partial kernel uses.  W = PA_DECODE_PROBE_WAVES waves
// (one per SIMD); wave w reads the chunks [w n / W, (w + 1) n / W) of the
// list through a ring of NBUF chunk slots in registers (~16 KiB): a slot is
// refilled with the chunk NBUF ahead as soon as its data has been folded
// into the wave's XOR, so the wave keeps its loads in flight from start to
// end.  Each wave then stores its XOR in sink[w]: no atomics (atomics on one
// word serialise at ~10 ns each on MI355X, microseconds for a few hundred
// workgroups).
// ---------------------------------------------------------------------------
template <int KPC>
__global__ __launch_bounds__(256) void read_probe_kernel(const char* base,
                                                         const uint64_t* chunk_addrs,
                                                         int32_t num_chunks, uint32_t* sink)
{
    constexpr int CB = KPC * kWave * 16;   // chunk bytes
    constexpr int NBUF = KPC == 8 ? 2 : KPC == 4 ? 4 : KPC == 3 ? 5 : 8;   // slots (15-16 KiB)
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) +
                                                 threadIdx.x / kWave);
    const int nwv = gridDim.x * (blockDim.x / kWave);
    const int c0 = int(int64_t(w) * num_chunks / nwv);
    const int c1 = int(int64_t(w + 1) * num_chunks / nwv);
    typedef __attribute__((address_space(1))) const u32x4 gvec;   // global memory
    auto chunk = [&](int c) -> uint64_t {
        return chunk_addrs ? chunk_addrs[c] : reinterpret_cast<uint64_t>(base) + uint64_t(c) * CB;
    };
    u32x4 r[NBUF][KPC];
    auto issue = [&](int s, int c) {
        const uint64_t a = chunk(c) + uint64_t(lane * 16);
#pragma unroll
        for (int k = 0; k < KPC; ++k)
            r[s][k] = __builtin_nontemporal_load(reinterpret_cast<gvec*>(a + uint64_t(k * kWave * 16)));
    };
#pragma unroll
    for (int s = 0; s < NBUF; ++s)
        if (c0 + s < c1) issue(s, c0 + s);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int c = c0; c < c1; c += NBUF) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
            if (c + s < c1) {
#pragma unroll
                for (int k = 0; k < KPC; ++k) acc ^= r[s][k];
                if (c + s + NBUF < c1) issue(s, c + s + NBUF);
            }
        }
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
    if (lane == 0)
        sink[w] = x;
}

}  // namespace

hipError_t launch_partial(int dtype, int head_dim, int group_t, const PartialParams& p, dim3 grid,
                          dim3 block, size_t lds, hipStream_t stream, LaunchEvents ev)
{
    return launch_partial_any<false>(dtype, head_dim, group_t, p, grid, block, lds, stream, ev);
}

int partial_waves_per_cu(int dtype, int head_dim, int group_t, bool rotary, int waves,
                         size_t lds)
{
    return partial_waves_any<false>(dtype, head_dim, group_t, rotary, waves, lds);
}

template <int DT, int D>
hipError_t launch_merge_t(const MergeParams& p, dim3 grid, dim3 block, hipStream_t stream,
                          LaunchEvents ev)
{
    if (p.ws_cnt) {
        const int cw = merge_slice_width(p.batch, p.num_q_heads, D);
        const int units = p.batch * p.num_q_heads * ((D + cw - 1) / cw);
        if (cw == 16)
            return launch(merge_count_kernel<DT, D, 16>, grid, block, 0, stream, ev, p, units);
        return launch(merge_count_kernel<DT, D, 64>, grid, block, 0, stream, ev, p, units);
    }
    if (p.num_partitions <= kMergeWaveMaxPartitions) {
        const int cw = merge_slice_width(p.batch, p.num_q_heads, D);
        const int units = p.batch * p.num_q_heads * ((D + cw - 1) / cw);
        if (cw == 16) {
            if (p.num_partitions <= 16)
                return launch(merge_wave_kernel<DT, D, 16, 16>, grid, block, 0, stream, ev, p, units);
            if (p.num_partitions <= 32)
                return launch(merge_wave_kernel<DT, D, 32, 16>, grid, block, 0, stream, ev, p, units);
            return launch(merge_wave_kernel<DT, D, 64, 16>, grid, block, 0, stream, ev, p, units);
        }
        if (p.num_partitions <= 16)
            return launch(merge_wave_kernel<DT, D, 16, 64>, grid, block, 0, stream, ev, p, units);
        if (p.num_partitions <= 32)
            return launch(merge_wave_kernel<DT, D, 32, 64>, grid, block, 0, stream, ev, p, units);
        return launch(merge_wave_kernel<DT, D, 64, 64>, grid, block, 0, stream, ev, p, units);
    }
    return launch(merge_kernel<DT, D>, grid, block, 0, stream, ev, p);
}

hipError_t launch_read_probe(const void* base, const uint64_t* chunk_addrs, int32_t num_chunks,
                             int kpc, uint32_t* sink, hipStream_t stream)
{
    if (num_chunks <= 0)
        return hipSuccess;   // nothing to read; the sink is left as it is
    // PA_DECODE_PROBE_WAVES waves in workgroups of four, whatever the chunk
    // count (waves without chunks store 0).
    static_assert(PA_DECODE_PROBE_WAVES % 4 == 0, "workgroups of four waves");
    const dim3 grid(PA_DECODE_PROBE_WAVES / 4), block(4 * kWave);
    const char* b = static_cast<const char*>(base);
    switch (kpc) {
    case 2: hipLaunchKernelGGL(read_probe_kernel<2>, grid, block, 0, stream, b, chunk_addrs, num_chunks, sink); break;
    case 3: hipLaunchKernelGGL(read_probe_kernel<3>, grid, block, 0, stream, b, chunk_addrs, num_chunks, sink); break;
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, grid, block, 0, stream, b, chunk_addrs, num_chunks, sink); break;
    case 8: hipLaunchKernelGGL(read_probe_kernel<8>, grid, block, 0, stream, b, chunk_addrs, num_chunks, sink); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(int dtype, int head_dim, const MergeParams& p, dim3 grid, dim3 block,
                        hipStream_t stream, LaunchEvents ev)
{
#define PA_MERGE(DT, D) return launch_merge_t<DT, D>(p, grid, block, stream, ev);
    if (dtype == PA_DTYPE_F32 && head_dim == 64) { PA_MERGE(PA_DTYPE_F32, 64) }
    if (dtype == PA_DTYPE_F16) {
        if (head_dim == 64) { PA_MERGE(PA_DTYPE_F16, 64) }
        if (head_dim == 96) { PA_MERGE(PA_DTYPE_F16, 96) }
        if (head_dim == 128) { PA_MERGE(PA_DTYPE_F16, 128) }
        if (head_dim == 256) { PA_MERGE(PA_DTYPE_F16, 256) }
    }
    if (dtype == PA_DTYPE_BF16) {
        if (head_dim == 64) { PA_MERGE(PA_DTYPE_BF16, 64) }
        if (head_dim == 96) { PA_MERGE(PA_DTYPE_BF16, 96) }
        if (head_dim == 128) { PA_MERGE(PA_DTYPE_BF16, 128) }
        if (head_dim == 256) { PA_MERGE(PA_DTYPE_BF16, 256) }
    }
#undef PA_MERGE
    return hipErrorInvalidValue;
}

}  // namespace pa
