// kernels.h -- launch interface of the gfx950 decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "planner.h"

namespace pa {

// Arguments of the partial kernel (fixed schedule: one workgroup per
// (group of partitions, KV head, b); balanced schedule: bal_waves waves per
// KV head).
struct PartialParams {
    const void* q;            // [B, Hq, D]
    const void* k;            // paged K, element strides below (D contiguous)
    const void* v;            // paged V, same strides
    int64_t stride_page, stride_head, stride_slot;
    const int32_t* page_table;    // dense: [B, pt_stride]; CSR: page indices
    int32_t pt_stride;
    const int32_t* context_lens;  // dense form only
    const int32_t* page_indptr;   // CSR form ([B + 1]); null for the dense form
    const int32_t* last_page_len; // CSR form ([B])
    int32_t num_q_heads;
    int32_t group;            // actual G = Hq / Hkv
    int32_t partition_size;   // S tokens
    int32_t num_partitions;   // P: partitions per (sequence, KV head)
    int32_t waves_per_partition;  // waves of a workgroup that share one partition
    int32_t window;           // <= 0: none
    float scale_log2;         // scale * log2(e)
    int32_t split;            // 1: write partition states; 0: write out/lse
    float* ws_o;              // [B, Hq, P, D]
    float* ws_m;              // [B, Hq, P], base-2 running max
    float* ws_l;              // [B, Hq, P], denominators
    void* out;                // [B, Hq, D]
    float* lse;               // [B, Hq] or null
    // Device-side contract (checked in the kernel, never trusted for an
    // address): page ids outside [0, num_pages) read page 0; context lengths
    // are clamped to [0, max_context_len]; CSR rows to [0, nnz_pages].  Each
    // violation ORs a PA_DECODE_VIOLATION_* bit into *status when status is
    // not null.
    int32_t num_pages;
    int32_t max_context_len;
    int32_t nnz_pages;
    int32_t* status;
    int32_t rotary;           // 1: rotary embedding of q and keys (rotary_mode 1)
    double rope_rho;          // rope_theta^(-2/D): theta_i = rope_rho^i / rope_scale
    double rope_f0;           // 1 / (2 pi rope_scale): theta_0 in revolutions
    float minus_one;          // -1 (a value the compiler cannot fold; see TurnedKey)
    // Length-balanced schedule (launch_partial_balanced only): the visible
    // pages of the batch's `batch` (<= 64) sequences, in sequence order, are
    // split into bal_waves contiguous ranges, one per wave of the KV head
    // (grid x * waves per workgroup = bal_waves).  ws_cnt[b * Hq + h]
    // receives the number of state rows of (sequence b, query head h): rows
    // of ws_o / ws_m / ws_l at partition index 0 .. count - 1,
    // num_partitions being their pitch.
    int32_t batch;
    int32_t bal_waves;
    int32_t bal_start;        // pages charged for each sequence's start (>= 0)
    int32_t* ws_cnt;
};

// Arguments of the merge kernel (one workgroup per (query head, b)).
struct MergeParams {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_partitions;
    const float* ws_o;
    const float* ws_m;
    const float* ws_l;
    void* out;
    float* lse;
    // Null: every (sequence, head) has num_partitions state rows.  Otherwise
    // (length-balanced schedule) (sequence b, query head h) has
    // ws_cnt[b * Hq + h] rows (at most the pitch num_partitions); the rows
    // past it hold no state and are never used.
    const int32_t* ws_cnt;
};

// Optional start/stop events recorded around one launch (both null: none).
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// dtype: PA_DTYPE_*; group_t: an instantiated group size (template_group).
hipError_t launch_partial(int dtype, int head_dim, int group_t, const PartialParams& p,
                          dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream,
                          LaunchEvents ev);
// The partial kernel with the length-balanced schedule (p.bal_waves > 0,
// p.batch <= 64, one wave per partition slot).
hipError_t launch_partial_balanced(int dtype, int head_dim, int group_t, const PartialParams& p,
                                   dim3 grid, dim3 block, size_t lds_bytes, hipStream_t stream,
                                   LaunchEvents ev);
hipError_t launch_merge(int dtype, int head_dim, const MergeParams& p, dim3 grid, dim3 block,
                        hipStream_t stream, LaunchEvents ev);

// Read probe (measurement): reads num_chunks chunks of kpc * 1024 bytes
// (kpc in {2, 3, 4, 8}) with the partial kernel's streaming load; chunk i at
// chunk_addrs[i], or at base + i * chunk bytes when chunk_addrs is null;
// *sink is XORed with the XOR of every 32-bit word read.
hipError_t launch_read_probe(const void* base, const uint64_t* chunk_addrs, int32_t num_chunks,
                             int kpc, uint32_t* sink, hipStream_t stream);

// Waves of the partial kernel (workgroups of `waves` waves with `lds_bytes`
// of dynamic LDS, with or without rotary) that one compute unit holds at
// once; 0 when unknown.
int partial_waves_per_cu(int dtype, int head_dim, int group_t, bool rotary, int waves,
                         size_t lds_bytes);
int partial_balanced_waves_per_cu(int dtype, int head_dim, int group_t, bool rotary, int waves,
                                  size_t lds_bytes);

}  // namespace pa
