// planner.h -- host-side dispatch plan for paged-KV decode attention.
//
// Pure host C++: no HIP call, so it is unit-testable without a GPU.
// The plan picks the partition size S (tokens per workgroup), the number of
// partitions per (sequence, KV head), the waves per workgroup, and whether
// the merge kernel runs at all.  A single partition per context means the
// partial kernel writes out/lse directly (the unsplit path for short
// contexts: TVM PR #20426, section "Change", host-side switch between a
// single-pass nest and the sharded one); otherwise the context is split and
// the partition states are merged by log-sum-exp (the paged_attention_v2
// commit page, "Phase 2").
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa_decode.h"

namespace pa {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxWavesPerGroup = 4;
constexpr int kMergeThreads = 256;
// Partition counts up to this use the merge with one wave per (sequence,
// query head, 64-dim slice); its grid is ceil(B * Hq * D/64 / 4) workgroups.
constexpr int kMergeWaveMaxPartitions = 64;
// Columns of head_dim per wave of the merge for up to 64 partitions: 64,
// or 16 when that leaves fewer than 256 waves (one sequence, few heads),
// which spreads the merge's reads over four times the waves.
inline int merge_slice_width(int batch, int num_q_heads, int head_dim)
{
    return int64_t(batch) * num_q_heads * ((head_dim + 63) / 64) < 256 ? 16 : 64;
}
// Largest y / z launch-grid dimension (sequences, KV heads).
constexpr int kMaxGridYZ = 65535;

// Bytes per element of a PA_DTYPE_* code (0 when unknown).
int dtype_bytes(int dtype);

// Pages of K (and of V) one wave holds in flight per step, from the bytes of
// one key row: 256 bytes of a token row times 16 rows, i.e. 4 KiB of K and
// 4 KiB of V per wave, clamped to 1 .. 4 pages (one page of 3 KiB at head_dim
// 96 with 2-byte types, one of 8 KiB at head_dim 256).  The planner and the
// partial kernel's template both take it from here.
constexpr int pages_per_block_for_row(int row_bytes)
{
    return row_bytes <= 0 || 256 / row_bytes < 1 ? 1 : (256 / row_bytes > 4 ? 4 : 256 / row_bytes);
}
int pages_per_block(int head_dim, int dtype);

// 16-byte slots per key row in the kernel's LDS tiles: the row's chunks,
// plus one when that count is not a power of two (head_dim 96).
int tile_row_slots(int head_dim, int dtype);

// The instantiated group size that serves an actual GQA group size G
// (the smallest built one >= G); 0 when G is not supported.
int template_group(int G);

// Checks the static description; returns a PA_DECODE_* status.
int check_desc(const pa_decode_desc& d);

// Overrides of the planner's choices for experiments (0 / -1: the planner's
// own).  They change the work split only, never the result's definition or
// the workspace size.  A handle reads them from the environment once, at
// pa_decode_create (tuning_from_env); the plan-query functions read them at
// each call.
struct PlanTuning {
    int waves_per_partition = 0;   // PA_DECODE_WAVES_PER_PARTITION: 1, 2 or 4
    int waves_per_group = 0;       // PA_DECODE_WAVES_PER_GROUP: 1, 2 or 4
    int balanced_start = -1;       // PA_DECODE_BALANCED_START: 0 .. 64 pages
    int balanced_waves_per_cu = 0; // PA_DECODE_BALANCED_WAVES_PER_CU: 1 .. 16
};
PlanTuning tuning_from_env();

// Fills `plan` for the given call sizes; returns a PA_DECODE_* status.
// waves_per_cu: how many waves of the partial kernel one compute unit holds
// at once (from the kernel's register and LDS use).
int make_plan(const pa_decode_desc& d, int num_cus, int waves_per_cu, const PlanTuning& tune,
              int batch, int max_context_len, int sliding_window, int partition_size,
              pa_decode_plan* plan);

// Ragged-batch rule of the CSR form with partition_size 0: a batch of
// kRaggedMinBatch .. 64 sequences whose mean page count is below
// kRaggedNum / kRaggedDen = 5/8 of the longest possible (nnz_pages * 8 <
// batch * ceil(max_context_len / page_size) * 5) runs the length-balanced
// schedule.  Measured on MI355X (batches of 4 .. 32 at head_dim 128, four
// length mixes, with and without rotary): the balanced schedule lost at
// every mix at batch 4 (3 - 15 %) and from a mean of ~0.66 of the longest on
// (1 - 9 %), while it gained 7 - 191 % at means of 0.10 - 0.57 (under fixed
// partitions the waves of the longest sequences, which hold the most
// blocks, set the step time).
constexpr int kRaggedMinBatch = 8;
constexpr int kRaggedNum = 5;
constexpr int kRaggedDen = 8;

// The plan for a CSR page table (nnz_pages pages in use).  With
// partition_size 0: the host switch of TVM PR #20426, section "Change" (one
// partition per (sequence, KV head) when nnz_pages <= batch * 256 /
// page_size); else, for a ragged batch (the rule above, also a page count
// known on the host), the length-balanced schedule; else the planner's fixed
// split.  max_context_len 0 stands for nnz_pages * page_size; the bound
// actually used is returned in *max_ctx_used (may be null).
int make_plan_csr(const pa_decode_desc& d, int num_cus, int waves_per_cu, const PlanTuning& tune,
                  int batch, int nnz_pages, int max_context_len, int sliding_window,
                  int partition_size, pa_decode_plan* plan, int* max_ctx_used);

// Waves per workgroup of the partial kernel for this description (1, 2 or 4;
// LDS-limited).
int workgroup_waves(const pa_decode_desc& d);

// LDS bytes of one wave's rotary base table (0 without rotary): the (cos,
// sin) of every frequency at each page of a block.
int64_t rotary_table_bytes(const pa_decode_desc& d);

// LDS bytes of a workgroup's rotary offset table (0 without rotary): the
// (cos, sin) of t theta_i for the 16 in-page offsets t.
int64_t rotary_offset_table_bytes(const pa_decode_desc& d);

// Dynamic LDS bytes of the partial kernel for a plan.
size_t partial_lds_bytes(const pa_decode_desc& d, const pa_decode_plan& plan);

// Workspace layout of a split plan: partition outputs o[B][Hq][P][D] (f32),
// maxima m[B][Hq][P] and denominators l[B][Hq][P] (f32), each region
// 256-byte aligned.
// The balanced schedule adds the state-row counts c[B][Hq] (int32).
struct WorkspaceLayout {
    size_t o_off, m_off, l_off, c_off, total;
};
WorkspaceLayout workspace_layout(const pa_decode_desc& d, int batch, int num_partitions,
                                 bool counts = false);

// Largest batch of the length-balanced schedule (one sequence per lane of a
// wave's prefix sum).
constexpr int kBalancedMaxBatch = 64;
// Pages the balanced schedule charges for each sequence's start (0 .. 64):
// four blocks' worth, three with rotary (a segment's start waits for its
// page ids and q before the first block's loads go out, and its pipeline
// starts empty).
int balanced_start_pages(const pa_decode_desc& d, const PlanTuning& tune);

}  // namespace pa
