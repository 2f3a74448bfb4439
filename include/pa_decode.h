/*
 * pa_decode.h -- C ABI of the MI355X (gfx950) paged-KV GQA decode-attention
 * library libpa_decode.so.
 *
 * Operation (one decode step, one query token per sequence):
 *   for every sequence b and query head h, with G = num_q_heads / num_kv_heads
 *   and KV head g = floor(h / G), over the visible keys j in [lo_b, n_b):
 *     s_j      = scale * q[b,h,:] . K_b[j,g,:]
 *     out[b,h] = sum_j softmax(s)_j * V_b[j,g,:]
 *     lse[b,h] = ln sum_j exp(s_j)                      (natural log)
 *   where n_b = context_lens[b] and lo_b = max(0, n_b - sliding_window) when a
 *   window is set (the window holds the W most recent keys, current one
 *   included), else 0.  n_b - lo_b == 0 gives out = 0, lse = -inf.
 *   With desc.rotary_mode == 1 the scores use q and K after the rotary
 *   position embedding (TVM PR #20426, section "Correctness", checks the
 *   kernel with `rotary_mode = 1`; the pages do not define it further, and
 *   this library takes the RoFormer rotation with the rotate-half pairing):
 *   for i < D/2 the pair (x[i], x[i + D/2]) of a vector at position p turns
 *   by the angle p * theta_i, theta_i = rope_theta^(-2i/D) / rope_scale,
 *     x'[i] = x[i] cos - x[i + D/2] sin,   x'[i + D/2] = x[i + D/2] cos + x[i] sin,
 *   key j of sequence b at position j and its query at position n_b - 1.
 *   The cache holds keys as they were before the embedding.
 *   Passages: output and LSE of paged-KV decode attention with a shuffled page
 *   table, sliding window and batch > 1 -- TVM PR #20426, section
 *   "Correctness"; K/V gathered per page through a block table and the
 *   [kv_h, gqa] -> [H] head grouping -- the paged_attention_v2_pytorch.py
 *   commit page, "KV gather" and the scores@V broadcast.
 *
 * How it is computed: the context is cut into partitions; one workgroup per
 * (sequence, KV head, partition) keeps an online-softmax state (running max,
 * denominator, weighted V) for all G query heads of the group, reading each
 * K/V page once; a second kernel merges the partition states by log-sum-exp
 * rescaling, (max, denominator) first and then the weighted outputs (the
 * commit page's "Phase 1: Per-partition attention" / "Phase 2: Cross-
 * partition reduction"; TVM PR #20426, section "Change", third bullet).  When
 * a single partition covers every context the merge is skipped and the
 * partial kernel writes out/lse itself (the host-side switch of TVM PR
 * #20426, section "Change": short contexts keep a single-pass kernel).
 *
 * Conventions for every entry point:
 *   - Returns PA_DECODE_OK (0) or a negative pa_decode_status.  No C++
 *     exception crosses the ABI.
 *   - All argument validation happens on the host before any HIP call.
 *   - Device pointers are caller-owned; the library keeps none of them after
 *     a call returns and never allocates device memory during pa_decode_run.
 *   - pa_decode_run is asynchronous on the caller's HIP stream: no host
 *     synchronisation, no allocation.  Calls on one handle from several host
 *     threads must be serialised by the caller.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    PA_DECODE_OK = 0,
    PA_DECODE_INVALID_ARG = -1,         /* null pointer, bad size, bad stride */
    PA_DECODE_UNSUPPORTED = -2,         /* head_dim / page_size / dtype / G not built */
    PA_DECODE_WORKSPACE_TOO_SMALL = -3, /* args.workspace_bytes below the plan's need */
    PA_DECODE_HIP_ERROR = -4,           /* a HIP call failed; see pa_decode_last_hip_error */
    PA_DECODE_EXCEEDS_SCRATCH = -5,     /* pa_decode_run_noalloc: the plan needs more than */
                                        /*   pa_decode_noalloc_scratch_bytes() of states   */
};

/* Bits of the device-side contract check (pa_decode_debug_status).  The
 * kernel never takes an address from a value that breaks the contract: it
 * clamps the value and, with desc.debug_checks, reports it. */
enum {
    PA_DECODE_VIOLATION_PAGE = 1,   /* a page id read is outside [0, num_pages): page 0 used */
    PA_DECODE_VIOLATION_LENGTH = 2, /* a context length is < 0 or > max_context_len: clamped */
    PA_DECODE_VIOLATION_ROW = 4,    /* CSR: indptr[b] < 0, indptr[b+1] < indptr[b] or */
                                    /*   > nnz_pages: the row is clamped into [0, nnz_pages] */
};

/* partition_size value that asks for the length-balanced schedule: the
 * visible pages of the whole batch (window start to last page of each
 * sequence, in sequence order) are split into equal contiguous ranges, one
 * per wave of each KV head, from the context lengths the kernel reads, so
 * that a few long sequences in a ragged batch do not set the step time.  A
 * wave's range is cut at sequence ends; each piece is one partition state,
 * and the merge combines a sequence's pieces.  This is the split-context
 * method of the paged_attention_v2 commit page (partition states merged by
 * log-sum-exp, "Phase 2") with partition bounds that follow the lengths
 * instead of fixed S-token blocks.  Needs batch <= 64 and
 * batch * (max_context_len / page_size + 66) < 2^31; UNSUPPORTED otherwise. */
#define PA_DECODE_PARTITION_BALANCED (-1)

/* Element types of q, the K/V caches and out (all three share one type). */
enum {
    PA_DTYPE_F32 = 0,
    PA_DTYPE_F16 = 1,
    PA_DTYPE_BF16 = 2,
};

/* Static problem description, fixed at pa_decode_create.
 * Supported: head_dim in {64, 96, 128, 256}; page_size 16; dtype in
 * {F32 (head_dim 64 only), F16, BF16}; G = num_q_heads / num_kv_heads an
 * integer in [1, 16]; rotary_mode 0 or 1 with any of these.  A zeroed tail
 * (rotary_mode 0) is the plain operation. */
typedef struct pa_decode_desc {
    int32_t num_q_heads;     /* Hq > 0 */
    int32_t num_kv_heads;    /* Hkv > 0, divides Hq, <= 65535 */
    int32_t head_dim;        /* D */
    int32_t page_size;       /* tokens per page */
    int32_t dtype;           /* PA_DTYPE_* of q, k/v cache and out */
    int32_t max_batch;       /* upper bound of args.batch, <= 65535 (UNSUPPORTED above) */
    int32_t max_context_len; /* upper bound of args.max_context_len */
    int32_t device;          /* HIP device ordinal the handle runs on (the handle */
                             /*   allocates 4 bytes there with debug_checks)    */
    int32_t rotary_mode;     /* 0: none; 1: rotary embedding of q and keys, applied */
                             /*   in the kernel as the keys are read (see above)   */
    float rope_theta;        /* rotary_mode 1: frequency base, finite and > 0     */
    float rope_scale;        /* rotary_mode 1: positions are divided by it, finite */
                             /*   and > 0 (1: no scaling)                           */
    int32_t debug_checks;    /* 1: keep a device status word that collects          */
                             /*   PA_DECODE_VIOLATION_* bits (pa_decode_debug_status); */
                             /*   0: values are clamped all the same, not reported   */
} pa_decode_desc;

/* Per-call arguments.  Element strides are in elements of the cache dtype.
 * q, k_cache, v_cache, out and (when the plan splits) workspace must be
 * 16-byte aligned, each stride times the element size a non-negative
 * multiple of 16 bytes, kv_stride_slot >= D, kv_stride_slot times the
 * element size below 2^27 bytes and num_pages * kv_stride_page times the
 * element size at most 2^50 bytes; otherwise pa_decode_run returns
 * PA_DECODE_INVALID_ARG (PA_DECODE_WORKSPACE_TOO_SMALL for a short
 * workspace) and launches nothing. */
typedef struct pa_decode_args {
    const void* q;              /* device, [batch, Hq, D] contiguous */
    const void* k_cache;        /* device, paged keys: element (page, kv, slot, d) at */
    const void* v_cache;        /*   page*kv_stride_page + kv*kv_stride_head +      */
                                /*   slot*kv_stride_slot + d (d contiguous);          */
                                /*   [num_pages, Hkv, page_size, D] contiguous is     */
                                /*   strides (Hkv*ps*D, ps*D, D); [num_pages, ps, Hkv, D] */
                                /*   works too.  K and V share the strides.           */
    int64_t kv_stride_page;
    int64_t kv_stride_head;
    int64_t kv_stride_slot;
    int32_t num_pages;          /* pages in the pool (page ids must be < num_pages) */
    const int32_t* page_table;  /* device, int32 [batch, pt_stride]; entry j of row b is */
                                /*   the page of tokens [j*ps, (j+1)*ps) of sequence b   */
    int32_t pt_stride;          /* row stride of page_table, >= ceil(max_context_len/ps) */
    const int32_t* context_lens;/* device, int32 [batch], 0 <= n_b <= max_context_len */
    int32_t batch;              /* B, 0 <= B <= desc.max_batch */
    int32_t max_context_len;    /* host upper bound of context_lens (used to plan) */
    float scale;                /* multiplies q.k */
    int32_t sliding_window;     /* <= 0: no window; else keys [n_b - W, n_b) */
    int32_t partition_size;     /* 0: planner's choice; else tokens per partition, */
                                /*   a positive multiple of page_size; or          */
                                /*   PA_DECODE_PARTITION_BALANCED                  */
    void* out;                  /* device, [batch, Hq, D] contiguous, desc.dtype */
    float* lse;                 /* device, float32 [batch, Hq], may be NULL */
    void* workspace;            /* device scratch of >= workspace_bytes needed by the */
    size_t workspace_bytes;     /*   plan (pa_decode_workspace_size); may be NULL/0   */
                                /*   when that size is 0.  Calls that share a         */
                                /*   workspace must not run concurrently.             */
} pa_decode_args;

/* The plan pa_decode_run derives from (batch, max_context_len, window,
 * partition_size) and the device's compute-unit count. */
typedef struct pa_decode_plan {
    int32_t split;              /* 1: partial kernel + merge kernel; 0: partial only */
    int32_t partition_size;     /* S, tokens per partition */
    int32_t num_partitions;     /* partitions per (sequence, KV head) */
    int32_t waves_per_group;    /* waves per workgroup of the partial kernel */
    int32_t waves_per_partition;/* waves of a workgroup sharing one partition; a   */
                                /*   workgroup covers waves_per_group /            */
                                /*   waves_per_partition consecutive partitions    */
    int32_t pages_per_block;    /* pages each wave holds in flight per step */
    int32_t grid_partial[3];    /* partial kernel grid (x = group of partitions,    */
                                /*   y = KV head, z = b)                            */
    int32_t block_partial;      /* threads per workgroup of the partial kernel */
    int32_t grid_merge[3];      /* merge kernel grid; 0s when split == 0.  Up to 64  */
                                /*   partitions: (ceil(waves / 4), 1, 1) with one wave  */
                                /*   per (b, query head, slice of 64 columns, or of 16  */
                                /*   when 64 would give fewer than 256 waves); beyond:  */
                                /*   (query head, b, head_dim / 16), one workgroup per  */
                                /*   16-column slice                                    */
    int32_t block_merge;        /* threads per merge workgroup (256) */
    int32_t num_cus;            /* compute units the plan was made for */
    int32_t waves_per_cu;       /* partial-kernel waves one compute unit holds     */
    int64_t workspace_bytes;    /* bytes of workspace the plan needs */
    int32_t balanced_waves;     /* > 0: the length-balanced schedule with this many */
                                /*   waves per KV head (grid x = balanced_waves /   */
                                /*   waves_per_group, y = KV head, z = 1); then      */
                                /*   partition_size is 0 and num_partitions is the  */
                                /*   most states one (sequence, head) can have.     */
                                /*   0: fixed partitions of partition_size tokens.  */
} pa_decode_plan;

typedef struct pa_decode_handle_s* pa_decode_handle;

/* Validate desc, read the device's properties and return a handle (with
 * desc.debug_checks = 1 it also allocates and zeroes the 4-byte status word
 * on desc.device).  The handle keeps what the host-side dispatch needs: the
 * compute-unit count and the partial kernel's occupancy, from which the
 * partition count is chosen per call (TVM PR #20426, section "Change": the
 * host picks the kernel and its split before the launch; section "Open for
 * reviewers": the split depends on the device), and the tuning overrides of
 * pa_decode_plan_query, read from the environment once, here.
 * Errors: INVALID_ARG (null pointer, non-positive sizes, Hq % Hkv != 0,
 * rotary_mode not 0 or 1, rope_theta or rope_scale not finite and > 0 with
 * rotary_mode 1), UNSUPPORTED (shape or dtype not built), HIP_ERROR (no such
 * device). */
int pa_decode_create(const pa_decode_desc* desc, pa_decode_handle* handle);

/* Release the handle (host memory only).  NULL is accepted. */
int pa_decode_destroy(pa_decode_handle handle);

/* Bytes of device workspace pa_decode_run needs for these sizes
 * (partition_size 0 = the planner's choice).  Pure host computation.  The
 * workspace holds the partition states the merge reads: per (sequence, query
 * head, partition) the normalised partial output, its maximum and its
 * denominator (the paged_attention_v2 commit page, "Phase 1: Per-partition
 * attention", stores the same three per partition), float32, laid out
 * o[B][Hq][P][D], m[B][Hq][P], l[B][Hq][P] (each region 256-byte aligned),
 * plus int32 state counts [B][Hq] under the length-balanced schedule.  0
 * when one partition covers every context (no merge). */
int pa_decode_workspace_size(pa_decode_handle handle, int32_t batch, int32_t max_context_len,
                             int32_t sliding_window, int32_t partition_size, size_t* bytes);

/* Run one decode step on `stream` (a hipStream_t; NULL = the null stream).
 * Errors: INVALID_ARG / UNSUPPORTED / WORKSPACE_TOO_SMALL from host checks,
 * HIP_ERROR when a launch fails.  Page ids, context lengths and page-table
 * rows live in device memory and are the caller's contract: every page id
 * read (rows b, entries [lo_b/ps, ceil(n_b/ps))) must be < num_pages and
 * n_b <= max_context_len.  Keys before lo_b and slots past n_b never reach
 * the result, so they may hold anything (NaN included); page-table entries
 * past ceil(n_b/ps) (within the row's pt_stride entries) may be read but are
 * never used to address K/V.  A run whose device-side values break the
 * contract reads no memory outside the caller's buffers (see
 * PA_DECODE_VIOLATION_*); its out/lse are then unspecified. */
int pa_decode_run(pa_decode_handle handle, const pa_decode_args* args, void* stream);

/* One decode step that allocates nothing, for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * plan, kernels and result as pa_decode_run, except that args->workspace and
 * args->workspace_bytes are ignored: the partition states go to a fixed
 * device array of pa_decode_noalloc_scratch_bytes() bytes (64 MiB) that the
 * library's code object holds on each GPU from its load until the process
 * ends.  Calls no allocating routine and never synchronises.
 * Limit: a plan whose workspace (pa_decode_workspace_size) exceeds that size
 * is rejected with PA_DECODE_EXCEEDS_SCRATCH before anything launches; plans
 * without a split need none.  Every handle on one GPU shares that GPU's
 * array, which keeps the last call's contents (nothing in it has to start
 * at zero: each call writes every state it reads): calls that can overlap on
 * one GPU (other streams, other threads, other handles) race and must be
 * serialised by the caller.  HIP_ERROR (pa_decode_last_hip_error) when the
 * array's address could not be found at pa_decode_create. */
int pa_decode_run_noalloc(pa_decode_handle handle, const pa_decode_args* args, void* stream);

/* Size in bytes of the fixed device scratch of pa_decode_run_noalloc. */
size_t pa_decode_noalloc_scratch_bytes(void);

/* Violation bits (PA_DECODE_VIOLATION_*) collected by the runs on this
 * handle since the previous call, then cleared.  Needs desc.debug_checks = 1
 * (else INVALID_ARG).  Synchronizes the device (hipDeviceSynchronize) before
 * it reads the word: a debugging aid, not for a timed loop. */
int pa_decode_debug_status(pa_decode_handle handle, int32_t* status);

/* The plan of the last successful pa_decode_run / pa_decode_run_csr on this
 * handle: the dispatch decision TVM PR #20426, section "Change", makes on the
 * host (single pass or split, and how), as it was taken.  INVALID_ARG before
 * the first run. */
int pa_decode_last_plan(pa_decode_handle handle, pa_decode_plan* plan);

/* Plan without a handle or device (pure host): the same planner that
 * pa_decode_run uses, for a given compute-unit count and number of
 * partial-kernel waves a compute unit holds at once (pa_decode_run uses the
 * device's values; the plan of a run reports them).
 * The split follows TVM PR #20426, section "Change" (a host-side choice
 * before the launch) and the commit page's split-context "Phase 1".
 * Tuning hooks for experiments: the environment variables
 * PA_DECODE_WAVES_PER_PARTITION and PA_DECODE_WAVES_PER_GROUP (1, 2 or 4)
 * override the plan's waves_per_partition / waves_per_group (the latter only
 * where it is a multiple of the former),
 * PA_DECODE_BALANCED_START (0 .. 64) the balanced schedule's start charge in
 * pages and PA_DECODE_BALANCED_WAVES_PER_CU (1 .. 16) its waves per compute
 * unit; other values are ignored.  This function reads them at each call, a
 * handle once at pa_decode_create.  They change the work split only, never
 * the result's definition or the workspace size. */
int pa_decode_plan_query(const pa_decode_desc* desc, int32_t num_cus, int32_t waves_per_cu,
                         int32_t batch, int32_t max_context_len, int32_t sliding_window,
                         int32_t partition_size, pa_decode_plan* plan);

/* ---------------------------------------------------------------------------
 * CSR page-table form.
 *
 * TVM PR #20426, section "Change", chooses between its single-pass kernel
 * and the sharded one on the host from the number of pages in use,
 * nnz_pages > B * 256 / page_size.  The page table that count belongs to is
 * a CSR (compressed-row) table: sequence b owns the pages
 *   page_indices[page_indptr[b]], ..., page_indices[page_indptr[b+1] - 1]
 * in token order, and the last of them holds last_page_len[b] tokens, so
 *   n_b = (page_indptr[b+1] - page_indptr[b] - 1) * page_size + last_page_len[b]
 * (n_b = 0 when the sequence owns no page; last_page_len is clamped to
 * [0, page_size]).  Everything else (the operation, windows, strides, out,
 * lse, workspace, ownership, errors) is as for pa_decode_args /
 * pa_decode_run: the same kernels run, only the page-id gather differs.
 * ------------------------------------------------------------------------- */
typedef struct pa_decode_csr_args {
    const void* q;                /* device, [batch, Hq, D] contiguous */
    const void* k_cache;          /* device, paged K/V as in pa_decode_args */
    const void* v_cache;
    int64_t kv_stride_page;
    int64_t kv_stride_head;
    int64_t kv_stride_slot;
    int32_t num_pages;            /* pages in the pool (page ids must be < num_pages) */
    const int32_t* page_indptr;   /* device, int32 [batch + 1], non-decreasing, [0] = 0 */
    const int32_t* page_indices;  /* device, int32 [nnz_pages] (NULL allowed when 0) */
    const int32_t* last_page_len; /* device, int32 [batch], 1..page_size for a      */
                                  /*   sequence that owns pages                      */
    int32_t nnz_pages;            /* host copy of page_indptr[batch] */
    int32_t batch;                /* B, 0 <= B <= desc.max_batch */
    int32_t max_context_len;      /* host upper bound of n_b; 0: nnz_pages * page_size */
    float scale;
    int32_t sliding_window;       /* <= 0: no window; else keys [n_b - W, n_b) */
    int32_t partition_size;       /* 0: the host switch above -- one partition per    */
                                  /*   (sequence, KV head) when nnz_pages <=          */
                                  /*   B * 256 / page_size; else, for 8 .. 64         */
                                  /*   sequences with 8 * nnz_pages < 5 * B *         */
                                  /*   ceil(max_context_len / page_size) (a ragged    */
                                  /*   batch: mean pages below 5/8 of the longest),   */
                                  /*   the length-balanced schedule; else the         */
                                  /*   planner's fixed split;                         */
                                  /*   > 0: tokens per partition, as in pa_decode_args; */
                                  /*   PA_DECODE_PARTITION_BALANCED as there          */
    void* out;                    /* device, [batch, Hq, D] contiguous, desc.dtype */
    float* lse;                   /* device, float32 [batch, Hq], may be NULL */
    void* workspace;              /* device scratch, pa_decode_workspace_size_csr bytes */
    size_t workspace_bytes;
} pa_decode_csr_args;

/* Workspace bytes pa_decode_run_csr needs (pure host). */
int pa_decode_workspace_size_csr(pa_decode_handle handle, int32_t batch, int32_t nnz_pages,
                                 int32_t max_context_len, int32_t sliding_window,
                                 int32_t partition_size, size_t* bytes);

/* One decode step from a CSR page table, on `stream`.  Errors as for
 * pa_decode_run; additionally INVALID_ARG when nnz_pages < 0, when
 * page_indptr / last_page_len are NULL with batch > 0, or when page_indices
 * is NULL with nnz_pages > 0.  Device-side contract: page_indptr and
 * last_page_len describe rows inside page_indices[0, nnz_pages), every page
 * id < num_pages, n_b <= max_context_len. */
int pa_decode_run_csr(pa_decode_handle handle, const pa_decode_csr_args* args, void* stream);

/* The plan pa_decode_run_csr makes for these sizes (pure host; as
 * pa_decode_plan_query, plus the host switch on nnz_pages). */
int pa_decode_plan_query_csr(const pa_decode_desc* desc, int32_t num_cus, int32_t waves_per_cu,
                             int32_t batch, int32_t nnz_pages, int32_t max_context_len,
                             int32_t sliding_window, int32_t partition_size,
                             pa_decode_plan* plan);

/* Kernel timing for measurement tools.  After pa_decode_profile_begin, the
 * next `max_launches` launches of each kernel (partial, merge) made by
 * pa_decode_run on this handle carry start/stop HIP events recorded on the
 * launch stream around the kernel itself.  pa_decode_profile_end waits for
 * those events, returns the summed kernel durations in milliseconds and the
 * launch counts (either output pointer may be NULL), and stops timing.
 * The events are created in pa_decode_profile_begin (host set-up, not in the
 * decode step).  Errors: INVALID_ARG (null handle, max_launches < 1),
 * HIP_ERROR (event creation or query failed). */
int pa_decode_profile_begin(pa_decode_handle handle, int32_t max_launches);
int pa_decode_profile_end(pa_decode_handle handle, double* partial_ms, int32_t* partial_launches,
                          double* merge_ms, int32_t* merge_launches);

/* Measurement tool (not part of the decode step): the memory system's read
 * rate for a set of KV chunks, e.g. the pages a decode step reads.  Reads
 * num_chunks chunks of chunk_bytes bytes each (2048, 3072, 4096 or 8192:
 * one KV head's slice of a page, 16 tokens x D x element size) on `stream`
 * (the current device), with the partial kernel's 16-byte streaming load,
 * in PA_DECODE_PROBE_WAVES waves (one per SIMD): wave w reads the chunks
 * [w n / W, (w + 1) n / W) of the list in order, keeping 15-16 KiB of loads
 * in flight from its start to its end.  Chunk i starts at chunk_addrs[i] (a
 * device array of device addresses, each 16-byte aligned, whole chunks
 * inside one allocation), or at base + i * chunk_bytes when chunk_addrs is
 * NULL (base 16-byte aligned).  sink (device, PA_DECODE_PROBE_WAVES 32-bit
 * words): word w is overwritten with the XOR of every 32-bit word wave w
 * read (0 for a wave without chunks), so the XOR of all the words is the
 * XOR of everything read; the data is used and a caller can check what
 * was read.  num_chunks = 0 launches nothing and leaves the sink as it is.  No atomics (a few hundred atomics on one word serialise into
 * microseconds).  Calls that share a sink must not overlap.  Asynchronous;
 * the caller times it.  Errors: INVALID_ARG (null sink, num_chunks < 0,
 * other chunk sizes, no base and no chunk_addrs, base misaligned),
 * HIP_ERROR (launch failed). */
#define PA_DECODE_PROBE_WAVES 1024
int pa_decode_read_probe(const void* base, const uint64_t* chunk_addrs, int32_t num_chunks,
                         int32_t chunk_bytes, uint32_t* sink, void* stream);

/* Last hipError_t recorded on the handle (0 when none). */
int pa_decode_last_hip_error(pa_decode_handle handle);

/* Static text for a status code. */
const char* pa_decode_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
