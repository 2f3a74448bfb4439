// validate.h -- host-side argument checks of pa_decode_run / pa_decode_run_csr.
//
// Pure host C++ (no HIP call): every check runs before anything is launched,
// and the file builds on its own for the CPU sanitizer tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pa_decode.h"

namespace pa {

// The arguments both page-table forms share.
struct StepArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    int64_t kv_stride_page, kv_stride_head, kv_stride_slot;
    int32_t num_pages;
    int32_t batch;
    int32_t max_context_len;
    float scale;
    int32_t sliding_window;
    int32_t partition_size;
    void* out;
    float* lse;
    void* workspace;
    size_t workspace_bytes;
};

template <typename A>
StepArgs common_args(const A& a)
{
    StepArgs c;
    c.q = a.q;
    c.k_cache = a.k_cache;
    c.v_cache = a.v_cache;
    c.kv_stride_page = a.kv_stride_page;
    c.kv_stride_head = a.kv_stride_head;
    c.kv_stride_slot = a.kv_stride_slot;
    c.num_pages = a.num_pages;
    c.batch = a.batch;
    c.max_context_len = a.max_context_len;
    c.scale = a.scale;
    c.sliding_window = a.sliding_window;
    c.partition_size = a.partition_size;
    c.out = a.out;
    c.lse = a.lse;
    c.workspace = a.workspace;
    c.workspace_bytes = a.workspace_bytes;
    return c;
}

bool aligned16(const void* p);

// PA_DECODE_OK or INVALID_ARG for the shared arguments (sizes against the
// descriptor, the partition size, a finite scale, non-null 16-byte aligned
// tensors, 16-byte granular non-negative strides, a slot stride >= D).
int check_common(const pa_decode_desc& d, const StepArgs& a);
// ... plus the dense page table (non-null, pt_stride covering max_context_len).
int check_args(const pa_decode_desc& d, const pa_decode_args& a);
// ... plus the CSR arrays (nnz_pages >= 0, non-null pointers where needed).
int check_csr_args(const pa_decode_desc& d, const pa_decode_csr_args& a);

}  // namespace pa
