// validate.cpp -- see validate.h.
#include "validate.h"

#include <cmath>

#include "planner.h"

namespace pa {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(const pa_decode_desc& d, const StepArgs& a)
{
    if (a.batch < 0 || a.batch > d.max_batch || a.max_context_len < 0 ||
        a.max_context_len > d.max_context_len ||
        (a.partition_size < 0 && a.partition_size != PA_DECODE_PARTITION_BALANCED))
        return PA_DECODE_INVALID_ARG;
    if (a.partition_size > 0 && a.partition_size % d.page_size != 0)
        return PA_DECODE_INVALID_ARG;
    if (!std::isfinite(a.scale))
        return PA_DECODE_INVALID_ARG;
    if (a.batch == 0)
        return PA_DECODE_OK;
    if (!a.q || !a.k_cache || !a.v_cache || !a.out || a.num_pages <= 0)
        return PA_DECODE_INVALID_ARG;
    const int eb = dtype_bytes(d.dtype);
    // Strides: non-negative, 16-byte granular (each lane reads 16-byte chunks),
    // and small enough that a byte offset cannot overflow int64.
    const int64_t strides[3] = {a.kv_stride_page, a.kv_stride_head, a.kv_stride_slot};
    for (int64_t s : strides)
        if (s < 0 || s > (int64_t(1) << 40) || (s * eb) % 16 != 0)
            return PA_DECODE_INVALID_ARG;
    if (a.kv_stride_slot < d.head_dim)
        return PA_DECODE_INVALID_ARG;
    // The kernel forms a lane's byte offset inside a page (up to 15 slot
    // strides) in 32 bits, and page * page stride in 64 bits.
    if (a.kv_stride_slot * eb >= (int64_t(1) << 27))
        return PA_DECODE_INVALID_ARG;
    if (a.kv_stride_page > ((int64_t(1) << 50) / eb) / a.num_pages)
        return PA_DECODE_INVALID_ARG;
    if (!aligned16(a.q) || !aligned16(a.k_cache) || !aligned16(a.v_cache) || !aligned16(a.out))
        return PA_DECODE_INVALID_ARG;
    return PA_DECODE_OK;
}

int check_args(const pa_decode_desc& d, const pa_decode_args& a)
{
    int st = check_common(d, common_args(a));
    if (st != PA_DECODE_OK || a.batch == 0)
        return st;
    if (!a.page_table || !a.context_lens || a.pt_stride <= 0)
        return PA_DECODE_INVALID_ARG;
    if (int64_t(a.pt_stride) * d.page_size < int64_t(a.max_context_len))
        return PA_DECODE_INVALID_ARG;
    return PA_DECODE_OK;
}

int check_csr_args(const pa_decode_desc& d, const pa_decode_csr_args& a)
{
    if (a.nnz_pages < 0 || (a.batch == 0 && a.nnz_pages != 0))
        return PA_DECODE_INVALID_ARG;
    int st = check_common(d, common_args(a));
    if (st != PA_DECODE_OK || a.batch == 0)
        return st;
    if (!a.page_indptr || !a.last_page_len || (a.nnz_pages > 0 && !a.page_indices))
        return PA_DECODE_INVALID_ARG;
    return PA_DECODE_OK;
}

}  // namespace pa
