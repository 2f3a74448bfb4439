// pa_decode_api.cpp -- the C ABI declared in include/pa_decode.h.
//
// Host side of one decode step: validate the arguments (no HIP call before
// that), plan the partitioning for the device's compute units, launch the
// partial kernel and, when the context is split, the merge kernel, all on the
// caller's stream.  pa_decode_run / pa_decode_run_csr neither synchronise nor
// allocate; device memory is allocated only at create (the 4-byte status
// word, with desc.debug_checks), and only pa_decode_debug_status and
// pa_decode_profile_end wait for the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.h"
#include "pa_decode.h"
#include "planner.h"
#include "scratch.h"
#include "validate.h"

// Start/stop event pairs for kernel timing (see pa_decode_profile_begin).
struct EventRing {
    std::vector<hipEvent_t> start, stop;
    int used = 0;
    pa::LaunchEvents next()
    {
        pa::LaunchEvents ev;
        if (used < int(start.size())) {
            ev.start = start[used];
            ev.stop = stop[used];
            ++used;
        }
        return ev;
    }
    void release()
    {
        for (hipEvent_t e : start) (void)hipEventDestroy(e);
        for (hipEvent_t e : stop) (void)hipEventDestroy(e);
        start.clear();
        stop.clear();
        used = 0;
    }
};

// The plans of the last few call shapes (a decode loop repeats one shape, or
// a few), so that a run with a shape seen before does not plan again.
struct PlanCache {
    struct Entry {
        bool valid = false;
        bool csr = false;
        int32_t batch = 0, max_context_len = 0, sliding_window = 0, partition_size = 0,
                nnz_pages = 0;
        pa_decode_plan plan = {};
        int32_t max_ctx_used = 0;
    };
    static constexpr int kEntries = 4;
    Entry e[kEntries];
    int next = 0;
    const Entry* find(bool csr, int32_t batch, int32_t max_ctx, int32_t window, int32_t S,
                      int32_t nnz) const
    {
        for (const Entry& x : e)
            if (x.valid && x.csr == csr && x.batch == batch && x.max_context_len == max_ctx &&
                x.sliding_window == window && x.partition_size == S && x.nnz_pages == nnz)
                return &x;
        return nullptr;
    }
    void put(bool csr, int32_t batch, int32_t max_ctx, int32_t window, int32_t S, int32_t nnz,
             const pa_decode_plan& plan, int32_t max_ctx_used)
    {
        Entry& x = e[next];
        next = (next + 1) % kEntries;
        x.valid = true;
        x.csr = csr;
        x.batch = batch;
        x.max_context_len = max_ctx;
        x.sliding_window = window;
        x.partition_size = S;
        x.nnz_pages = nnz;
        x.plan = plan;
        x.max_ctx_used = max_ctx_used;
    }
};

struct pa_decode_handle_s {
    pa_decode_desc desc;
    int num_cus;
    int waves_per_cu;  // partial-kernel waves one compute unit holds at once
    pa::PlanTuning tune;  // read from the environment once, at create
    PlanCache plans;
    pa_decode_plan last_plan;
    bool has_plan;
    int last_hip_error;
    bool profiling;
    EventRing prof_partial, prof_merge;
    int32_t* status_word;  // device, with desc.debug_checks: violation bits
    void* scratch;         // desc.device's fixed scratch array (pa_decode_run_noalloc)
    int scratch_error;     // hipError_t of its address lookup at create (0: found)
};

namespace {

// Where the kernels find page ids and context lengths.
struct PageSource {
    const int32_t* page_table;    // dense rows, or CSR page indices
    int32_t pt_stride;
    const int32_t* context_lens;
    const int32_t* page_indptr;   // null for the dense form
    const int32_t* last_page_len;
    int32_t nnz_pages;            // CSR: entries of page_indices
};

// Launches one planned decode step on `stream` (arguments already checked).
int launch_step(pa_decode_handle handle, const pa::StepArgs& a, const PageSource& src,
                const pa_decode_plan& plan, void* stream)
{
    const pa_decode_desc& d = handle->desc;
    if (plan.split && (!a.workspace || a.workspace_bytes < size_t(plan.workspace_bytes)))
        return PA_DECODE_WORKSPACE_TOO_SMALL;
    if (plan.split && !pa::aligned16(a.workspace))
        return PA_DECODE_INVALID_ARG;
    handle->last_plan = plan;
    handle->has_plan = true;
    if (a.batch == 0)
        return PA_DECODE_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int G = d.num_q_heads / d.num_kv_heads;
    const bool balanced = plan.balanced_waves > 0;
    const pa::WorkspaceLayout wl =
        pa::workspace_layout(d, a.batch, plan.num_partitions, balanced);
    char* ws = static_cast<char*>(a.workspace);

    pa::PartialParams pp;
    pp.q = a.q;
    pp.k = a.k_cache;
    pp.v = a.v_cache;
    pp.stride_page = a.kv_stride_page;
    pp.stride_head = a.kv_stride_head;
    pp.stride_slot = a.kv_stride_slot;
    pp.page_table = src.page_table;
    pp.pt_stride = src.pt_stride;
    pp.context_lens = src.context_lens;
    pp.page_indptr = src.page_indptr;
    pp.last_page_len = src.last_page_len;
    pp.num_q_heads = d.num_q_heads;
    pp.group = G;
    pp.partition_size = plan.partition_size;
    pp.num_partitions = plan.num_partitions;
    pp.waves_per_partition = plan.waves_per_partition;
    pp.window = a.sliding_window;
    pp.scale_log2 = float(double(a.scale) * 1.4426950408889634);
    pp.split = plan.split;
    pp.ws_o = plan.split ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
    pp.ws_m = plan.split ? reinterpret_cast<float*>(ws + wl.m_off) : nullptr;
    pp.ws_l = plan.split ? reinterpret_cast<float*>(ws + wl.l_off) : nullptr;
    pp.out = a.out;
    pp.lse = a.lse;
    pp.num_pages = a.num_pages;
    pp.max_context_len = a.max_context_len;
    pp.nnz_pages = src.nnz_pages;
    pp.status = handle->status_word;
    pp.rotary = d.rotary_mode;
    // theta_i = rope_theta^(-2i/D) / rope_scale = rope_rho^i / rope_scale
    pp.rope_rho = d.rotary_mode ? std::pow(double(d.rope_theta), -2.0 / d.head_dim) : 1.0;
    pp.rope_f0 = d.rotary_mode ? 1.0 / (6.283185307179586477 * double(d.rope_scale)) : 0.0;
    pp.minus_one = -1.0f;
    pp.batch = a.batch;
    pp.bal_waves = plan.balanced_waves;
    pp.bal_start = balanced ? pa::balanced_start_pages(d, handle->tune) : 0;
    pp.ws_cnt = balanced ? reinterpret_cast<int32_t*>(ws + wl.c_off) : nullptr;
#if PA_FUSED_MERGE
    if (!balanced && plan.split)
        pp.ws_cnt = reinterpret_cast<int32_t*>(ws + wl.c_off);   // merge counters (zero between calls)
#endif

    const dim3 grid(plan.grid_partial[0], plan.grid_partial[1], plan.grid_partial[2]);
    const dim3 block(plan.block_partial);
    const pa::LaunchEvents ev_partial =
        handle->profiling ? handle->prof_partial.next() : pa::LaunchEvents();
    const size_t lds = pa::partial_lds_bytes(d, plan);
    hipError_t e =
        balanced ? pa::launch_partial_balanced(d.dtype, d.head_dim, pa::template_group(G), pp,
                                               grid, block, lds, s, ev_partial)
                 : pa::launch_partial(d.dtype, d.head_dim, pa::template_group(G), pp, grid,
                                      block, lds, s, ev_partial);
    if (e != hipSuccess) {
        handle->last_hip_error = int(e);
        return PA_DECODE_HIP_ERROR;
    }
#if PA_FUSED_MERGE
    const bool merge_kernel = plan.split && balanced;
#else
    const bool merge_kernel = plan.split;
#endif
    if (merge_kernel) {
        pa::MergeParams mp;
        mp.batch = a.batch;
        mp.num_q_heads = d.num_q_heads;
        mp.num_partitions = plan.num_partitions;
        mp.ws_o = pp.ws_o;
        mp.ws_m = pp.ws_m;
        mp.ws_l = pp.ws_l;
        mp.out = a.out;
        mp.lse = a.lse;
        mp.ws_cnt = pp.ws_cnt;
        const dim3 mgrid(plan.grid_merge[0], plan.grid_merge[1], plan.grid_merge[2]);
        const pa::LaunchEvents ev_merge =
            handle->profiling ? handle->prof_merge.next() : pa::LaunchEvents();
        e = pa::launch_merge(d.dtype, d.head_dim, mp, mgrid, dim3(plan.block_merge), s, ev_merge);
        if (e != hipSuccess) {
            handle->last_hip_error = int(e);
            return PA_DECODE_HIP_ERROR;
        }
    }
    return PA_DECODE_OK;
}

// The plan of a dense-table call (cached per call shape).
int plan_dense(pa_decode_handle h, int32_t batch, int32_t max_ctx, int32_t window, int32_t S,
               pa_decode_plan* plan)
{
    if (const PlanCache::Entry* x = h->plans.find(false, batch, max_ctx, window, S, 0)) {
        *plan = x->plan;
        return PA_DECODE_OK;
    }
    const int st = pa::make_plan(h->desc, h->num_cus, h->waves_per_cu, h->tune, batch, max_ctx,
                                 window, S, plan);
    if (st == PA_DECODE_OK)
        h->plans.put(false, batch, max_ctx, window, S, 0, *plan, max_ctx);
    return st;
}

// The plan of a CSR call and the context bound it used (cached per call shape).
int plan_csr(pa_decode_handle h, int32_t batch, int32_t nnz, int32_t max_ctx, int32_t window,
             int32_t S, pa_decode_plan* plan, int* max_ctx_used)
{
    if (const PlanCache::Entry* x = h->plans.find(true, batch, max_ctx, window, S, nnz)) {
        *plan = x->plan;
        if (max_ctx_used) *max_ctx_used = x->max_ctx_used;
        return PA_DECODE_OK;
    }
    int used = 0;
    const int st = pa::make_plan_csr(h->desc, h->num_cus, h->waves_per_cu, h->tune, batch, nnz,
                                     max_ctx, window, S, plan, &used);
    if (st == PA_DECODE_OK)
        h->plans.put(true, batch, max_ctx, window, S, nnz, *plan, used);
    if (max_ctx_used) *max_ctx_used = used;
    return st;
}

}  // namespace

extern "C" {

int pa_decode_create(const pa_decode_desc* desc, pa_decode_handle* handle)
{
    if (!desc || !handle)
        return PA_DECODE_INVALID_ARG;
    *handle = nullptr;
    int st = pa::check_desc(*desc);
    if (st != PA_DECODE_OK)
        return st;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || desc->device >= count)
        return PA_DECODE_HIP_ERROR;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, desc->device) !=
            hipSuccess ||
        cus <= 0)
        return PA_DECODE_HIP_ERROR;
    auto* h = new (std::nothrow) pa_decode_handle_s();
    if (!h)
        return PA_DECODE_HIP_ERROR;
    h->desc = *desc;
    h->num_cus = cus;
    h->tune = pa::tuning_from_env();
    {
        // Occupancy of the partial kernel this description uses, for the
        // largest workgroup the planner gives it.
        pa_decode_plan probe = {};
        probe.waves_per_group = pa::workgroup_waves(*desc);
        probe.pages_per_block = pa::pages_per_block(desc->head_dim, desc->dtype);
        const int G = desc->num_q_heads / desc->num_kv_heads;
        int w = pa::partial_waves_per_cu(desc->dtype, desc->head_dim, pa::template_group(G),
                                         desc->rotary_mode == 1, probe.waves_per_group,
                                         pa::partial_lds_bytes(*desc, probe));
        h->waves_per_cu = w > 0 ? w : 8;
    }
    h->has_plan = false;
    h->last_hip_error = 0;
    h->profiling = false;
    h->status_word = nullptr;
    // The device address of the fixed scratch array, looked up once per
    // device (the lookup makes desc.device current and restores the caller's
    // device).  A failure only disables pa_decode_run_noalloc on this handle.
    h->scratch = nullptr;
    h->scratch_error = int(pa::scratch_address(desc->device, &h->scratch));
    if (desc->debug_checks) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e == hipSuccess) e = hipSetDevice(desc->device);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&h->status_word), sizeof(int32_t));
        if (e == hipSuccess) e = hipMemset(h->status_word, 0, sizeof(int32_t));
        if (prev >= 0) (void)hipSetDevice(prev);
        if (e != hipSuccess) {
            if (h->status_word) (void)hipFree(h->status_word);
            delete h;
            return PA_DECODE_HIP_ERROR;
        }
    }
    *handle = h;
    return PA_DECODE_OK;
}

int pa_decode_destroy(pa_decode_handle handle)
{
    if (handle) {
        handle->prof_partial.release();
        handle->prof_merge.release();
        if (handle->status_word) (void)hipFree(handle->status_word);
    }
    delete handle;
    return PA_DECODE_OK;
}

int pa_decode_profile_begin(pa_decode_handle handle, int32_t max_launches)
{
    if (!handle || max_launches < 1)
        return PA_DECODE_INVALID_ARG;
    handle->prof_partial.release();
    handle->prof_merge.release();
    for (EventRing* r : {&handle->prof_partial, &handle->prof_merge}) {
        for (int i = 0; i < max_launches; ++i) {
            hipEvent_t a = nullptr, b = nullptr;
            hipError_t e = hipEventCreate(&a);
            if (e == hipSuccess) e = hipEventCreate(&b);
            if (e != hipSuccess) {
                if (a) (void)hipEventDestroy(a);
                r->release();
                handle->last_hip_error = int(e);
                return PA_DECODE_HIP_ERROR;
            }
            r->start.push_back(a);
            r->stop.push_back(b);
        }
    }
    handle->profiling = true;
    return PA_DECODE_OK;
}

int pa_decode_profile_end(pa_decode_handle handle, double* partial_ms, int32_t* partial_launches,
                          double* merge_ms, int32_t* merge_launches)
{
    if (!handle)
        return PA_DECODE_INVALID_ARG;
    handle->profiling = false;
    double sums[2] = {0.0, 0.0};
    int counts[2] = {handle->prof_partial.used, handle->prof_merge.used};
    EventRing* rings[2] = {&handle->prof_partial, &handle->prof_merge};
    for (int k = 0; k < 2; ++k) {
        for (int i = 0; i < counts[k]; ++i) {
            hipError_t e = hipEventSynchronize(rings[k]->stop[i]);
            float ms = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, rings[k]->start[i], rings[k]->stop[i]);
            if (e != hipSuccess) {
                handle->last_hip_error = int(e);
                rings[0]->release();
                rings[1]->release();
                return PA_DECODE_HIP_ERROR;
            }
            sums[k] += ms;
        }
    }
    rings[0]->release();
    rings[1]->release();
    if (partial_ms) *partial_ms = sums[0];
    if (partial_launches) *partial_launches = counts[0];
    if (merge_ms) *merge_ms = sums[1];
    if (merge_launches) *merge_launches = counts[1];
    return PA_DECODE_OK;
}

int pa_decode_workspace_size(pa_decode_handle handle, int32_t batch, int32_t max_context_len,
                             int32_t sliding_window, int32_t partition_size, size_t* bytes)
{
    if (!handle || !bytes)
        return PA_DECODE_INVALID_ARG;
    pa_decode_plan plan;
    int st = plan_dense(handle, batch, max_context_len, sliding_window, partition_size, &plan);
    if (st != PA_DECODE_OK)
        return st;
    *bytes = size_t(plan.workspace_bytes);
    return PA_DECODE_OK;
}

int pa_decode_plan_query(const pa_decode_desc* desc, int32_t num_cus, int32_t waves_per_cu,
                         int32_t batch, int32_t max_context_len, int32_t sliding_window,
                         int32_t partition_size, pa_decode_plan* plan)
{
    if (!desc || !plan)
        return PA_DECODE_INVALID_ARG;
    return pa::make_plan(*desc, num_cus, waves_per_cu, pa::tuning_from_env(), batch,
                         max_context_len, sliding_window, partition_size, plan);
}

int pa_decode_run(pa_decode_handle handle, const pa_decode_args* args, void* stream)
{
    if (!handle || !args)
        return PA_DECODE_INVALID_ARG;
    const pa_decode_desc& d = handle->desc;
    const pa_decode_args& a = *args;
    int st = pa::check_args(d, a);
    if (st != PA_DECODE_OK)
        return st;
    pa_decode_plan plan;
    st = plan_dense(handle, a.batch, a.max_context_len, a.sliding_window, a.partition_size, &plan);
    if (st != PA_DECODE_OK)
        return st;
    PageSource src = {a.page_table, a.pt_stride, a.context_lens, nullptr, nullptr, 0};
    return launch_step(handle, pa::common_args(a), src, plan, stream);
}

int pa_decode_run_noalloc(pa_decode_handle handle, const pa_decode_args* args, void* stream)
{
    if (!handle || !args)
        return PA_DECODE_INVALID_ARG;
    const pa_decode_desc& d = handle->desc;
    const pa_decode_args& a = *args;
    int st = pa::check_args(d, a);
    if (st != PA_DECODE_OK)
        return st;
    pa_decode_plan plan;
    st = plan_dense(handle, a.batch, a.max_context_len, a.sliding_window, a.partition_size, &plan);
    if (st != PA_DECODE_OK)
        return st;
    if (plan.workspace_bytes > int64_t(pa::kScratchBytes))
        return PA_DECODE_EXCEEDS_SCRATCH;
    if (!handle->scratch) {
        handle->last_hip_error = handle->scratch_error;
        return PA_DECODE_HIP_ERROR;
    }
    pa::StepArgs c = pa::common_args(a);
    c.workspace = handle->scratch;   // the device address, never the array's host-side name
    c.workspace_bytes = pa::kScratchBytes;
    PageSource src = {a.page_table, a.pt_stride, a.context_lens, nullptr, nullptr, 0};
    return launch_step(handle, c, src, plan, stream);
}

size_t pa_decode_noalloc_scratch_bytes(void) { return pa::kScratchBytes; }

int pa_decode_workspace_size_csr(pa_decode_handle handle, int32_t batch, int32_t nnz_pages,
                                 int32_t max_context_len, int32_t sliding_window,
                                 int32_t partition_size, size_t* bytes)
{
    if (!handle || !bytes)
        return PA_DECODE_INVALID_ARG;
    pa_decode_plan plan;
    int st = plan_csr(handle, batch, nnz_pages, max_context_len, sliding_window, partition_size,
                      &plan, nullptr);
    if (st != PA_DECODE_OK)
        return st;
    *bytes = size_t(plan.workspace_bytes);
    return PA_DECODE_OK;
}

int pa_decode_plan_query_csr(const pa_decode_desc* desc, int32_t num_cus, int32_t waves_per_cu,
                             int32_t batch, int32_t nnz_pages, int32_t max_context_len,
                             int32_t sliding_window, int32_t partition_size,
                             pa_decode_plan* plan)
{
    if (!desc || !plan)
        return PA_DECODE_INVALID_ARG;
    return pa::make_plan_csr(*desc, num_cus, waves_per_cu, pa::tuning_from_env(), batch,
                             nnz_pages, max_context_len, sliding_window, partition_size, plan,
                             nullptr);
}

int pa_decode_run_csr(pa_decode_handle handle, const pa_decode_csr_args* args, void* stream)
{
    if (!handle || !args)
        return PA_DECODE_INVALID_ARG;
    const pa_decode_desc& d = handle->desc;
    const pa_decode_csr_args& a = *args;
    int st = pa::check_csr_args(d, a);
    if (st != PA_DECODE_OK)
        return st;
    pa_decode_plan plan;
    int max_ctx = 0;
    st = plan_csr(handle, a.batch, a.nnz_pages, a.max_context_len, a.sliding_window,
                  a.partition_size, &plan, &max_ctx);
    if (st != PA_DECODE_OK)
        return st;
    pa::StepArgs c = pa::common_args(a);
    c.max_context_len = max_ctx;
    PageSource src = {a.page_indices, 0, nullptr, a.page_indptr, a.last_page_len, a.nnz_pages};
    return launch_step(handle, c, src, plan, stream);
}

int pa_decode_read_probe(const void* base, const uint64_t* chunk_addrs, int32_t num_chunks,
                         int32_t chunk_bytes, uint32_t* sink, void* stream)
{
    if (!sink || num_chunks < 0 || (!base && !chunk_addrs && num_chunks > 0))
        return PA_DECODE_INVALID_ARG;
    if (chunk_bytes != 2048 && chunk_bytes != 3072 && chunk_bytes != 4096 && chunk_bytes != 8192)
        return PA_DECODE_INVALID_ARG;
    if (base && !pa::aligned16(base))
        return PA_DECODE_INVALID_ARG;
    const hipError_t e = pa::launch_read_probe(base, chunk_addrs, num_chunks, chunk_bytes / 1024,
                                               sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_DECODE_OK : PA_DECODE_HIP_ERROR;
}

int pa_decode_debug_status(pa_decode_handle handle, int32_t* status)
{
    if (!handle || !status || !handle->status_word)
        return PA_DECODE_INVALID_ARG;
    int32_t v = 0;
    const int32_t zero = 0;
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess) e = hipSetDevice(handle->desc.device);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(&v, handle->status_word, sizeof v, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(handle->status_word, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        handle->last_hip_error = int(e);
        return PA_DECODE_HIP_ERROR;
    }
    *status = v;
    return PA_DECODE_OK;
}

int pa_decode_last_plan(pa_decode_handle handle, pa_decode_plan* plan)
{
    if (!handle || !plan || !handle->has_plan)
        return PA_DECODE_INVALID_ARG;
    *plan = handle->last_plan;
    return PA_DECODE_OK;
}

int pa_decode_last_hip_error(pa_decode_handle handle)
{
    return handle ? handle->last_hip_error : 0;
}

const char* pa_decode_status_string(int status)
{
    switch (status) {
    case PA_DECODE_OK: return "ok";
    case PA_DECODE_INVALID_ARG: return "invalid argument";
    case PA_DECODE_UNSUPPORTED: return "unsupported configuration";
    case PA_DECODE_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_DECODE_HIP_ERROR: return "HIP error";
    case PA_DECODE_EXCEEDS_SCRATCH:
        return "the plan's partition states exceed the fixed device scratch of "
               "pa_decode_run_noalloc";
    default: return "unknown status";
    }
}

}  // extern "C"
