"""paged_kv_decode_amd: paged-KV GQA decode attention for AMD MI355X (gfx950).

The computation lives in libpa_decode.so (hand-written HIP kernels behind the
C ABI of include/pa_decode.h); ``binding`` is its ctypes front end and
``workloads`` draws seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    PA_DECODE_PARTITION_BALANCED,
    PA_DECODE_PROBE_WAVES,
    PagedDecode,
    PaDecodeArgs,
    PaDecodeDesc,
    PaDecodeError,
    PaDecodePlan,
    load_library,
    make_desc,
    pa_decode_create,
    pa_decode_debug_status,
    pa_decode_destroy,
    pa_decode_last_hip_error,
    pa_decode_last_plan,
    pa_decode_plan_query,
    pa_decode_profile_begin,
    pa_decode_profile_end,
    pa_decode_read_probe,
    pa_decode_run,
    pa_decode_status_string,
    pa_decode_workspace_size,
)
