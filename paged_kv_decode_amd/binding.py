"""Thin ctypes binding of libpa_decode.so (include/pa_decode.h).

The functions carry the C names and only marshal arguments; every step of the
decode-attention computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams only (``PagedDecode`` allocates out, lse
and the workspace with torch and passes raw pointers).  There is no fallback:
if the library is missing or fails, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch  # loaded first so the library binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_decode.so")

PA_DECODE_OK = 0
PA_DECODE_INVALID_ARG = -1
PA_DECODE_UNSUPPORTED = -2
PA_DECODE_WORKSPACE_TOO_SMALL = -3
PA_DECODE_HIP_ERROR = -4
PA_DECODE_EXCEEDS_SCRATCH = -5

# partition_size value for the length-balanced schedule (batch <= 64).
PA_DECODE_PARTITION_BALANCED = -1
# Words of the read probe's sink (one per probe wave).
PA_DECODE_PROBE_WAVES = 1024

PA_DTYPE_F32 = 0
PA_DTYPE_F16 = 1
PA_DTYPE_BF16 = 2

DTYPE_CODE = {torch.float32: PA_DTYPE_F32, torch.float16: PA_DTYPE_F16,
              torch.bfloat16: PA_DTYPE_BF16}

# Symbols include/pa_decode.h declares.
EXPORTED = ["pa_decode_create", "pa_decode_destroy", "pa_decode_workspace_size",
            "pa_decode_run", "pa_decode_last_plan", "pa_decode_plan_query",
            "pa_decode_profile_begin", "pa_decode_profile_end",
            "pa_decode_last_hip_error", "pa_decode_status_string",
            "pa_decode_workspace_size_csr", "pa_decode_run_csr", "pa_decode_plan_query_csr",
            "pa_decode_debug_status", "pa_decode_read_probe", "pa_decode_run_noalloc",
            "pa_decode_noalloc_scratch_bytes"]


class PaDecodeDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("device", ctypes.c_int32),
                ("rotary_mode", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rope_scale", ctypes.c_float), ("debug_checks", ctypes.c_int32)]


class PaDecodeArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("kv_stride_page", ctypes.c_int64),
                ("kv_stride_head", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int32), ("context_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("scale", ctypes.c_float), ("sliding_window", ctypes.c_int32),
                ("partition_size", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class PaDecodeCsrArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("kv_stride_page", ctypes.c_int64),
                ("kv_stride_head", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("page_indptr", ctypes.c_void_p),
                ("page_indices", ctypes.c_void_p), ("last_page_len", ctypes.c_void_p),
                ("nnz_pages", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("scale", ctypes.c_float),
                ("sliding_window", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class PaDecodePlan(ctypes.Structure):
    _fields_ = [("split", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("num_partitions", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("waves_per_partition", ctypes.c_int32), ("pages_per_block", ctypes.c_int32), ("grid_partial", ctypes.c_int32 * 3),
                ("block_partial", ctypes.c_int32), ("grid_merge", ctypes.c_int32 * 3),
                ("block_merge", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("waves_per_cu", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("balanced_waves", ctypes.c_int32)]

    def as_dict(self):
        return {"split": self.split, "partition_size": self.partition_size,
                "num_partitions": self.num_partitions, "waves_per_group": self.waves_per_group,
                "waves_per_partition": self.waves_per_partition,
                "pages_per_block": self.pages_per_block,
                "grid_partial": list(self.grid_partial), "block_partial": self.block_partial,
                "grid_merge": list(self.grid_merge), "block_merge": self.block_merge,
                "num_cus": self.num_cus, "waves_per_cu": self.waves_per_cu,
                "workspace_bytes": self.workspace_bytes, "balanced_waves": self.balanced_waves}


class PaDecodeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, pa_decode_status_string(status), status))


_lib = None
_lock = threading.Lock()


def load_library(path: Optional[str] = None):
    """Load libpa_decode.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libpa_decode.so is not built (%s); run "
                               "`python -m paged_kv_decode_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.pa_decode_create.argtypes = [ctypes.POINTER(PaDecodeDesc), ctypes.POINTER(vp)]
        lib.pa_decode_destroy.argtypes = [vp]
        lib.pa_decode_workspace_size.argtypes = [vp, i32, i32, i32, i32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
        lib.pa_decode_run.argtypes = [vp, ctypes.POINTER(PaDecodeArgs), vp]
        lib.pa_decode_last_plan.argtypes = [vp, ctypes.POINTER(PaDecodePlan)]
        lib.pa_decode_plan_query.argtypes = [ctypes.POINTER(PaDecodeDesc), i32, i32, i32, i32,
                                             i32, i32, ctypes.POINTER(PaDecodePlan)]
        lib.pa_decode_profile_begin.argtypes = [vp, i32]
        lib.pa_decode_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(i32)]
        lib.pa_decode_workspace_size_csr.argtypes = [vp, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(ctypes.c_size_t)]
        lib.pa_decode_run_csr.argtypes = [vp, ctypes.POINTER(PaDecodeCsrArgs), vp]
        lib.pa_decode_plan_query_csr.argtypes = [ctypes.POINTER(PaDecodeDesc), i32, i32, i32,
                                                 i32, i32, i32, i32,
                                                 ctypes.POINTER(PaDecodePlan)]
        lib.pa_decode_last_hip_error.argtypes = [vp]
        lib.pa_decode_debug_status.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
        lib.pa_decode_read_probe.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.pa_decode_run_noalloc.argtypes = [vp, ctypes.POINTER(PaDecodeArgs), vp]
        lib.pa_decode_noalloc_scratch_bytes.argtypes = []
        lib.pa_decode_status_string.argtypes = [ctypes.c_int]
        lib.pa_decode_status_string.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "pa_decode_status_string":
                getattr(lib, name).restype = ctypes.c_int
        lib.pa_decode_noalloc_scratch_bytes.restype = ctypes.c_size_t
        if path is None:
            _lib = lib
        return lib


def use_library(path: str):
    """Load the library at `path` (a comparison build, for measurement) and
    make it the one every call of this module uses."""
    global _lib
    lib = load_library(path)
    with _lock:
        _lib = lib
    return lib


def _check(status: int, what: str):
    if status != PA_DECODE_OK:
        raise PaDecodeError(status, what)


def pa_decode_workspace_size_csr(handle, batch: int, nnz_pages: int, max_context_len: int = 0,
                                 sliding_window: int = 0, partition_size: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(load_library().pa_decode_workspace_size_csr(handle, batch, nnz_pages, max_context_len,
                                                       sliding_window, partition_size,
                                                       ctypes.byref(n)),
           "pa_decode_workspace_size_csr")
    return int(n.value)


def pa_decode_run_csr(handle, args: PaDecodeCsrArgs, stream: int = 0) -> None:
    _check(load_library().pa_decode_run_csr(handle, ctypes.byref(args), ctypes.c_void_p(stream)),
           "pa_decode_run_csr")


def pa_decode_plan_query_csr(desc: PaDecodeDesc, num_cus: int, waves_per_cu: int, batch: int,
                             nnz_pages: int, max_context_len: int = 0, sliding_window: int = 0,
                             partition_size: int = 0) -> PaDecodePlan:
    plan = PaDecodePlan()
    _check(load_library().pa_decode_plan_query_csr(ctypes.byref(desc), num_cus, waves_per_cu,
                                                   batch, nnz_pages, max_context_len,
                                                   sliding_window, partition_size,
                                                   ctypes.byref(plan)),
           "pa_decode_plan_query_csr")
    return plan


def pa_decode_status_string(status: int) -> str:
    return load_library().pa_decode_status_string(int(status)).decode()


def pa_decode_create(desc: PaDecodeDesc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().pa_decode_create(ctypes.byref(desc), ctypes.byref(h)),
           "pa_decode_create")
    return h


def pa_decode_destroy(handle) -> None:
    _check(load_library().pa_decode_destroy(handle), "pa_decode_destroy")


def pa_decode_workspace_size(handle, batch: int, max_context_len: int, sliding_window: int = 0,
                             partition_size: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(load_library().pa_decode_workspace_size(handle, batch, max_context_len,
                                                   sliding_window, partition_size,
                                                   ctypes.byref(n)),
           "pa_decode_workspace_size")
    return int(n.value)


def pa_decode_run(handle, args: PaDecodeArgs, stream: int = 0) -> None:
    _check(load_library().pa_decode_run(handle, ctypes.byref(args), ctypes.c_void_p(stream)),
           "pa_decode_run")


def pa_decode_run_noalloc(handle, args: PaDecodeArgs, stream: int = 0) -> None:
    """pa_decode_run with the partition states in the library's fixed device
    scratch (args.workspace is ignored); allocates nothing."""
    _check(load_library().pa_decode_run_noalloc(handle, ctypes.byref(args),
                                                ctypes.c_void_p(stream)),
           "pa_decode_run_noalloc")


def pa_decode_noalloc_scratch_bytes() -> int:
    return int(load_library().pa_decode_noalloc_scratch_bytes())


def pa_decode_last_plan(handle) -> PaDecodePlan:
    plan = PaDecodePlan()
    _check(load_library().pa_decode_last_plan(handle, ctypes.byref(plan)), "pa_decode_last_plan")
    return plan


def pa_decode_plan_query(desc: PaDecodeDesc, num_cus: int, waves_per_cu: int, batch: int,
                         max_context_len: int, sliding_window: int = 0,
                         partition_size: int = 0) -> PaDecodePlan:
    plan = PaDecodePlan()
    _check(load_library().pa_decode_plan_query(ctypes.byref(desc), num_cus, waves_per_cu, batch,
                                               max_context_len, sliding_window, partition_size,
                                               ctypes.byref(plan)),
           "pa_decode_plan_query")
    return plan


def pa_decode_profile_begin(handle, max_launches: int) -> None:
    _check(load_library().pa_decode_profile_begin(handle, max_launches), "pa_decode_profile_begin")


def pa_decode_profile_end(handle):
    """Returns (partial_ms_total, partial_launches, merge_ms_total, merge_launches)."""
    pm, mm = ctypes.c_double(), ctypes.c_double()
    pn, mn = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().pa_decode_profile_end(handle, ctypes.byref(pm), ctypes.byref(pn),
                                                ctypes.byref(mm), ctypes.byref(mn)),
           "pa_decode_profile_end")
    return pm.value, pn.value, mm.value, mn.value


def pa_decode_last_hip_error(handle) -> int:
    return int(load_library().pa_decode_last_hip_error(handle))


# Violation bits of pa_decode_debug_status (include/pa_decode.h).
PA_DECODE_VIOLATION_PAGE = 1
PA_DECODE_VIOLATION_LENGTH = 2
PA_DECODE_VIOLATION_ROW = 4


def pa_decode_debug_status(handle) -> int:
    """Violation bits collected since the last call (synchronizes the device)."""
    v = ctypes.c_int32()
    _check(load_library().pa_decode_debug_status(handle, ctypes.byref(v)),
           "pa_decode_debug_status")
    return int(v.value)


def pa_decode_read_probe(base: int, chunk_addrs: int, num_chunks: int, chunk_bytes: int,
                         sink: int, stream: int = 0) -> None:
    """Measurement tool: read num_chunks chunks (device addresses in the
    uint64 device array at chunk_addrs, or contiguous from base when
    chunk_addrs is 0) on `stream`.  sink: a device array of
    PA_DECODE_PROBE_WAVES uint32 words, each overwritten with the XOR of the
    words one probe wave read (their XOR is that of everything read)."""
    _check(load_library().pa_decode_read_probe(base or None, chunk_addrs or None, num_chunks,
                                               chunk_bytes, sink or None, stream or None),
           "pa_decode_read_probe")


def make_desc(num_q_heads, num_kv_heads, head_dim, dtype, max_batch, max_context_len,
              page_size=16, device=0, rope=None, rotary_mode=None,
              debug_checks=0) -> PaDecodeDesc:
    """rope: None (rotary_mode 0) or (rope_theta, rope_scale) for rotary_mode 1;
    rotary_mode overrides the mode (to pass invalid values through in tests);
    debug_checks: 1 keeps the device status word (pa_decode_debug_status)."""
    code = DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    mode = (0 if rope is None else 1) if rotary_mode is None else int(rotary_mode)
    theta, rscale = (0.0, 0.0) if rope is None else (float(rope[0]), float(rope[1]))
    return PaDecodeDesc(num_q_heads, num_kv_heads, head_dim, page_size, code, max_batch,
                        max_context_len, device, mode, theta, rscale, int(debug_checks))



def _storage_elems(t: torch.Tensor) -> int:
    """Elements of t's storage from t's first element on."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _check_step_shapes(desc: PaDecodeDesc, dtype, q, k_cache, v_cache, out, lse):
    """Shapes the C ABI cannot see (it takes raw pointers): q and out
    [B, Hq, D], caches [num_pages, Hkv, page_size, D] with D contiguous, lse
    [B, Hq].  Raises TypeError / ValueError before anything launches."""
    Hq, Hkv, D, ps = desc.num_q_heads, desc.num_kv_heads, desc.head_dim, desc.page_size
    if q.dtype != dtype or k_cache.dtype != dtype or v_cache.dtype != dtype or \
            out.dtype != dtype:
        raise TypeError("q, k/v caches and out must be %s" % dtype)
    if q.dim() != 3 or q.shape[1] != Hq or q.shape[2] != D:
        raise ValueError("q must be [B, %d, %d], got %s" % (Hq, D, tuple(q.shape)))
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape %s, got %s" % (tuple(q.shape), tuple(out.shape)))
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (Hkv, ps, D) or k_cache.stride(3) != 1:
        raise ValueError("caches must be [num_pages, %d, %d, %d] with D contiguous, got %s"
                         % (Hkv, ps, D, tuple(k_cache.shape)))
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_cache.shape[0] < 1:
        raise ValueError("the caches hold no page")
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise TypeError("lse must be contiguous float32")
        if tuple(lse.shape) != tuple(q.shape[:2]):
            raise ValueError("lse must be [B, Hq] = %s, got %s" % (tuple(q.shape[:2]),
                                                                  tuple(lse.shape)))


def check_dense_shapes(desc: PaDecodeDesc, dtype, q, k_cache, v_cache, page_table, context_lens,
                       out, lse, max_context_len: int) -> None:
    """Every shape of a pa_decode_run call checked against the descriptor and
    the batch (B = q.shape[0]): page_table int32 [>= B, >= ceil(max_context_len
    / page_size)] with unit inner stride, and storage behind each of its first
    B rows for a whole row stride (the kernel may read a row's entries up to
    the stride); context_lens int32 with >= B entries."""
    _check_step_shapes(desc, dtype, q, k_cache, v_cache, out, lse)
    B = q.shape[0]
    if page_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("page_table and context_lens must be int32")
    if page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be [B, pt_stride] with unit inner stride")
    if not context_lens.is_contiguous() or context_lens.dim() != 1:
        raise ValueError("context_lens must be a contiguous 1-D tensor")
    if B == 0:
        return
    ps = desc.page_size
    if page_table.shape[0] < B:
        raise ValueError("page_table has %d rows for a batch of %d" % (page_table.shape[0], B))
    if page_table.shape[1] * ps < max_context_len:
        raise ValueError("page_table rows of %d pages cannot hold %d tokens"
                         % (page_table.shape[1], max_context_len))
    if page_table.stride(0) < page_table.shape[1] or \
            _storage_elems(page_table) < B * page_table.stride(0):
        raise ValueError("page_table storage must hold %d rows of stride %d"
                         % (B, page_table.stride(0)))
    if context_lens.numel() < B:
        raise ValueError("context_lens has %d entries for a batch of %d"
                         % (context_lens.numel(), B))


def check_csr_shapes(desc: PaDecodeDesc, dtype, q, k_cache, v_cache, page_indptr, page_indices,
                     last_page_len, nnz_pages: int, out, lse) -> None:
    """Every shape of a pa_decode_run_csr call: page_indptr >= B + 1 entries,
    last_page_len >= B, page_indices >= nnz_pages (all contiguous int32)."""
    _check_step_shapes(desc, dtype, q, k_cache, v_cache, out, lse)
    B = q.shape[0]
    for name, t in (("page_indptr", page_indptr), ("page_indices", page_indices),
                    ("last_page_len", last_page_len)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1:
            raise TypeError("%s must be a contiguous 1-D int32 tensor" % name)
    if nnz_pages < 0 or page_indices.numel() < nnz_pages:
        raise ValueError("page_indices has %d entries for nnz_pages %d"
                         % (page_indices.numel(), nnz_pages))
    if B > 0 and (page_indptr.numel() < B + 1 or last_page_len.numel() < B):
        raise ValueError("page_indptr needs %d entries and last_page_len %d (batch %d)"
                         % (B + 1, B, B))


class PagedDecode:
    """Handle-owning front end for torch tensors on one GPU.

    ``make_args`` builds the C argument block once (a timing loop can reuse it
    with ``run_args``); ``__call__`` allocates out/lse/workspace with torch.
    """

    def __init__(self, num_q_heads, num_kv_heads, head_dim, dtype, max_batch,
                 max_context_len, page_size=16, device=0, rope=None, debug_checks=0):
        self.desc = make_desc(num_q_heads, num_kv_heads, head_dim, dtype, max_batch,
                              max_context_len, page_size, device, rope=rope,
                              debug_checks=debug_checks)
        self.dtype = dtype
        self.device = torch.device("cuda", device)
        self.handle = pa_decode_create(self.desc)
        self._workspace = None

    def close(self):
        if self.handle is not None:
            pa_decode_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, batch, max_context_len, sliding_window=0, partition_size=0):
        return pa_decode_workspace_size(self.handle, batch, max_context_len, sliding_window,
                                        partition_size)

    def workspace(self, nbytes: int) -> torch.Tensor:
        """A cached uint8 device buffer of at least nbytes (never shrinks)."""
        if self._workspace is None or self._workspace.numel() < nbytes:
            self._workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8,
                                          device=self.device)
        return self._workspace

    def make_args(self, q, k_cache, v_cache, page_table, context_lens, scale, out, lse=None,
                  max_context_len=None, sliding_window=0, partition_size=0,
                  workspace=None) -> PaDecodeArgs:
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                        ("page_table", page_table), ("context_lens", context_lens),
                        ("out", out)) + ((("lse", lse),) if lse is not None else ()):
            if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
                raise TypeError("%s must be a device tensor" % name)
        B = q.shape[0] if q.dim() > 0 else 0
        if max_context_len is None:
            max_context_len = int(context_lens[:B].max().item()) if B else 0
        check_dense_shapes(self.desc, self.dtype, q, k_cache, v_cache, page_table, context_lens,
                           out, lse, max_context_len)
        ws_bytes = self.workspace_size(B, max_context_len, sliding_window, partition_size)
        if workspace is None:
            workspace = self.workspace(ws_bytes)
        a = PaDecodeArgs()
        a.q = q.data_ptr()
        a.k_cache = k_cache.data_ptr()
        a.v_cache = v_cache.data_ptr()
        a.kv_stride_page = k_cache.stride(0)
        a.kv_stride_head = k_cache.stride(1)
        a.kv_stride_slot = k_cache.stride(2)
        a.num_pages = k_cache.shape[0]
        a.page_table = page_table.data_ptr()
        a.pt_stride = page_table.stride(0)
        a.context_lens = context_lens.data_ptr()
        a.batch = B
        a.max_context_len = max_context_len
        a.scale = float(scale)
        a.sliding_window = int(sliding_window)
        a.partition_size = int(partition_size)
        a.out = out.data_ptr()
        a.lse = lse.data_ptr() if lse is not None else None
        a.workspace = workspace.data_ptr() if workspace is not None else None
        a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        a._keep = (q, k_cache, v_cache, page_table, context_lens, out, lse, workspace)
        return a

    def run_args(self, args: PaDecodeArgs, stream: Optional[int] = None) -> None:
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        pa_decode_run(self.handle, args, stream)

    def run_noalloc_args(self, args: PaDecodeArgs, stream: Optional[int] = None) -> None:
        """pa_decode_run_noalloc on an argument block from make_args (its
        workspace is ignored)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        pa_decode_run_noalloc(self.handle, args, stream)

    def __call__(self, q, k_cache, v_cache, page_table, context_lens, scale,
                 max_context_len=None, sliding_window=0, partition_size=0, out=None,
                 lse=None):
        """One decode step; returns (out, lse).  partition_size: 0 for the
        planner's fixed partitions, a multiple of 16 to force their size, or
        PA_DECODE_PARTITION_BALANCED for the length-balanced schedule (ragged
        batches of up to 64 sequences)."""
        B, Hq, D = q.shape
        if out is None:
            out = torch.empty((B, Hq, D), dtype=self.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        args = self.make_args(q, k_cache, v_cache, page_table, context_lens, scale, out, lse,
                              max_context_len, sliding_window, partition_size)
        self.run_args(args)
        return out, lse

    def make_csr_args(self, q, k_cache, v_cache, page_indptr, page_indices, last_page_len,
                      nnz_pages, scale, out, lse=None, max_context_len=0, sliding_window=0,
                      partition_size=0, workspace=None) -> PaDecodeCsrArgs:
        """Argument block of pa_decode_run_csr; nnz_pages is the host copy of
        page_indptr[-1]."""
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                        ("page_indptr", page_indptr), ("page_indices", page_indices),
                        ("last_page_len", last_page_len), ("out", out)) + \
                ((("lse", lse),) if lse is not None else ()):
            if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
                raise TypeError("%s must be a device tensor" % name)
        check_csr_shapes(self.desc, self.dtype, q, k_cache, v_cache, page_indptr, page_indices,
                         last_page_len, int(nnz_pages), out, lse)
        B = q.shape[0]
        ws_bytes = pa_decode_workspace_size_csr(self.handle, B, nnz_pages, max_context_len,
                                                sliding_window, partition_size)
        if workspace is None:
            workspace = self.workspace(ws_bytes)
        a = PaDecodeCsrArgs()
        a.q = q.data_ptr()
        a.k_cache = k_cache.data_ptr()
        a.v_cache = v_cache.data_ptr()
        a.kv_stride_page = k_cache.stride(0)
        a.kv_stride_head = k_cache.stride(1)
        a.kv_stride_slot = k_cache.stride(2)
        a.num_pages = k_cache.shape[0]
        a.page_indptr = page_indptr.data_ptr()
        a.page_indices = page_indices.data_ptr() if page_indices.numel() else None
        a.last_page_len = last_page_len.data_ptr()
        a.nnz_pages = int(nnz_pages)
        a.batch = B
        a.max_context_len = int(max_context_len)
        a.scale = float(scale)
        a.sliding_window = int(sliding_window)
        a.partition_size = int(partition_size)
        a.out = out.data_ptr()
        a.lse = lse.data_ptr() if lse is not None else None
        a.workspace = workspace.data_ptr() if workspace is not None else None
        a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        a._keep = (q, k_cache, v_cache, page_indptr, page_indices, last_page_len, out, lse,
                   workspace)
        return a

    def run_csr_args(self, args: PaDecodeCsrArgs, stream: Optional[int] = None) -> None:
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        pa_decode_run_csr(self.handle, args, stream)

    def last_plan(self) -> PaDecodePlan:
        return pa_decode_last_plan(self.handle)
