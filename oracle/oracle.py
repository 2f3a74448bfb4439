"""ctypes front end of the plain-C float64 oracle (``pa_oracle.c``).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library.

The C file holds all of the arithmetic; this module only compiles it with gcc,
marshals CPU tensors into raw pointers and allocates the float64 outputs.
The definition it follows is the one stated at the top of ``pa_oracle.c``:
out = softmax(scale * q K^T) V per query head over the visible keys, walking
the page table; lse = ln sum exp(scale * q K^T); with rotary_mode 1, q and
every key are first turned by the rotary embedding (rotate-half pairing,
theta_i = rope_theta^(-2i/D) / rope_scale, key j at position j, the query at
position n_b - 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_lib = None
_lock = threading.Lock()

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into oracle/libpa_oracle.so with gcc (OpenMP, -O2)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load an oracle shared library built from pa_oracle.c (or a planted-mistake copy)."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        _lib = load_library(build(force=False))
        return _lib


def _declare(lib):
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    f64 = ctypes.c_double
    problem = [i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, i64, i64, i64,
               vp, i32, vp, f64, i32, i32, f64, f64]
    lib.pa_oracle_decode.argtypes = problem + [i32, vp, vp]
    lib.pa_oracle_decode.restype = i32
    lib.pa_oracle_decode_split.argtypes = problem + [i32, i32, vp, vp]
    lib.pa_oracle_decode_split.restype = i32
    lib.pa_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.pa_oracle_f16_to_f64.restype = ctypes.c_double
    lib.pa_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.pa_oracle_bf16_to_f64.restype = ctypes.c_double
    lib.pa_oracle_max_threads.argtypes = []
    lib.pa_oracle_max_threads.restype = i32


def max_threads() -> int:
    return int(_load().pa_oracle_max_threads())


def f16_to_f64(bits: int) -> float:
    return float(_load().pa_oracle_f16_to_f64(bits))


def bf16_to_f64(bits: int) -> float:
    return float(_load().pa_oracle_bf16_to_f64(bits))


def _problem_args(q, k_cache, v_cache, page_table, context_lens, scale, window, rotary):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("page_table", page_table), ("context_lens", context_lens)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cpu":
            raise TypeError("oracle: %s must be a CPU torch tensor" % name)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("oracle: q must be a contiguous [B, Hq, D] tensor")
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or \
            k_cache.stride() != v_cache.stride():
        raise ValueError("oracle: k/v cache must be [num_pages, Hkv, page_size, D] alike")
    if k_cache.stride(3) != 1:
        raise ValueError("oracle: the D axis of the cache must be contiguous")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("oracle: k and v caches must share a dtype")
    if page_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("oracle: page_table and context_lens must be int32")
    if page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("oracle: page_table must be [B, pt_stride] with unit inner stride")
    B, Hq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if Dk != D or page_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("oracle: shape mismatch")
    context_lens = context_lens.contiguous()
    args = [B, Hq, Hkv, D, page_size, _DTYPE_CODE[q.dtype], q.data_ptr(),
            _DTYPE_CODE[k_cache.dtype], k_cache.data_ptr(), v_cache.data_ptr(), num_pages,
            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), page_table.data_ptr(),
            page_table.stride(0), context_lens.data_ptr(), float(scale), int(window)]
    mode, theta, rscale = (0, 1.0, 1.0) if rotary is None else (1, float(rotary[0]), float(rotary[1]))
    args += [mode, theta, rscale]
    keep = (q, k_cache, v_cache, page_table, context_lens)
    return args, keep, (B, Hq, D)


def _outputs(shape):
    B, Hq, D = shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    return out, lse


def decode(q, k_cache, v_cache, page_table, context_lens, scale, window=0, threads=0,
           lib=None, rotary=None):
    """Direct f64 decode attention. Returns (out [B,Hq,D], lse [B,Hq]) as float64 numpy.

    ``scale`` is used as given (pass float(np.float32(s)) to match a float32 scale).
    ``rotary``: None (no rotary embedding) or (rope_theta, rope_scale) for
    rotary_mode 1, each used as given.
    """
    args, keep, shape = _problem_args(q, k_cache, v_cache, page_table, context_lens, scale,
                                      window, rotary)
    out, lse = _outputs(shape)
    rc = (lib or _load()).pa_oracle_decode(*args, int(threads), out.ctypes.data,
                                           lse.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError("oracle: invalid problem (code %d)" % rc)
    return out, lse


def decode_split(q, k_cache, v_cache, page_table, context_lens, scale, partition_size,
                 window=0, threads=0, rotary=None):
    """Partitioned f64 decode attention: per-partition states then the LSE merge."""
    args, keep, shape = _problem_args(q, k_cache, v_cache, page_table, context_lens, scale,
                                      window, rotary)
    out, lse = _outputs(shape)
    rc = _load().pa_oracle_decode_split(*args, int(partition_size), int(threads),
                                        out.ctypes.data, lse.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError("oracle: invalid problem (code %d)" % rc)
    return out, lse
