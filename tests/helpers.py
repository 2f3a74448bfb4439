"""Shared helpers of the GPU parity tests: run a problem through the HIP
library and compare with the float64 oracle.

Tolerances (the GPU path accumulates in float32 and rounds out to its dtype;
the figures are defined in tests/parity.py):
  * out: relative L2 error against the oracle rounded (RNE) to the output
    dtype, over the whole [B, Hq, D] tensor: <= 1e-3 for f16/bf16, <= 1e-5 for
    f32; and the same bound on every (sequence, query head) row for the error
    beyond one output ulp per element;
  * lse: absolute error <= 1e-4 on finite entries; -inf exactly where the
    oracle has -inf (empty contexts).
"""
import dataclasses

import numpy as np
import torch

import oracle
from paged_kv_decode_amd import binding
from paged_kv_decode_amd import workloads as W

import parity

OUT_TOL = parity.OUT_TOL
LSE_TOL = parity.LSE_TOL


def to_device(p: W.Problem, device="cuda"):
    return dataclasses.replace(
        p, q=p.q.to(device), k_cache=p.k_cache.to(device), v_cache=p.v_cache.to(device),
        page_table=p.page_table.to(device), context_lens=p.context_lens.to(device))


_HANDLES = {}


def engine(p: W.Problem) -> binding.PagedDecode:
    w = p.workload
    key = (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.rope)
    eng = _HANDLES.get(key)
    if eng is None:
        eng = binding.PagedDecode(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype,
                                  max_batch=4096, max_context_len=1 << 20, rope=w.rope)
        _HANDLES[key] = eng
    return eng


def run_gpu(p: W.Problem, partition_size=None, dev=None):
    """Run the HIP path; returns (out, lse) on the CPU and the plan."""
    d = dev if dev is not None else to_device(p)
    eng = engine(p)
    S = p.workload.partition_size if partition_size is None else partition_size
    out, lse = eng(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                   max_context_len=p.max_context_len, sliding_window=p.window,
                   partition_size=S)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), eng.last_plan().as_dict()


def run_gpu_csr(p: W.Problem, csr: W.CsrTable, partition_size=None, max_context_len=None):
    """Run the HIP path from a CSR page table (pa_decode_run_csr); returns
    (out, lse) on the CPU and the plan."""
    eng = engine(p)
    S = p.workload.partition_size if partition_size is None else partition_size
    q, k, v = p.q.cuda(), p.k_cache.cuda(), p.v_cache.cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    mc = p.max_context_len if max_context_len is None else max_context_len
    args = eng.make_csr_args(q, k, v, csr.indptr.cuda(), csr.indices.cuda(),
                             csr.last_page_len.cuda(), csr.nnz_pages, p.scale, out, lse,
                             max_context_len=mc, sliding_window=p.window, partition_size=S)
    eng.run_csr_args(args)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), eng.last_plan().as_dict()


def run_oracle(p: W.Problem):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens, p.scale,
                         window=p.window, rotary=p.workload.rope)


def compare(out, lse, ref_out, ref_lse, dtype, what="", lse_rel=0.0):
    """Assert the tolerances (tests/parity.py) on the whole tensor and on every
    (sequence, query head) row; returns (rel_l2, lse_max_abs_err) and prints
    the worst row.  lse_rel > 0 widens the lse bound to LSE_TOL + lse_rel *
    |lse| per entry (scores far from order 1, where the float32 lse itself
    carries an error proportional to its magnitude); the excess over LSE_TOL
    is then printed."""
    g = out.double()
    assert torch.isfinite(g).all(), "%s: non-finite output" % what
    e = parity.out_errors(out, ref_out, dtype)
    heads = out.shape[1] if out.dim() == 3 else 1
    lerr, same_inf = parity.lse_error(lse, ref_lse)
    assert same_inf, "%s: -inf lse pattern differs" % what
    print("  %s: %s lse_err=%.3g" % (what, parity.describe(e, heads), lerr), flush=True)
    tol = OUT_TOL[dtype]
    assert e["rel_l2"] <= tol, "%s: out rel-L2 %.3g > %.3g" % (what, e["rel_l2"], tol)
    assert e["row_excess"] <= tol, "%s: row error %.3g > %.3g (%s)" % (
        what, e["row_excess"], tol, parity.describe(e, heads))
    if lse_rel > 0:
        ref = np.asarray(ref_lse, dtype=np.float64).reshape(-1)
        l = lse.double().numpy().reshape(-1)
        fin = ~np.isneginf(ref)
        bound = LSE_TOL + lse_rel * np.abs(ref[fin])
        worst = float((np.abs(l[fin] - ref[fin]) / bound).max()) if fin.any() else 0.0
        if lerr > LSE_TOL:
            print("  %s: lse err %.3g exceeds %.0e by %.3g (|lse| up to %.0f)" % (
                what, lerr, LSE_TOL, lerr - LSE_TOL, float(np.abs(ref[fin]).max())), flush=True)
        assert worst <= 1.0, "%s: lse err %.3g above %.0f%% of its bound" % (what, lerr, 100 * worst)
    else:
        assert lerr <= LSE_TOL, "%s: lse abs err %.3g > %.3g" % (what, lerr, LSE_TOL)
    return e["rel_l2"], lerr
