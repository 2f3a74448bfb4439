"""Shared helpers of the GPU parity tests: run a problem through the HIP
library and compare with the float64 oracle.

Tolerances (the GPU path accumulates in float32 and rounds out to its dtype):
  * out: relative L2 error against the oracle rounded (RNE) to the output
    dtype, over the whole [B, Hq, D] tensor: <= 1e-3 for f16/bf16, <= 1e-5 for
    f32;
  * lse: absolute error <= 1e-4 on finite entries; -inf exactly where the
    oracle has -inf (empty contexts).
"""
import dataclasses

import numpy as np
import torch

import oracle
from paged_kv_decode_amd import binding
from paged_kv_decode_amd import workloads as W

OUT_TOL = {torch.float32: 1e-5, torch.float16: 1e-3, torch.bfloat16: 1e-3}
LSE_TOL = 1e-4


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
    """Assert the tolerances above; returns (rel_l2, lse_max_abs_err).
    lse_rel > 0 widens the lse bound to LSE_TOL + lse_rel * |lse| per entry
    (for scores far from order 1, where float32 itself carries an error
    proportional to the magnitude)."""
    ref_r = torch.from_numpy(ref_out).to(dtype).double()
    g = out.double()
    assert torch.isfinite(g).all(), "%s: non-finite output" % what
    denom = ref_r.norm().item()
    rel = (g - ref_r).norm().item() / denom if denom > 0 else (g - ref_r).norm().item()
    lse_d = lse.double().numpy()
    inf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse_d), inf_ref), "%s: -inf lse pattern differs" % what
    fin = ~inf_ref
    lerr = float(np.abs(lse_d[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    assert rel <= OUT_TOL[dtype], "%s: out rel-L2 %.3g > %.3g" % (what, rel, OUT_TOL[dtype])
    if lse_rel > 0:
        bound = LSE_TOL + lse_rel * np.abs(ref_lse[fin])
        worst = float((np.abs(lse_d[fin] - ref_lse[fin]) / bound).max()) if fin.any() else 0.0
        assert worst <= 1.0, "%s: lse err %.3g above %.0f%% of its bound" % (what, lerr, 100 * worst)
    else:
        assert lerr <= LSE_TOL, "%s: lse abs err %.3g > %.3g" % (what, lerr, LSE_TOL)
    return rel, lerr
