"""GPU: the device-side contract check (needs an MI355X).

The caller promises that every page id read is < num_pages, that context
lengths lie in [0, max_context_len] and (CSR) that every row lies inside
[0, nnz_pages].  The kernel never takes an address from a value that breaks
this: page ids outside the pool read page 0, lengths and rows are clamped.
With desc.debug_checks = 1 the handle also collects a violation bit per kind
(pa_decode_debug_status).  Here:
  * valid runs report nothing and give the same bits as a handle without
    the check;
  * out-of-range page ids (past the pool, negative) in the dense, windowed
    and CSR paths, lengths above max_context_len or negative, and CSR rows
    that run backwards or past nnz_pages are reported; the run finishes and
    reads nothing outside the caller's buffers; the next valid run reports
    nothing.
Each case runs under both schedules: fixed partitions and the
length-balanced one (whose waves read every sequence's length and row).
"""
import dataclasses

import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, run_oracle

pytestmark = pytest.mark.gpu


def _engine(w, debug):
    return B.PagedDecode(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=64,
                         max_context_len=1 << 16, rope=w.rope, debug_checks=debug)


SCHEDULES = [0, B.PA_DECODE_PARTITION_BALANCED]


def _run(eng, p, page_table=None, lens=None, max_ctx=None, S=0):
    d = lambda t: t.cuda()  # noqa: E731
    pt = d(p.page_table if page_table is None else page_table)
    cl = d(p.context_lens if lens is None else lens)
    out, lse = eng(d(p.q), d(p.k_cache), d(p.v_cache), pt, cl, p.scale,
                   max_context_len=p.max_context_len if max_ctx is None else max_ctx,
                   sliding_window=p.window, partition_size=S)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("S", SCHEDULES)
@pytest.mark.parametrize("rope", [None, (500000.0, 1.0)])
def test_valid_runs_report_nothing_and_match(rope, S):
    w = W.custom(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=torch.float16,
                 context_lens=[1, 700, 3060], seed=700, rope=rope)
    p = W.generate(w)
    plain, checked = _engine(w, 0), _engine(w, 1)
    a = _run(plain, p, S=S)
    b = _run(checked, p, S=S)
    assert B.pa_decode_debug_status(checked.handle) == 0
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(B.PaDecodeError):
        B.pa_decode_debug_status(plain.handle)   # no status word without the check
    ref = run_oracle(p)
    compare(b[0], b[1], ref[0], ref[1], w.dtype, what="checked run")


@pytest.mark.parametrize("S", SCHEDULES)
@pytest.mark.parametrize("window", [0, 500])
@pytest.mark.parametrize("bad_id", ["past_pool", "negative"])
def test_out_of_range_page_ids_are_reported(window, bad_id, S):
    w = W.custom(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[900, 2000], seed=701, window=window)
    p = W.generate(w)
    eng = _engine(w, 1)
    pt = p.page_table.clone()
    num_pages = p.k_cache.shape[0]
    pt[1, 100] = num_pages + 7 if bad_id == "past_pool" else -1   # a page of tokens 1600..1615
    out, lse = _run(eng, p, page_table=pt, S=S)
    assert B.pa_decode_debug_status(eng.handle) & B.PA_DECODE_VIOLATION_PAGE
    # Sequence 0 is untouched by the bad entry of row 1.
    ref = run_oracle(p)
    compare(out[:1], lse[:1], ref[0][:1], ref[1][:1], w.dtype, what="row 0 beside a bad row")
    _run(eng, p, S=S)
    assert B.pa_decode_debug_status(eng.handle) == 0


@pytest.mark.parametrize("S", SCHEDULES)
def test_lengths_outside_the_contract_are_reported(S):
    w = W.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                 context_lens=[300, 1000, 64], seed=702)
    p = W.generate(w)
    eng = _engine(w, 1)
    for bad in (1001, 5000, -5):
        lens = p.context_lens.clone()
        lens[1] = bad
        out, lse = _run(eng, p, lens=lens, max_ctx=1000, S=S)
        assert B.pa_decode_debug_status(eng.handle) & B.PA_DECODE_VIOLATION_LENGTH, bad
        assert torch.isfinite(out).all()
    _run(eng, p, S=S)
    assert B.pa_decode_debug_status(eng.handle) == 0


@pytest.mark.parametrize("S", SCHEDULES)
def test_csr_rows_outside_the_contract_are_reported(S):
    w = W.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[50, 700, 333], seed=703)
    p = W.generate(w)
    csr = W.to_csr(p)
    eng = _engine(w, 1)
    q, k, v = p.q.cuda(), p.k_cache.cuda(), p.v_cache.cuda()

    def run(indptr, indices):
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        args = eng.make_csr_args(q, k, v, indptr.cuda(), indices.cuda(),
                                 csr.last_page_len.cuda(), csr.nnz_pages, p.scale, out, lse,
                                 max_context_len=p.max_context_len, partition_size=S)
        eng.run_csr_args(args)
        torch.cuda.synchronize()
        return B.pa_decode_debug_status(eng.handle)

    assert run(csr.indptr, csr.indices) == 0
    backwards = csr.indptr.clone()
    backwards[2] = backwards[1] - 3            # row 1 runs backwards, row 2 starts early
    assert run(backwards, csr.indices) & B.PA_DECODE_VIOLATION_ROW
    past = csr.indptr.clone()
    past[3] = csr.nnz_pages + 40               # the last row runs past nnz_pages
    assert run(past, csr.indices) & B.PA_DECODE_VIOLATION_ROW
    bad_ids = csr.indices.clone()
    bad_ids[5] = p.k_cache.shape[0] + 1
    assert run(csr.indptr, bad_ids) & B.PA_DECODE_VIOLATION_PAGE
    assert run(csr.indptr, csr.indices) == 0


@pytest.mark.parametrize("S", SCHEDULES)
def test_rotary_kernel_reports_bad_page_ids(S):
    w = W.custom(batch=1, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=torch.float16,
                 context_lens=[1500], seed=704, rope=(10000.0, 1.0))
    p = W.generate(w)
    eng = _engine(w, 1)
    pt = p.page_table.clone()
    pt[0, 10] = 1 << 30
    _run(eng, p, page_table=pt, S=S)
    assert B.pa_decode_debug_status(eng.handle) & B.PA_DECODE_VIOLATION_PAGE
