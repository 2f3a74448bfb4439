"""GPU: pa_decode_run / pa_decode_run_csr reject bad arguments on the host.

Every argument the library can check without reading device memory is
checked before anything is launched: null pointers, 16-byte alignment of q,
the caches, out and the workspace, stride granularity and kv_stride_slot >=
D, partition sizes, batch and max_context_len against the description, the
page-table row stride, a non-finite scale, and (CSR) nnz_pages.  Each
rejected call returns PA_DECODE_INVALID_ARG, launches nothing (out keeps a
sentinel) and leaves the handle usable: a valid call afterwards is right.
A zero batch is a valid no-op; the balanced schedule refuses more than 64
sequences (PA_DECODE_UNSUPPORTED).
"""
import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, engine, run_oracle, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _dense_setup():
    p = W.generate(W.CONFIGS["llama1b_ctx3060_f16"])
    d = to_device(p)
    eng = engine(p)
    out = torch.full_like(d.q, SENTINEL)
    lse = torch.full(d.q.shape[:2], SENTINEL, dtype=torch.float32, device="cuda")
    # A forced small partition size makes the plan split, so the workspace
    # checks apply too.  The workspace has 256 spare bytes, so that the
    # misaligned variant below still lies inside it.
    need = eng.workspace_size(1, p.max_context_len, 0, 128)
    assert need > 0
    ws = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale, out,
                         lse, max_context_len=p.max_context_len, partition_size=128,
                         workspace=ws)
    return p, eng, out, lse, args


def _clone(a):
    """A byte copy of a ctypes argument block (the original keeps the
    tensors alive)."""
    return type(a).from_buffer_copy(a)


def _bad_dense(a, eng):
    """(name, mutator) pairs, each giving one argument outside the contract."""
    D = eng.desc.head_dim
    ws_ok = a.workspace

    def f(**kw):
        def m(x):
            for k, v in kw.items():
                setattr(x, k, v(getattr(x, k)) if callable(v) else v)
        return m
    return [
        ("q null", f(q=None)),
        ("k null", f(k_cache=None)),
        ("out null", f(out=None)),
        ("page table null", f(page_table=None)),
        ("context lens null", f(context_lens=None)),
        ("q misaligned", f(q=lambda v: v + 2)),
        ("k misaligned", f(k_cache=lambda v: v + 2)),
        ("v misaligned", f(v_cache=lambda v: v + 8)),
        ("out misaligned", f(out=lambda v: v + 2)),
        ("workspace misaligned", f(workspace=lambda v: ws_ok + 8, workspace_bytes=lambda v: v - 8)),
        ("page stride not 16-byte granular", f(kv_stride_page=lambda v: v + 1)),
        ("head stride negative", f(kv_stride_head=-8)),
        ("slot stride below head_dim", f(kv_stride_slot=D - 8)),
        ("no pages", f(num_pages=0)),
        ("row stride too short", f(pt_stride=1)),
        ("partition size not a page multiple", f(partition_size=24)),
        ("partition size negative", f(partition_size=-16)),
        ("batch negative", f(batch=-1)),
        ("batch above max_batch", f(batch=lambda v: eng.desc.max_batch + 1)),
        ("max_context_len negative", f(max_context_len=-1)),
        ("max_context_len above the description", f(max_context_len=lambda v: eng.desc.max_context_len + 1)),
        ("scale nan", f(scale=float("nan"))),
        ("scale inf", f(scale=float("inf"))),
    ]


def test_dense_run_rejects_bad_arguments_and_launches_nothing():
    p, eng, out, lse, args = _dense_setup()
    for name, mutate in _bad_dense(args, eng):
        a = _clone(args)
        mutate(a)
        with pytest.raises(B.PaDecodeError) as e:
            eng.run_args(a)
        assert e.value.status == B.PA_DECODE_INVALID_ARG, name
        torch.cuda.synchronize()
        assert torch.all(out == SENTINEL), "%s: out was written" % name
        assert torch.all(lse == SENTINEL), "%s: lse was written" % name
    # The handle still works.
    eng.run_args(args)
    torch.cuda.synchronize()
    ref = run_oracle(p)
    compare(out.cpu(), lse.cpu(), ref[0], ref[1], p.workload.dtype, "after rejected calls")


def test_zero_batch_is_a_no_op():
    p, eng, out, lse, args = _dense_setup()
    a = _clone(args)
    a.batch = 0
    eng.run_args(a)
    torch.cuda.synchronize()
    assert torch.all(out == SENTINEL) and torch.all(lse == SENTINEL)


def test_csr_run_rejects_bad_arguments_and_launches_nothing():
    p = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    csr = W.to_csr(p)
    eng = engine(p)
    q, k, v = p.q.cuda(), p.k_cache.cuda(), p.v_cache.cuda()
    out = torch.full_like(q, SENTINEL)
    lse = torch.full(q.shape[:2], SENTINEL, dtype=torch.float32, device="cuda")
    args = eng.make_csr_args(q, k, v, csr.indptr.cuda(), csr.indices.cuda(),
                             csr.last_page_len.cuda(), csr.nnz_pages, p.scale, out, lse,
                             max_context_len=p.max_context_len, partition_size=256)
    bad = [
        ("nnz negative", dict(nnz_pages=-1)),
        ("indptr null", dict(page_indptr=None)),
        ("last_page_len null", dict(last_page_len=None)),
        ("indices null with pages", dict(page_indices=None)),
        ("q misaligned", dict(q=args.q + 2)),
        ("slot stride below head_dim", dict(kv_stride_slot=64)),
        ("partition size not a page multiple", dict(partition_size=40)),
        ("batch above max_batch", dict(batch=eng.desc.max_batch + 1)),
        ("scale nan", dict(scale=float("nan"))),
    ]
    for name, kw in bad:
        a = _clone(args)
        for key, val in kw.items():
            setattr(a, key, val)
        with pytest.raises(B.PaDecodeError) as e:
            eng.run_csr_args(a)
        assert e.value.status == B.PA_DECODE_INVALID_ARG, name
        torch.cuda.synchronize()
        assert torch.all(out == SENTINEL), "%s: out was written" % name
    eng.run_csr_args(args)
    torch.cuda.synchronize()
    ref = run_oracle(p)
    compare(out.cpu(), lse.cpu(), ref[0], ref[1], p.workload.dtype, "csr after rejected calls")


def test_balanced_schedule_above_64_sequences_is_unsupported():
    """The length-balanced schedule takes at most 64 sequences: a call with
    65 returns PA_DECODE_UNSUPPORTED and launches nothing; 64 runs."""
    for batch, ok in ((65, False), (64, True)):
        w = W.custom(batch=batch, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                     context_lens=[1 + 37 * i for i in range(batch)], seed=batch)
        p = W.generate(w)
        d = to_device(p)
        eng = engine(p)
        out = torch.full_like(d.q, SENTINEL)
        lse = torch.full(d.q.shape[:2], SENTINEL, dtype=torch.float32, device="cuda")
        if not ok:
            with pytest.raises(B.PaDecodeError) as e:
                eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                              out, lse, max_context_len=p.max_context_len,
                              partition_size=B.PA_DECODE_PARTITION_BALANCED)
            assert e.value.status == B.PA_DECODE_UNSUPPORTED
            torch.cuda.synchronize()
            assert torch.all(out == SENTINEL)
            continue
        args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                             out, lse, max_context_len=p.max_context_len,
                             partition_size=B.PA_DECODE_PARTITION_BALANCED)
        eng.run_args(args)
        torch.cuda.synchronize()
        ref = run_oracle(p)
        compare(out.cpu(), lse.cpu(), ref[0], ref[1], torch.float16, "balanced batch 64")
