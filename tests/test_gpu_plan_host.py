"""GPU: host-side planning state of a handle (needs an MI355X for
pa_decode_create).

* The tuning overrides (PA_DECODE_WAVES_PER_PARTITION and the others) are
  read from the environment once, at pa_decode_create: a handle made while
  an override is set keeps it, one made without keeps the planner's choice,
  whatever the environment holds when they run; pa_decode_plan_query reads
  the environment at each call.
* Plans are cached per call shape: one handle alternating between dense and
  CSR calls and between call shapes (more shapes than the cache holds) gets
  the plan of each shape every time, and every result matches the oracle.
"""
import os

import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, run_oracle

pytestmark = pytest.mark.gpu


def _run(eng, p, S=0, csr=None):
    q, k, v = p.q.cuda(), p.k_cache.cuda(), p.v_cache.cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    if csr is None:
        args = eng.make_args(q, k, v, p.page_table.cuda(), p.context_lens.cuda(), p.scale, out,
                             lse, max_context_len=p.max_context_len, sliding_window=p.window,
                             partition_size=S)
        eng.run_args(args)
    else:
        args = eng.make_csr_args(q, k, v, csr.indptr.cuda(), csr.indices.cuda(),
                                 csr.last_page_len.cuda(), csr.nnz_pages, p.scale, out, lse,
                                 max_context_len=p.max_context_len, sliding_window=p.window,
                                 partition_size=S)
        eng.run_csr_args(args)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), eng.last_plan().as_dict()


def test_tuning_overrides_are_read_once_at_create(monkeypatch):
    w = W.CONFIGS["llama1b_ctx3060_f16"]
    p = W.generate(w)
    ref = run_oracle(p)
    env = "PA_DECODE_WAVES_PER_PARTITION"
    for name in (env, "PA_DECODE_WAVES_PER_GROUP", "PA_DECODE_BALANCED_START",
                 "PA_DECODE_BALANCED_WAVES_PER_CU"):
        monkeypatch.delenv(name, raising=False)

    def handle():
        return B.PagedDecode(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=4,
                             max_context_len=8192)

    eng_plain = handle()
    _, _, plain = _run(eng_plain, p, S=128)
    base = plain["waves_per_partition"]
    override = 1 if base != 1 else 2
    monkeypatch.setenv(env, str(override))
    eng_over = handle()
    # The plan query reads the environment at its call.
    q = B.pa_decode_plan_query(eng_over.desc, plain["num_cus"], plain["waves_per_cu"], 1,
                               p.max_context_len, 0, 128)
    assert q.waves_per_partition == override
    # A value set after both handles exist reaches neither.
    monkeypatch.setenv(env, str(next(v for v in (4, 2, 1) if v not in (base, override))))
    for eng, want in ((eng_plain, base), (eng_over, override)):
        out, lse, plan = _run(eng, p, S=128)
        assert plan["waves_per_partition"] == want, plan
        compare(out, lse, ref[0], ref[1], w.dtype, "waves per partition %d" % want)
        eng.close()


def test_plan_cache_alternating_shapes_and_forms():
    """Six call shapes (dense and CSR, forced and planned partition sizes,
    a window), more than the four cached plans, in two rounds on one handle:
    each call's plan equals the plan query's for its shape, and each result
    matches the oracle."""
    eng = B.PagedDecode(32, 8, 128, torch.float16, max_batch=64, max_context_len=1 << 16)
    probs = []
    for i, lens in enumerate(([3000, 17, 900], [1, 4096, 2048, 33], [8192] * 2)):
        w = W.custom(batch=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                     dtype=torch.float16, context_lens=lens, seed=930 + i,
                     window=1000 if i == 2 else 0)
        probs.append(W.generate(w))
    refs = [run_oracle(p) for p in probs]
    for round_ in range(2):
        for i, p in enumerate(probs):
            for form, S in (("dense", 0), ("csr", 0), ("dense", 256)):
                csr = W.to_csr(p) if form == "csr" else None
                out, lse, plan = _run(eng, p, S=S, csr=csr)
                compare(out, lse, refs[i][0], refs[i][1], torch.float16,
                        "round %d shape %d %s S=%d" % (round_, i, form, S))
                if form == "dense":
                    q = B.pa_decode_plan_query(eng.desc, plan["num_cus"], plan["waves_per_cu"],
                                               p.q.shape[0], p.max_context_len, p.window, S)
                else:
                    q = B.pa_decode_plan_query_csr(eng.desc, plan["num_cus"],
                                                   plan["waves_per_cu"], p.q.shape[0],
                                                   csr.nnz_pages, p.max_context_len, p.window, S)
                assert q.as_dict() == plan, (round_, i, form, S)
    eng.close()
