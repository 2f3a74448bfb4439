"""GPU: the no-allocation entry point pa_decode_run_noalloc against
pa_decode_run (needs an MI355X).

pa_decode_run_noalloc takes the same arguments as pa_decode_run but keeps the
partition states in the library's fixed per-device scratch array instead of
a caller workspace.  Checked through the C ABI:
  * two calls in a row, the second on a smaller input, each bitwise equal to
    pa_decode_run on the same inputs with its own workspace, and within the
    tolerances against the float64 oracle (whole tensor and every row);
  * an unsplit plan (no states at all) and the length-balanced schedule;
  * a plan whose states exceed the scratch is rejected with
    PA_DECODE_EXCEEDS_SCRATCH and writes nothing.
"""
import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, engine, run_oracle, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _both(p, partition_size):
    """(out, lse) of pa_decode_run and of pa_decode_run_noalloc on the same
    inputs (fresh output buffers), and the plan."""
    d = to_device(p)
    eng = engine(p)
    res = []
    for noalloc in (False, True):
        out = torch.full_like(d.q, SENTINEL)
        lse = torch.full(d.q.shape[:2], SENTINEL, dtype=torch.float32, device="cuda")
        args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                             out, lse, max_context_len=p.max_context_len,
                             sliding_window=p.window, partition_size=partition_size)
        if noalloc:
            args.workspace = None      # ignored by the entry point
            args.workspace_bytes = 0
            eng.run_noalloc_args(args)
        else:
            eng.run_args(args)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu(), eng.last_plan().as_dict()))
    return res


def test_noalloc_matches_run_on_two_calls_in_a_row():
    big = W.generate(W.CONFIGS["ctx100k_gqa6_f16"])           # 196 partitions, 4.9 MB of states
    small = W.generate(W.CONFIGS["llama1b_ctx3060_f16"])      # 24 partitions
    for p, what in ((big, "100k"), (small, "3060 after 100k")):
        (o1, l1, plan1), (o2, l2, plan2) = _both(p, p.workload.partition_size)
        assert plan1 == plan2 and plan2["split"] == 1
        assert 0 < plan2["workspace_bytes"] <= B.pa_decode_noalloc_scratch_bytes()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), what
        ref = run_oracle(p)
        compare(o2, l2, ref[0], ref[1], p.workload.dtype, "noalloc " + what)


def test_noalloc_unsplit_and_balanced():
    tiny = W.generate(W.CONFIGS["tiny_gqa4_f32"])
    (o1, l1, plan1), (o2, l2, plan2) = _both(tiny, 320)           # one partition: no states
    assert plan2["split"] == 0 and plan2["workspace_bytes"] == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref = run_oracle(tiny)
    compare(o2, l2, ref[0], ref[1], torch.float32, "noalloc unsplit")
    ragged = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])      # balanced schedule, counts too
    (o1, l1, plan1), (o2, l2, plan2) = _both(ragged, W.BALANCED)
    assert plan2["balanced_waves"] > 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref = run_oracle(ragged)
    compare(o2, l2, ref[0], ref[1], torch.float16, "noalloc balanced")


def test_noalloc_rejects_states_beyond_the_scratch():
    """64 sequences on the balanced schedule at up to 4096 tokens need 128
    state rows per (sequence, head): 134 MB, over the 64 MiB scratch."""
    Bsz, Hq, Hkv, D = 64, 32, 8, 128
    eng = B.PagedDecode(Hq, Hkv, D, torch.float16, max_batch=64, max_context_len=4096)
    q = torch.zeros(Bsz, Hq, D, dtype=torch.float16, device="cuda")
    kc = torch.zeros(8, Hkv, 16, D, dtype=torch.float16, device="cuda")
    pt = torch.zeros(Bsz, 256, dtype=torch.int32, device="cuda")
    lens = torch.ones(Bsz, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, SENTINEL)
    lse = torch.full((Bsz, Hq), SENTINEL, dtype=torch.float32, device="cuda")
    need = eng.workspace_size(Bsz, 4096, 0, B.PA_DECODE_PARTITION_BALANCED)
    assert need > B.pa_decode_noalloc_scratch_bytes()
    args = eng.make_args(q, kc, kc, pt, lens, 0.1, out, lse, max_context_len=4096,
                         partition_size=B.PA_DECODE_PARTITION_BALANCED, workspace=out)
    with pytest.raises(B.PaDecodeError) as e:
        eng.run_noalloc_args(args)
    assert e.value.status == B.PA_DECODE_EXCEEDS_SCRATCH
    assert "scratch" in B.pa_decode_status_string(B.PA_DECODE_EXCEEDS_SCRATCH)
    torch.cuda.synchronize()
    assert torch.all(out == SENTINEL) and torch.all(lse == SENTINEL)
    # the same sizes with fixed partitions fit and run
    args = eng.make_args(q, kc, kc, pt, lens, 0.1, out, lse, max_context_len=4096)
    eng.run_noalloc_args(args)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    eng.close()
