"""GPU: the length-balanced schedule (partition_size
PA_DECODE_PARTITION_BALANCED) against the float64 oracle.

Under this schedule the kernel splits the batch's visible pages evenly over
each KV head's waves from the lengths it reads, cuts each wave's range at
sequence ends, and the merge combines each sequence's pieces.  Covered:
  * the batch workloads (ragged Llama-3.1-8B shape, head_dim 96 ragged,
    rotary ragged, head_dim 256 with a window) and single sequences;
  * edge batches: every context empty, 64 one-token sequences, 64 sequences
    mixing empty, one-token, page-multiple and long contexts, windows that
    cut pages; the same batches with rotary (waves without a segment);
  * NaN in every slot the method must not read;
  * the CSR page table and a token-major cache layout;
  * a workspace filled with garbage, then a second call with a smaller batch
    into the same workspace (state counts of the first call must not leak);
  * graph replays;
  * 32 seeded random shapes.
"""
import dataclasses
import random

import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, engine, run_gpu, run_gpu_csr, run_oracle, to_device

pytestmark = pytest.mark.gpu

BAL = B.PA_DECODE_PARTITION_BALANCED


def _check(p, what=""):
    ref_out, ref_lse = run_oracle(p)
    out, lse, plan = run_gpu(p, partition_size=BAL)
    assert p.workload.batch == 0 or plan["balanced_waves"] > 0, plan
    rel, lerr = compare(out, lse, ref_out, ref_lse, p.workload.dtype,
                        what="%s plan=%s" % (what, plan))
    print("%s balanced W=%d P=%d rel_l2=%.3g lse_err=%.3g" %
          (what, plan["balanced_waves"], plan["num_partitions"], rel, lerr), flush=True)
    return out, lse


@pytest.mark.parametrize("name", ["llama8b_b16_ragged_f16", "d96_b16_ragged_f16",
                                  "llama8b_b16_ragged_rope_f16", "d256_window4096_bf16",
                                  "tiny_gqa4_f32", "llama1b_ctx3060_f16",
                                  "llama1b_ctx3060_rope_f16"])
def test_balanced_workloads(name):
    _check(W.generate(W.CONFIGS[name]), name)


EDGE = {
    "all empty": [0, 0, 0],
    "64 one-token": [1] * 64,
    "64 mixed": [0, 1, 16, 17, 4096, 0, 3000, 33] * 8,
    "one long, many short": [9000] + [1, 2, 3, 0, 15, 16, 31] * 3,
    "two": [16, 5000],
}


@pytest.mark.parametrize("label", sorted(EDGE))
@pytest.mark.parametrize("D,dtype,G,hkv", [(64, torch.float16, 4, 2), (128, torch.bfloat16, 8, 1),
                                           (256, torch.float16, 1, 4), (96, torch.bfloat16, 6, 2),
                                           (64, torch.float32, 16, 1)])
def test_balanced_edge_batches(label, D, dtype, G, hkv):
    lens = EDGE[label]
    w = W.custom(batch=len(lens), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=len(lens) + D)
    _check(W.generate(w), "%s D=%d G=%d" % (label, D, G))


@pytest.mark.parametrize("label", sorted(EDGE))
@pytest.mark.parametrize("D,dtype,G,hkv", [(128, torch.float16, 4, 2), (256, torch.bfloat16, 2, 4)])
def test_balanced_rotary_edge_batches(label, D, dtype, G, hkv):
    """Rotary under the balanced schedule with waves that have no segment
    (every context empty, or fewer charged pages than waves): each wave
    still joins the workgroup's one barrier, where the rotary tables are
    built, exactly once."""
    lens = EDGE[label]
    w = W.custom(batch=len(lens), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=2 * len(lens) + D, rope=(500000.0, 1.0))
    _check(W.generate(w), "rotary %s D=%d G=%d" % (label, D, G))


@pytest.mark.parametrize("window", [1, 100, 4096])
def test_balanced_windows_with_poison(window):
    lens = [0, 1, 17, 99, 100, 101, 5000, 4097, 12000, 16]
    w = W.custom(batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128,
                 dtype=torch.float16, context_lens=lens, seed=77, window=window)
    _check(W.generate(w, poison=True, extra_pages=3), "window %d poisoned" % window)


def test_balanced_rotary_window():
    lens = [3000, 17, 0, 8000, 1]
    w = W.custom(batch=len(lens), num_q_heads=16, num_kv_heads=4, head_dim=128,
                 dtype=torch.bfloat16, context_lens=lens, seed=78, window=700,
                 rope=(500000.0, 2.0))
    _check(W.generate(w, poison=True), "rotary window 700")


@pytest.mark.parametrize("name", ["llama8b_b16_ragged_f16", "d96_b16_ragged_f16"])
def test_balanced_csr(name):
    p = W.generate(W.CONFIGS[name])
    csr = W.to_csr(p)
    ref_out, ref_lse = run_oracle(p)
    out, lse, plan = run_gpu_csr(p, csr, partition_size=BAL)
    assert plan["balanced_waves"] > 0
    compare(out, lse, ref_out, ref_lse, p.workload.dtype, "csr balanced %s" % name)


def test_balanced_token_major_cache():
    """[num_pages, page_size, Hkv, D] storage viewed as [num_pages, Hkv,
    page_size, D]: only the strides differ."""
    p = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    k = p.k_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = p.v_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    ref_out, ref_lse = run_oracle(p)
    out, lse, plan = run_gpu(dataclasses.replace(p, k_cache=k, v_cache=v), partition_size=BAL)
    assert plan["balanced_waves"] > 0
    compare(out, lse, ref_out, ref_lse, p.workload.dtype, "token-major balanced")


def test_balanced_garbage_workspace_then_smaller_batch():
    """The workspace starts as 0xFF bytes (NaN states, counts of -1); a call
    with 16 sequences, then one with 5 other sequences into the same
    workspace, both match the oracle."""
    big = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    small = W.generate(W.custom(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                dtype=torch.float16, context_lens=[2000, 0, 1, 700, 4096],
                                seed=91))
    eng = engine(big)
    need = eng.workspace_size(16, big.max_context_len, 0, BAL)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for p in (big, small):
        d = to_device(p)
        out = torch.empty_like(d.q)
        lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda")
        assert eng.workspace_size(p.workload.batch, p.max_context_len, 0, BAL) <= need
        args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                             out, lse, max_context_len=p.max_context_len, partition_size=BAL,
                             workspace=ws)
        eng.run_args(args)
        torch.cuda.synchronize()
        assert eng.last_plan().balanced_waves > 0
        ref_out, ref_lse = run_oracle(p)
        compare(out.cpu(), lse.cpu(), ref_out, ref_lse, torch.float16,
                "batch %d after garbage" % p.workload.batch)


def test_balanced_graph_replays_match_eager():
    p = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    d = to_device(p)
    eng = engine(p)
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda")
    args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale, out,
                         lse, max_context_len=p.max_context_len, partition_size=BAL)
    eng.run_args(args)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    ref_out, ref_lse = run_oracle(p)
    compare(eager[0].cpu(), eager[1].cpu(), ref_out, ref_lse, torch.float16, "eager balanced")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            eng.run_args(args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1]), "replay %d" % i
        eng.run_args(args)
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0])


def _draw(seed):
    r = random.Random(seed)
    D = r.choice([64, 96, 128, 256])
    dtype = r.choice([torch.float16, torch.bfloat16] + ([torch.float32] if D == 64 else []))
    hkv = r.choice([1, 2, 4, 8])
    G = r.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16])
    Bn = r.choice([1, 2, 3, 5, 8, 16, 33, 64])
    lens = []
    for _ in range(Bn):
        k = r.random()
        lens.append(0 if k < 0.1 else 1 if k < 0.2 else 16 * r.randint(1, 200) if k < 0.3
                    else r.randint(2, 6000))
    window = r.choice([0, 0, r.randint(1, 3000)])
    rope = None if r.random() < 0.7 else (r.choice([1e4, 5e5]), r.choice([1.0, 2.0]))
    return D, dtype, hkv, G, lens, window, rope


@pytest.mark.parametrize("seed", range(32))
def test_balanced_random_shape(seed):
    D, dtype, hkv, G, lens, window, rope = _draw(9100 + seed)
    w = W.custom(batch=len(lens), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D,
                 dtype=dtype, context_lens=lens, seed=9100 + seed, window=window, rope=rope)
    _check(W.generate(w), "seed %d: D=%d %s Hkv=%d G=%d B=%d window=%d rope=%s" % (
        seed, D, dtype, hkv, G, len(lens), window, rope))
