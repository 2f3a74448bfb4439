"""GPU parity of the rotary embedding (rotary_mode 1), needs an MI355X.

TVM PR #20426, section "Correctness", checks the kernel with `rotary_mode =
1`; the embedding is taken as the RoFormer rotation with the rotate-half
pairing (pairs (i, i + D/2), theta_i = rope_theta^(-2i/D) / rope_scale, key j
at position j, the query at n_b - 1).  The kernel turns each key by its
distance to the query and leaves q as it is; the oracle turns q and every
key to their own positions.  Both sides read the same seeded caches (keys
before the embedding); out and lse must meet the tolerances of helpers.py:
  * the rotary workloads at full size (3060 tokens, batch 16 ragged, 100,000
    tokens GQA-6 in 512-token partitions), in the launch configuration the
    benchmark times;
  * nine context lengths from 1 to 3060 for head_dim 64 / 96 / 128 / 256 in
    f16, bf16 and f32 (head_dim 96 pairs chunks of different lane groups);
  * forced partition sizes, several group sizes, rope_scale != 1 and other
    bases;
  * sliding windows deep into long contexts (positions near 100,000, where
    the angles need the f64 reduction);
  * the CSR page table (bitwise equal to the dense one), NaN in every slot
    the method must not read, and n = 1 (no turn at distance 0: exactly v0).
"""
import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_decode_amd import workloads as W

from helpers import compare, run_gpu, run_gpu_csr, run_oracle

pytestmark = pytest.mark.gpu


def _check(p, S=None, what=""):
    assert p.workload.rope is not None
    ref_out, ref_lse = run_oracle(p)
    out, lse, plan = run_gpu(p, partition_size=S)
    rel, lerr = compare(out, lse, ref_out, ref_lse, p.workload.dtype,
                        what="%s S=%s plan=%s" % (what, S, plan))
    print("%s S=%s plan(S=%d,P=%d,nw=%d,split=%d) rel_l2=%.3g lse_err=%.3g" %
          (what, S, plan["partition_size"], plan["num_partitions"], plan["waves_per_group"],
           plan["split"], rel, lerr), flush=True)
    return out, lse


@pytest.mark.parametrize("name", ["llama1b_ctx3060_rope_f16", "llama8b_b16_ragged_rope_f16",
                                  "ctx100k_gqa6_rope_f16"])
def test_rotary_workload_full_size(name):
    _check(W.generate(W.CONFIGS[name]), what=name)


@pytest.mark.parametrize("D,dtype", [(64, torch.float16), (96, torch.float16),
                                     (128, torch.float16), (256, torch.float16),
                                     (64, torch.bfloat16), (96, torch.bfloat16),
                                     (128, torch.bfloat16), (256, torch.bfloat16),
                                     (64, torch.float32)])
def test_rotary_nine_context_lengths(D, dtype):
    lens = [1, 2, 15, 16, 17, 255, 257, 1000, 3060]
    w = W.custom(batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=400 + D, num_pages=600, rope=(10000.0, 1.0))
    _check(W.generate(w), what="rope nine-lengths D=%d %s" % (D, dtype))


@pytest.mark.parametrize("S", [16, 48, 512, 4096])
def test_rotary_forced_partition_sizes(S):
    w = W.custom(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                 context_lens=[1, 3060, 777], seed=410, rope=(500000.0, 1.0))
    _check(W.generate(w), S=S, what="rope forced")


@pytest.mark.parametrize("G", [1, 3, 8, 16])
def test_rotary_group_sizes(G):
    for D, dtype in ((64, torch.float16), (96, torch.bfloat16), (128, torch.bfloat16)):
        w = W.custom(batch=2, num_q_heads=G * 2, num_kv_heads=2, head_dim=D, dtype=dtype,
                     context_lens=[333, 1200], seed=420 + G, rope=(10000.0, 1.0))
        _check(W.generate(w), what="rope G=%d D=%d" % (G, D))


@pytest.mark.parametrize("rope", [(100.0, 1.0), (10000.0, 4.0), (1000000.0, 0.5)])
def test_rotary_bases_and_scales(rope):
    w = W.custom(batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=torch.float16,
                 context_lens=[2049, 613], seed=430, rope=rope)
    _check(W.generate(w), what="rope %s" % (rope,))


@pytest.mark.parametrize("D,dtype", [(128, torch.float16), (256, torch.bfloat16),
                                     (96, torch.float16)])
def test_rotary_window_at_far_positions(D, dtype):
    """Windows deep into long contexts: keys near position 100,000, where an
    angle kept in f32 would be off by ~1e-2 rad."""
    lens = [100000, 70001, 5000]
    w = W.custom(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=440 + D, window=700, rope=(500000.0, 1.0),
                 num_pages=sum(-(-n // 16) for n in lens) + 8)
    _check(W.generate(w), what="rope far window D=%d" % D)


def test_rotary_csr_equals_dense_bitwise():
    """The CSR table gives the dense table's bits under the same schedule:
    the plan the CSR host picks (fixed partitions for these four sequences),
    the length-balanced schedule and forced fixed partitions, asked of both."""
    w = W.custom(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                 context_lens=[1, 17, 3060, 700], seed=450, rope=(500000.0, 1.0))
    p = W.generate(w)
    b_out, b_lse, b_plan = run_gpu_csr(p, W.to_csr(p))
    S = W.BALANCED if b_plan["balanced_waves"] > 0 else 0
    a_out, a_lse, a_plan = run_gpu(p, partition_size=S)
    assert a_plan == b_plan
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)
    for S in (W.BALANCED,):
        a = run_gpu(p, partition_size=S)
        c = run_gpu_csr(p, W.to_csr(p), partition_size=S)
        assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]) and a[2] == c[2], S
    for S in (64, 1024):
        a = run_gpu(p, partition_size=S)
        c = run_gpu_csr(p, W.to_csr(p), partition_size=S)
        assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]) and a[2] == c[2], S
    ref_out, ref_lse = run_oracle(p)
    compare(b_out, b_lse, ref_out, ref_lse, w.dtype, what="rope csr")


def test_rotary_never_reads_masked_slots():
    w = W.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                 context_lens=[5000, 33, 1], seed=460, window=1000, rope=(10000.0, 1.0))
    p = W.generate(w, poison=True)
    _check(p, what="rope poison")


def test_rotary_single_key_gives_exactly_v0():
    """n = 1: key and query share position 0; every angle is 0, the turn is
    the identity and out is exactly the key's value row."""
    w = W.custom(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=torch.float16,
                 context_lens=[1, 1], seed=470, rope=(500000.0, 1.0))
    p = W.generate(w, keep_logical=True)
    out, lse, _ = run_gpu(p)
    for b in range(2):
        for h in range(8):
            assert torch.equal(out[b, h], p.logical_v[b, 0, h // 4])
    ref_out, ref_lse = run_oracle(p)
    compare(out, lse, ref_out, ref_lse, w.dtype, what="rope n=1")


def test_rotary_changes_the_kernel_result():
    """Guards against a rotary switch that the kernel ignores."""
    w = W.custom(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[500], seed=480, rope=(10000.0, 1.0))
    p = W.generate(w)
    a_out, a_lse, _ = run_gpu(p)
    p0 = dataclasses.replace(p, workload=dataclasses.replace(w, rope=None))
    b_out, b_lse, _ = run_gpu(p0)
    assert float((a_lse - b_lse).abs().max()) > 1e-2


def test_rotary_token_major_cache_layout():
    """[num_pages, page_size, Hkv, D] storage (slot stride Hkv * D): the key
    rows reach the turn through the same tiles."""
    w = W.custom(batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=torch.bfloat16,
                 context_lens=[999, 1500], seed=490, rope=(500000.0, 1.0))
    p = W.generate(w)
    k = p.k_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = p.v_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert k.stride(2) == 4 * 128
    p2 = dataclasses.replace(p, k_cache=k, v_cache=v)
    ref_out, ref_lse = run_oracle(p)
    for S in (0, 64):
        out, lse, _ = run_gpu(p2, partition_size=S)
        compare(out, lse, ref_out, ref_lse, w.dtype, what="rope token-major S=%d" % S)



@pytest.mark.parametrize("name", ["llama8b_b16_ragged_rope_f16", "llama8b_ctx32k_rope_f16"])
def test_rotary_runs_are_bitwise_repeatable(name):
    """The same inputs give the same bits on every run (waves interleave
    differently from run to run, so a missing wait in the turned-key path
    would show up here as differing results)."""
    p = W.generate(W.CONFIGS[name])
    from helpers import to_device
    d = to_device(p)
    first = run_gpu(p, dev=d)
    for _ in range(6):
        again = run_gpu(p, dev=d)
        assert torch.equal(again[0], first[0]) and torch.equal(again[1], first[1])
