"""GPU parity: the HIP path against the float64 oracle (needs an MI355X).

Every case draws seeded inputs, runs pa_decode_run through the C ABI and
compares out (relative L2 against the oracle rounded to the output dtype) and
lse (absolute error) with the tolerances in helpers.py.  Covered:
  * the five workloads at full size (tiny GQA-4 fp32; Llama-3.2-1B-shaped
    batch-1 at 3060 tokens; Llama-3.1-8B-shaped batch 16 with ragged lengths
    including 1, 17 and 4096; head_dim 256 bf16 with a 4096-token sliding
    window; 100,000 tokens GQA-6 cut into 196 partitions of 512) in the
    launch configuration the benchmark times;
  * nine context lengths from 1 to 3060 with a shuffled page table, for
    head_dim 64 / 96 / 128 / 256 (TVM PR #20426, section "Correctness", checks
    nine lengths in that range with a shuffled table; its "Tests" lay out
    D = 96 too);
  * forced partition sizes (16 ... 1024 tokens) and the unsplit path;
  * the ragged batches with fixed partitions too (their workloads use the
    length-balanced schedule, covered in test_gpu_balanced.py);
  * every built group size G in 1..16;
  * NaN in every slot the method must not read (tail slots, keys before the
    window, unused pages, page-table padding);
  * an empty context in a batch (out = 0, lse = -inf) and batch 0;
  * a token-major cache layout [num_pages, page_size, Hkv, D];
  * bitwise invariants: physical page shuffling, run-to-run repeatability,
    n = 1 giving exactly v0.
"""
import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

from helpers import compare, engine, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _check(p, S=None, what=""):
    ref_out, ref_lse = run_oracle(p)
    out, lse, plan = run_gpu(p, partition_size=S)
    rel, lerr = compare(out, lse, ref_out, ref_lse, p.workload.dtype,
                        what="%s S=%s plan=%s" % (what, S, plan))
    print("%s S=%s plan(S=%d,P=%d,nw=%d,split=%d) rel_l2=%.3g lse_err=%.3g" %
          (what, S, plan["partition_size"], plan["num_partitions"], plan["waves_per_group"],
           plan["split"], rel, lerr), flush=True)
    return out, lse


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_workload_full_size(name):
    p = W.generate(W.CONFIGS[name])
    _check(p, what=name)


@pytest.mark.parametrize("name", ["llama8b_b16_ragged_f16", "d96_b16_ragged_f16",
                                  "llama8b_b16_ragged_rope_f16"])
def test_ragged_workloads_with_fixed_partitions(name):
    """The ragged batches run with the balanced schedule by default; here
    with the planner's fixed partitions."""
    p = W.generate(W.CONFIGS[name])
    _check(p, S=0, what=name + " fixed")


@pytest.mark.parametrize("D,dtype", [(64, torch.float16), (96, torch.float16), (128, torch.float16),
                                     (96, torch.bfloat16), (256, torch.bfloat16),
                                     (64, torch.float32)])
def test_nine_context_lengths_shuffled_pages(D, dtype):
    lens = [1, 2, 15, 16, 17, 255, 257, 1000, 3060]
    G = 4
    w = W.custom(batch=len(lens), num_q_heads=8, num_kv_heads=8 // G, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=100 + D, num_pages=600)
    _check(W.generate(w), what="nine-lengths D=%d %s" % (D, dtype))


@pytest.mark.parametrize("S", [16, 32, 48, 64, 128, 512, 1024, 4096])
def test_forced_partition_sizes(S):
    w = W.custom(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                 context_lens=[1, 3060, 777], seed=200)
    _check(W.generate(w), S=S, what="forced")


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16])
def test_every_group_size(G):
    Hkv = 2
    for D, dtype in ((64, torch.float16), (96, torch.bfloat16), (256, torch.bfloat16)):
        w = W.custom(batch=2, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                     context_lens=[333, 1200], seed=300 + G)
        _check(W.generate(w), what="G=%d D=%d" % (G, D))


@pytest.mark.parametrize("S", [16, 64, 256, 4096])
def test_head_dim_96_partitions_and_merges(S):
    """head_dim 96: 12-chunk rows through the padded LDS tiles; S = 16
    gives more than 64 partitions (workgroup merge with a partial 64-column
    slice), the others the wave merge or the unsplit path; NaN in every
    slot the method must not read."""
    w = W.custom(batch=3, num_q_heads=12, num_kv_heads=4, head_dim=96, dtype=torch.float16,
                 context_lens=[1, 2000, 777], seed=250)
    _check(W.generate(w, poison=True, extra_pages=2), S=S, what="D96")


@pytest.mark.parametrize("name", W.CONFIG_ORDER[:4])
def test_poisoned_unread_slots(name):
    w = W.CONFIGS[name]
    if name == "d256_window4096_bf16":
        w = dataclasses.replace(w, context_lens=[8192, 5000, 4097, 333], window=4096,
                                num_pages=2048)
    p = W.generate(w, poison=True, extra_pages=3)
    for S in (0, 16, 64):
        _check(p, S=S, what="poison " + name)


def test_window_edges():
    for Wn in (1, 15, 16, 17, 100, 4095):
        w = W.custom(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=256, dtype=torch.bfloat16,
                     context_lens=[5000, Wn, Wn + 1], seed=400, window=Wn)
        p = W.generate(w, poison=True)
        for S in (0, 32, 512):
            _check(p, S=S, what="window %d" % Wn)


def test_empty_context_and_empty_batch():
    w = W.custom(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=torch.float16,
                 context_lens=[0, 5, 0, 2000], seed=500)
    p = W.generate(w)
    for S in (0, 16, 4096):
        out, lse = _check(p, S=S, what="empty")
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    # batch 0: nothing to do, but still a valid call
    eng = engine(p)
    d = to_device(p)
    out = torch.empty((0, 8, 128), dtype=torch.float16, device="cuda")
    args = eng.make_args(d.q[:0], d.k_cache, d.v_cache, d.page_table[:0], d.context_lens[:0],
                         p.scale, out, None, max_context_len=0)
    eng.run_args(args)
    torch.cuda.synchronize()


def test_token_major_cache_layout():
    w = W.custom(batch=2, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=torch.float16,
                 context_lens=[999, 1500], seed=600)
    p = W.generate(w)
    # [num_pages, ps, Hkv, D] storage viewed as [num_pages, Hkv, ps, D]
    k = p.k_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = p.v_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert k.stride(2) == 4 * 128
    p2 = dataclasses.replace(p, k_cache=k, v_cache=v)
    ref = run_oracle(p)
    for S in (0, 64):
        out, lse, _ = run_gpu(p2, partition_size=S)
        compare(out, lse, ref[0], ref[1], torch.float16, "token-major")


def test_bitwise_page_shuffle_and_repeatability():
    p = W.generate(W.CONFIGS["llama1b_ctx3060_f16"])
    a = run_gpu(p)
    b = run_gpu(p)
    c = run_gpu(W.permute_pages(p, seed=77))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


def test_single_key_is_exactly_v0():
    w = W.custom(batch=3, num_q_heads=24, num_kv_heads=4, head_dim=256, dtype=torch.float16,
                 context_lens=[1, 1, 1], seed=700)
    p = W.generate(w, keep_logical=True)
    for S in (0, 16):
        out, lse, _ = run_gpu(p, partition_size=S)
        for h in range(24):
            assert torch.equal(out[:, h], p.logical_v[:, 0, h // 6])
        ref = run_oracle(p)
        assert np.abs(lse.double().numpy() - ref[1]).max() <= 1e-5


def test_workspace_too_small_is_reported():
    p = W.generate(W.CONFIGS["llama1b_ctx3060_f16"])
    d = to_device(p)
    eng = engine(p)
    out = torch.empty_like(d.q)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale, out,
                         None, max_context_len=3060, partition_size=16, workspace=small)
    with pytest.raises(B.PaDecodeError) as e:
        eng.run_args(args)
    assert e.value.status == B.PA_DECODE_WORKSPACE_TOO_SMALL


def test_repeated_calls_reuse_the_workspace():
    """Many calls with different plans on one workspace: each is right, and a
    repeated plan gives identical bits."""
    w = W.CONFIGS["llama8b_b16_ragged_f16"]
    p = W.generate(w)
    d = to_device(p)
    eng = engine(p)
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda")
    results = []
    for S in (0, 64, 0, 1024, 16, 0):
        args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale,
                             out, lse, max_context_len=p.max_context_len, partition_size=S)
        for _ in range(3):
            eng.run_args(args)
        torch.cuda.synchronize()
        results.append((S, out.cpu(), lse.cpu()))
    ref = run_oracle(p)
    for S, o, l in results:
        compare(o, l, ref[0], ref[1], w.dtype, "repeat S=%d" % S)
    base = [r for r in results if r[0] == 0]
    for _, o, l in base[1:]:
        assert torch.equal(o, base[0][1]) and torch.equal(l, base[0][2])


@pytest.mark.parametrize("name", ["llama1b_ctx3060_f16", "ctx100k_gqa6_f16",
                                  "llama1b_ctx3060_rope_f16", "llama8b_b16_ragged_rope_f16"])
def test_graph_replays_match_eager(name):
    """Captured steps replayed several times, with eager work and syncs between
    replays, give the eager result every time."""
    p = W.generate(W.CONFIGS[name])
    d = to_device(p)
    eng = engine(p)
    out = torch.empty_like(d.q)
    lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda")
    args = eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale, out,
                         lse, max_context_len=p.max_context_len,
                         partition_size=p.workload.partition_size)
    eng.run_args(args)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            eng.run_args(args, torch.cuda.current_stream().cuda_stream)
            eng.run_args(args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1]), "replay %d" % i
        eng.run_args(args)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0])


def test_layer_stacked_step_under_one_graph():
    """A decode step over L layers (distinct KV caches and queries, one shared
    page table, as in a model's stack) captured as one graph of L back-to-back
    calls: every layer's output equals the oracle's on every replay (the
    pages measure attention time per decode step summed over 16-32 layers,
    TVM PR #20426, "Measurements")."""
    base = W.CONFIGS["llama1b_ctx3060_f16"]
    L = 4
    layers = [W.generate(dataclasses.replace(base, seed=1000 + l)) for l in range(L)]
    pt = layers[0].page_table
    layers = [dataclasses.replace(p, page_table=pt) for p in layers]   # one shared table
    eng = engine(layers[0])
    dev = [to_device(p) for p in layers]
    outs = [torch.empty_like(d.q) for d in dev]
    lses = [torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda") for d in dev]
    args = [eng.make_args(d.q, d.k_cache, d.v_cache, d.page_table, d.context_lens, p.scale, o, ls,
                          max_context_len=p.max_context_len,
                          workspace=torch.zeros(1 << 22, dtype=torch.uint8, device="cuda"))
            for p, d, o, ls in zip(layers, dev, outs, lses)]
    refs = [run_oracle(p) for p in layers]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for a in args:
                eng.run_args(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o, ls in zip(outs, lses):
            o.zero_()
            ls.zero_()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            compare(outs[l].cpu(), lses[l].cpu(), refs[l][0], refs[l][1], base.dtype,
                    "layer %d replay %d" % (l, rep))


@pytest.mark.parametrize("rope", [None, (500000.0, 1.0)])
@pytest.mark.parametrize("window", [300, 0])
def test_million_token_context(window, rope):
    """One sequence of 1,000,000 tokens: page ids up to 62,500, 253
    partitions for the workgroup merge without a window, and, with rotary,
    angles at positions near 10^6."""
    n = 1_000_000
    w = W.custom(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype=torch.float16,
                 context_lens=[n], seed=610, window=window, rope=rope, num_pages=n // 16 + 4)
    _check(W.generate(w), what="1M tokens, window %d, rope=%s" % (window, rope))


def test_batch_of_512_short_ragged_sequences():
    """A wide grid (512 sequences x 8 KV heads) of short, ragged contexts,
    empty ones included."""
    gen = torch.Generator().manual_seed(611)
    lens = torch.randint(0, 300, (512,), generator=gen).tolist()
    lens[0], lens[1], lens[2] = 0, 1, 299
    w = W.custom(batch=512, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                 context_lens=lens, seed=612)
    _check(W.generate(w), what="batch 512")


@pytest.mark.parametrize("scale", [0.0, 1e-4, -0.5, 2.0, 8.0])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_extreme_score_scales(scale, dtype):
    """Score ranges from flat (scale 0: out = mean of V, lse = ln n) to very
    peaked (scale 8 on N(0,1) data: scores up to ~300 apart, so the softmax
    reference value jumps many times), negative scale included; several
    partitions and a ragged tail.  The lse bound grows with |lse| (1e-4 +
    1e-6 |lse|): at |lse| ~ 400 float32 spacing alone is 3e-5, and a float32
    q.k over 128 terms of size ~8 carries ~1e-5 absolute error before the
    scale multiplies it."""
    w = W.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=dtype,
                 context_lens=[3001, 517, 64], seed=620)
    p = dataclasses.replace(W.generate(w), scale=scale)
    ref_out, ref_lse = run_oracle(p)
    for S in (None, 128):
        out, lse, plan = run_gpu(p, partition_size=S)
        rel, lerr = compare(out, lse, ref_out, ref_lse, dtype, "scale %g S=%s" % (scale, S),
                            lse_rel=1e-6)
        print("scale %g %s S=%s rel_l2=%.3g lse_err=%.3g" % (scale, dtype, S, rel, lerr),
              flush=True)


def test_batch_permutation_permutes_outputs_bitwise():
    """Sequences are independent: reordering the batch (q rows, page-table
    rows, lengths) reorders out and lse, bit for bit, under fixed partitions
    (whose plan depends only on the batch size and the longest context,
    which do not change; the balanced schedule's split points follow the
    order of the lengths, so there the rounding may differ)."""
    p = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    out, lse, plan = run_gpu(p, partition_size=0)
    perm = torch.randperm(p.q.shape[0], generator=torch.Generator().manual_seed(621))
    pp = dataclasses.replace(p, q=p.q[perm].contiguous(), page_table=p.page_table[perm].contiguous(),
                             context_lens=p.context_lens[perm].contiguous())
    out2, lse2, plan2 = run_gpu(pp, partition_size=0)
    assert plan2 == plan
    assert torch.equal(out2, out[perm]) and torch.equal(lse2, lse[perm])


def test_aliased_pages_in_the_dense_table():
    """Two sequences whose page-table rows point at the same physical pages
    (a shared prefix) read them independently; both match the oracle."""
    w = W.custom(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=64, dtype=torch.float16,
                 context_lens=[900, 900, 400], seed=622)
    p = W.generate(w)
    pt = p.page_table.clone()
    pt[1, :40] = pt[0, :40]          # 640 shared tokens, then its own pages
    pt[2, :25] = pt[0, :25]          # the whole of sequence 2 is a prefix of sequence 0
    _check(dataclasses.replace(p, page_table=pt), what="aliased pages")


def test_windowed_batch8_full_size():
    """The windowed head_dim-256 shape at batch 8, whose partitions the
    planner sizes with one to spare for an unaligned window start (640
    tokens, 8 partitions), at full size against the oracle."""
    p = W.generate(W.CONFIGS["d256_window4096_b8_bf16"])
    _check(p, what="d256 window batch 8")


@pytest.mark.parametrize("D,dtype,hkv,G,lens,window", [
    (64, torch.float16, 1, 8, [32768] * 3, 0),                      # S 448, 222 workgroups
    (128, torch.float16, 2, 4, [16384, 9000, 16384, 1, 16384, 12345], 0),
    (128, torch.bfloat16, 8, 4, [8192, 8192, 7000, 8192], 4096),     # S 640, 256 workgroups
    (96, torch.float16, 8, 2, [25314, 100, 20000, 25314, 17], 0),
])
def test_layouts_of_the_grid_rule(D, dtype, hkv, G, lens, window):
    """Shapes where the planner takes more pages per wave than its first
    count so that the grid stays within one workgroup per compute unit: the
    partitions it then draws still give the oracle's result."""
    w = W.custom(batch=len(lens), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=940 + D + hkv, window=window)
    _check(W.generate(w), what="grid rule D=%d hkv=%d B=%d" % (D, hkv, len(lens)))


def test_head_dim_256_two_partitions_per_workgroup():
    """head_dim 256, a fixed partition size whose partitions the planner
    packs two to a workgroup with two waves each: the oracle's result."""
    w = W.custom(batch=4, num_q_heads=8, num_kv_heads=4, head_dim=256, dtype=torch.bfloat16,
                 context_lens=[8192, 8000, 8192, 5000], seed=961)
    _check(W.generate(w), S=496, what="d256 fixed S 496")
