"""Pins for the float64 CPU oracle (CPU only).

The oracle is checked against things other than itself:
  * a 50-digit mpmath brute force that reads the *logical* K/V (it never sees the
    page table), on tiny random problems with and without a sliding window;
  * hand-derived closed-form cases stored in tests/golden/closed_forms.json;
  * closed forms stated for the method: n = 1 gives out = v0 and lse = scale q.k0;
    equal keys give the mean of V and lse = s + ln n; q = 0 gives the mean of V
    and ln n; constant V gives that constant; a dominant key selects its value;
  * the textbook special case: with an identity page table the result is
    scaled-dot-product attention (torch, float64) and torch.logsumexp;
  * invariants: physical page shuffling (bitwise), every partition size of the
    partitioned form, GQA == MHA with duplicated KV heads (bitwise), batch
    permutation (bitwise), sliding window == truncated context, V -> -2V;
  * the f16 / bf16 decoders, exhaustively against numpy / torch.
Definition followed (TVM PR #20426, section "Correctness"; the
paged_attention_v2_pytorch.py commit page, "Phase 1"/"Phase 2" and the
[kv_h, gqa] head reshape): out = softmax(scale q K^T) V, lse = ln sum exp(scale q K^T),
query head h reads KV head floor(h / (Hq / Hkv)).
"""
import dataclasses
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def run(p, **kw):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens, p.scale,
                         window=p.window, **kw)


def run_split(p, S):
    return oracle.decode_split(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens,
                               p.scale, S, window=p.window)


def brute(q, lk, lv, lens, scale, window, G):
    """50-digit softmax attention over the logical (un-paged) K/V."""
    mpmath.mp.dps = 50
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    qd, kd, vd = q.double().numpy(), lk.double().numpy(), lv.double().numpy()
    for b in range(B):
        n = lens[b]
        keys = [j for j in range(n) if window <= 0 or j >= n - window]
        for h in range(Hq):
            g = h // G
            if not keys:
                lse[b, h] = -math.inf
                continue
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(qd[b, h, d]) * mpmath.mpf(kd[b, j, g, d])
                                                 for d in range(D)) for j in keys]
            z = mpmath.fsum(mpmath.exp(x) for x in s)
            for d in range(D):
                out[b, h, d] = float(mpmath.fsum(mpmath.exp(x) * mpmath.mpf(vd[b, j, g, d])
                                                 for x, j in zip(s, keys)) / z)
            lse[b, h] = float(mpmath.log(z))
    return out, lse


BRUTE_CASES = [
    # (B, Hq, Hkv, D, dtype, lens, window, page_size)
    (1, 1, 1, 4, torch.float32, [1], 0, 4),
    (1, 2, 1, 8, torch.float32, [9], 0, 4),
    (2, 3, 1, 16, torch.float16, [17, 5], 0, 4),
    (3, 4, 2, 8, torch.bfloat16, [40, 1, 23], 0, 4),
    (2, 6, 2, 16, torch.float32, [33, 12], 7, 4),
    (2, 2, 2, 4, torch.float16, [0, 13], 0, 4),
    (1, 6, 3, 8, torch.float32, [31], 16, 8),
    (2, 4, 4, 8, torch.bfloat16, [3, 37], 3, 2),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_mpmath_brute_force(case):
    B, Hq, Hkv, D, dtype, lens, window, ps = case
    w = W.custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=11 + len(lens) + D, window=window, page_size=ps,
                 num_pages=sum((n + ps - 1) // ps for n in lens) + 3)
    p = W.generate(w, keep_logical=True)
    out, lse = run(p)
    bo, bl = brute(p.q, p.logical_k, p.logical_v, lens, p.scale, window, Hq // Hkv)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = ~np.isinf(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)


def _golden_problem(c, page_size=2, seed=0):
    n = len(c["k"])
    w = W.custom(batch=1, num_q_heads=c["num_q_heads"], num_kv_heads=c["num_kv_heads"],
                 head_dim=c["head_dim"], dtype=torch.float32, context_lens=[n],
                 window=c["window"], page_size=page_size, num_pages=n + 2, seed=seed)
    q = torch.tensor([c["q"]], dtype=torch.float32)
    lk = torch.tensor([c["k"]], dtype=torch.float32)
    lv = torch.tensor([c["v"]], dtype=torch.float32)
    gen = torch.Generator().manual_seed(seed)
    p = W.paginate(w, q, lk, lv, [n], gen, poison=True)
    return dataclasses.replace(p, scale=float(c["scale"]))


@pytest.mark.parametrize("name", [c["name"] for c in json.load(open(GOLDEN))["cases"]])
def test_oracle_matches_hand_derived_cases(name):
    c = [c for c in json.load(open(GOLDEN))["cases"] if c["name"] == name][0]
    for ps in (1, 2, 3):
        p = _golden_problem(c, page_size=ps, seed=ps)
        out, lse = run(p)
        np.testing.assert_allclose(out[0], np.array(c["out"]), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[0], np.array(c["lse"]), rtol=1e-14, atol=1e-14)


def test_single_key_gives_v0_and_its_score():
    w = W.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[1, 1, 1], seed=3)
    p = W.generate(w, keep_logical=True)
    out, lse = run(p)
    for b in range(3):
        for h in range(8):
            g = h // 4
            v0 = p.logical_v[b, 0, g].double().numpy()
            assert np.array_equal(out[b, h], v0)  # exactly v0
            s0 = p.scale * float(np.dot(p.q[b, h].double().numpy(),
                                        p.logical_k[b, 0, g].double().numpy()))
            assert abs(lse[b, h] - s0) <= 1e-14 * max(1.0, abs(s0))


def test_equal_keys_give_mean_v_and_log_n():
    n = 37
    w = W.custom(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype=torch.float32,
                 context_lens=[n], seed=5)
    p = W.generate(w, keep_logical=True)
    lk = p.logical_k.clone()
    lk[:, :] = lk[:, :1]  # every key equals key 0
    gen = torch.Generator().manual_seed(9)
    p2 = W.paginate(w, p.q, lk, p.logical_v, [n], gen)
    out, lse = run(p2)
    for h in range(4):
        g = h // 2
        s = p.scale * float(np.dot(p.q[0, h].double().numpy(), lk[0, 0, g].double().numpy()))
        np.testing.assert_allclose(out[0, h], p.logical_v[0, :n, g].double().mean(0).numpy(),
                                   rtol=1e-13, atol=1e-14)
        assert abs(lse[0, h] - (s + math.log(n))) <= 1e-13


def test_zero_query_gives_mean_v_and_log_n():
    n = 50
    w = W.custom(batch=1, num_q_heads=3, num_kv_heads=1, head_dim=32, dtype=torch.bfloat16,
                 context_lens=[n], seed=6)
    p = W.generate(w, keep_logical=True)
    p = dataclasses.replace(p, q=torch.zeros_like(p.q))
    out, lse = run(p)
    mean_v = p.logical_v[0, :n, 0].double().mean(0).numpy()
    for h in range(3):
        np.testing.assert_allclose(out[0, h], mean_v, rtol=1e-13, atol=1e-14)
        assert abs(lse[0, h] - math.log(n)) <= 1e-14


def test_constant_v_gives_the_constant():
    w = W.custom(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=8, dtype=torch.float32,
                 context_lens=[29, 64], seed=7)
    p = W.generate(w, keep_logical=True)
    c = torch.arange(8, dtype=torch.float32) * 0.5 - 1.0
    lv = torch.zeros_like(p.logical_v) + c
    p2 = W.paginate(w, p.q, p.logical_k, lv, [29, 64], torch.Generator().manual_seed(1))
    out, _ = run(p2)
    np.testing.assert_allclose(out, np.broadcast_to(c.double().numpy(), out.shape),
                               rtol=1e-14, atol=1e-14)


def test_dominant_key_selects_its_value():
    n, D = 40, 16
    w = W.custom(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=D, dtype=torch.float32,
                 context_lens=[n], seed=8)
    p = W.generate(w, keep_logical=True)
    lk = p.logical_k.clone() * 0.01
    t = 17
    lk[0, t, 0] = p.q[0, 0] * (100.0 / (p.scale * float(p.q[0, 0].double().pow(2).sum())))
    p2 = W.paginate(w, p.q, lk, p.logical_v, [n], torch.Generator().manual_seed(2))
    out, _ = run(p2)
    np.testing.assert_allclose(out[0, 0], p.logical_v[0, t, 0].double().numpy(),
                               rtol=0, atol=1e-20 + 1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_identity_page_table_is_textbook_sdpa(dtype):
    B, Hq, Hkv, D, n, ps = 2, 8, 2, 64, 333, 16
    w = W.custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                 context_lens=[n, n], seed=12)
    p = W.generate(w, keep_logical=True)
    out, lse = run(p)
    G = Hq // Hkv
    q = p.q.double()[:, :, None, :]                                   # [B, Hq, 1, D]
    k = p.logical_k.double().permute(0, 2, 1, 3).repeat_interleave(G, dim=1)  # [B,Hq,n,D]
    v = p.logical_v.double().permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=p.scale)[:, :, 0]
    ref_lse = torch.logsumexp(p.scale * (q @ k.transpose(-1, -2))[:, :, 0], dim=-1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-13, atol=1e-13)


def test_page_shuffle_is_bitwise_invariant():
    for name in ("tiny_gqa4_f32", "llama1b_ctx3060_f16"):
        p = W.generate(W.CONFIGS[name])
        a = run(p)
        b = run(W.permute_pages(p, seed=123))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("S", [1, 16, 32, 48, 64, 100, 512, 4096])
def test_every_partition_size_gives_the_direct_result(S):
    w = W.custom(batch=3, num_q_heads=6, num_kv_heads=2, head_dim=32, dtype=torch.float16,
                 context_lens=[1, 700, 513], seed=13, window=0)
    p = W.generate(w)
    a = run(p)
    b = run_split(p, S)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("S", [16, 48, 512])
def test_partition_sizes_with_window(S):
    w = W.custom(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype=torch.float32,
                 context_lens=[900, 70], seed=14, window=333)
    p = W.generate(w)
    a = run(p)
    b = run_split(p, S)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-13)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    p = W.generate(W.CONFIGS["tiny_gqa4_f32"])
    G = p.workload.gqa
    w2 = dataclasses.replace(p.workload, num_kv_heads=p.workload.num_q_heads)
    p2 = dataclasses.replace(p, workload=w2,
                             k_cache=p.k_cache.repeat_interleave(G, dim=1).contiguous(),
                             v_cache=p.v_cache.repeat_interleave(G, dim=1).contiguous())
    a, b = run(p), run(p2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_batch_permutation_permutes_outputs():
    w = W.custom(batch=4, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype=torch.float16,
                 context_lens=[5, 80, 33, 1], seed=15)
    p = W.generate(w)
    perm = torch.tensor([2, 0, 3, 1])
    p2 = dataclasses.replace(p, q=p.q[perm].contiguous(), page_table=p.page_table[perm].contiguous(),
                             context_lens=p.context_lens[perm].contiguous())
    a, b = run(p), run(p2)
    assert np.array_equal(a[0][perm.numpy()], b[0]) and np.array_equal(a[1][perm.numpy()], b[1])


def test_window_equals_truncated_context():
    n, Wn = 300, 77
    w = W.custom(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=16, dtype=torch.float32,
                 context_lens=[n], seed=16, window=Wn)
    p = W.generate(w, keep_logical=True)
    a = run(p)
    w2 = W.custom(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=16, dtype=torch.float32,
                  context_lens=[Wn], seed=0)
    p2 = W.paginate(w2, p.q, p.logical_k[:, n - Wn:].contiguous(),
                    p.logical_v[:, n - Wn:].contiguous(), [Wn], torch.Generator().manual_seed(3))
    p2 = dataclasses.replace(p2, scale=p.scale)
    b = run(p2)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14, atol=1e-15)
    # window >= n means no masking
    w3 = dataclasses.replace(p.workload, window=n)
    c = run(dataclasses.replace(p, workload=w3, window=n))
    d = run(dataclasses.replace(p, window=0))
    assert np.array_equal(c[0], d[0])


def test_output_is_linear_in_v():
    p = W.generate(W.CONFIGS["tiny_gqa4_f32"])
    a = run(p)
    b = run(dataclasses.replace(p, v_cache=p.v_cache * -2.0))
    np.testing.assert_allclose(b[0], -2.0 * a[0], rtol=1e-14, atol=1e-14)
    assert np.array_equal(a[1], b[1])


def test_empty_context_gives_zero_and_minus_inf():
    w = W.custom(batch=2, num_q_heads=2, num_kv_heads=1, head_dim=8, dtype=torch.float32,
                 context_lens=[0, 5], seed=17)
    p = W.generate(w)
    out, lse = run(p)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_poisoned_slots_are_never_read():
    for name in ("tiny_gqa4_f32", "d256_window4096_bf16"):
        w = W.CONFIGS[name]
        if name.startswith("d256"):
            w = dataclasses.replace(w, batch=1, context_lens=[1000], window=333, num_pages=70)
        a = run(W.generate(w))
        b = run(W.generate(w, poison=True))
        assert np.all(np.isfinite(b[0]))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_f16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_exhaustive():
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(b) & 0xFFFF) for b in bits.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_invalid_page_id_is_rejected_not_read():
    p = W.generate(W.CONFIGS["tiny_gqa4_f32"])
    pt = p.page_table.clone()
    pt[0, 3] = p.k_cache.shape[0]
    with pytest.raises(ValueError):
        run(dataclasses.replace(p, page_table=pt))
