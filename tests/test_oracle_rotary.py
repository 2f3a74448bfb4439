"""Pins for the oracle's rotary embedding (rotary_mode 1), CPU only.

TVM PR #20426, section "Correctness", checks the sharded nest with
`rotary_mode = 1` but does not define it.  The reading the oracle takes: the
rotary embedding of the RoFormer paper with the rotate-half pairing of the
models the PR measures (Llama 3.x, Qwen3, Gemma 2): for i < D/2 the pair
(x[i], x[i + D/2]) of a vector at position pos turns by pos * theta_i,
theta_i = rope_theta^(-2i/D) / rope_scale; key j sits at position j and the
query at position n_b - 1.

Pinned against things other than the oracle's own formula:
  * hand-derived closed forms on head_dim 4 (they fix the turning direction,
    the pairing, the frequency exponent, the query position and the scaling);
  * a 50-digit mpmath brute force that applies the embedding in its complex
    form, (x[i] + i x[i + D/2]) * exp(i pos theta_i), on the logical K/V,
    including positions near 70,000 (reached through a sliding window);
  * invariants: shifting every position by the same amount leaves the result
    unchanged (the score depends on the distance only), a single key at
    position 0 is not turned, and the partitioned form and a shuffled page
    table give the direct result.
"""
import dataclasses
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_amd import workloads as W


def run(p, rope, **kw):
    return oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens, p.scale,
                         window=p.window, rotary=rope, **kw)


def _logical_problem(q, k, v, window=0, scale=1.0, page_size=2, seed=0):
    """One sequence from logical q [Hq, D], K and V [n, Hkv, D] (float32)."""
    n, Hkv, D = k.shape
    w = W.custom(batch=1, num_q_heads=q.shape[0], num_kv_heads=Hkv, head_dim=D,
                 dtype=torch.float32, context_lens=[n], window=window, page_size=page_size,
                 num_pages=n + 2, seed=seed)
    p = W.paginate(w, q[None].float(), k[None].float(), v[None].float(), [n],
                   torch.Generator().manual_seed(seed), poison=True)
    return dataclasses.replace(p, scale=float(scale))


def _softmax_expect(scores, values):
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = sum(e)
    out = [sum(ei * vi[d] for ei, vi in zip(e, values)) / z for d in range(len(values[0]))]
    return np.array(out), m + math.log(z)


# Hand derivations, head_dim 4, rope_theta 100: theta_0 = 100^0 = 1 and
# theta_1 = 100^(-2/4) = 0.1; pairs (0, 2) and (1, 3).
V2 = [[2.0, 0.0, -1.0, 4.0], [0.0, 1.0, 3.0, -2.0]]


@pytest.mark.parametrize("rope_scale", [1.0, 2.0])
def test_two_keys_closed_form(rope_scale):
    """n = 2, q = (1, 1, 0, 0) at position 1, K0 = (0, 0, 1, 1) at 0, K1 = q at 1.

    Turning q by the angles a0 = 1/c, a1 = 0.1/c (c = rope_scale) gives
    q' = (cos a0, cos a1, sin a0, sin a1); K0 at position 0 is unchanged, so
    s0 = sin a0 + sin a1; K1 at position 1 turns exactly like q, so s1 = |q|^2
    = 2.  The opposite direction would give s0 = -(sin a0 + sin a1); the
    interleaved pairing, the exponent -i/D, a query at position n, or
    multiplying by rope_scale would each change s0 or s1.
    """
    q = torch.tensor([[1.0, 1.0, 0.0, 0.0]])
    k = torch.tensor([[[0.0, 0.0, 1.0, 1.0]], [[1.0, 1.0, 0.0, 0.0]]])
    v = torch.tensor([[V2[0]], [V2[1]]])
    a0, a1 = 1.0 / rope_scale, 0.1 / rope_scale
    exp_out, exp_lse = _softmax_expect([math.sin(a0) + math.sin(a1), 2.0], V2)
    for ps in (1, 2, 3):
        p = _logical_problem(q, k, v, page_size=ps, seed=ps)
        out, lse = run(p, (100.0, rope_scale))
        np.testing.assert_allclose(out[0, 0], exp_out, rtol=1e-14, atol=1e-14)
        assert abs(lse[0, 0] - exp_lse) <= 1e-14


def test_window_and_query_position_closed_form():
    """n = 3, window 2: keys 1 and 2 are visible, q = (1, 0, 0, 0) at position 2.

    Relative to the query, key 1 sits at distance -1: K1 = (0, 0, 1, 0) turned
    by -1 in the (0, 2) plane becomes (sin 1, ., cos 1, .), so s1 = sin 1.  Key 2
    = (0, 0, 0, 1) sits at the query's position: s2 = q . K2 = 0.  Scale 0.5.
    Key 0 (score 10 before any turn) must not leak in.
    """
    q = torch.tensor([[1.0, 0.0, 0.0, 0.0]])
    k = torch.tensor([[[10.0, 0.0, 0.0, 0.0]], [[0.0, 0.0, 1.0, 0.0]], [[0.0, 0.0, 0.0, 1.0]]])
    vals = [[9.0, 9.0, 9.0, 9.0], V2[0], V2[1]]
    v = torch.tensor([[x] for x in vals])
    exp_out, exp_lse = _softmax_expect([0.5 * math.sin(1.0), 0.0], vals[1:])
    p = _logical_problem(q, k, v, window=2, scale=0.5)
    out, lse = run(p, (100.0, 1.0))
    np.testing.assert_allclose(out[0, 0], exp_out, rtol=1e-14, atol=1e-14)
    assert abs(lse[0, 0] - exp_lse) <= 1e-14


def test_single_key_is_not_turned():
    """n = 1: the key and the query both sit at position 0, where every angle
    is 0, so the result is the one without rotary: out = v0, lse = scale q.k0."""
    w = W.custom(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[1, 1], seed=21)
    p = W.generate(w)
    a = run(p, (10000.0, 1.0))
    b = run(p, None)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)


def brute_rope(q, lk, lv, lens, scale, window, G, theta, rscale):
    """50 digits: the embedding as complex multiplication on the logical K/V."""
    mpmath.mp.dps = 50
    B, Hq, D = q.shape
    h2 = D // 2
    freqs = [mpmath.mpf(theta) ** (mpmath.mpf(-2 * i) / D) / mpmath.mpf(rscale)
             for i in range(h2)]
    qd, kd, vd = q.double().numpy(), lk.double().numpy(), lv.double().numpy()

    def turned(x, pos):
        return [mpmath.mpc(x[i], x[i + h2]) * mpmath.expj(pos * freqs[i]) for i in range(h2)]

    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        n = lens[b]
        keys = [j for j in range(n) if window <= 0 or j >= n - window]
        for h in range(Hq):
            g = h // G
            if not keys:
                lse[b, h] = -math.inf
                continue
            zq = turned(qd[b, h], n - 1)
            s = []
            for j in keys:
                zk = turned(kd[b, j, g], j)
                # Re(zq * conj(zk)) is the dot product of the two 2-vectors.
                s.append(mpmath.mpf(scale) * mpmath.fsum(mpmath.re(a * mpmath.conj(c))
                                                         for a, c in zip(zq, zk)))
            z = mpmath.fsum(mpmath.exp(x) for x in s)
            for d in range(D):
                out[b, h, d] = float(mpmath.fsum(mpmath.exp(x) * mpmath.mpf(vd[b, j, g, d])
                                                 for x, j in zip(s, keys)) / z)
            lse[b, h] = float(mpmath.log(z))
    return out, lse


BRUTE_ROPE_CASES = [
    # (B, Hq, Hkv, D, dtype, lens, window, page_size, theta, rope_scale)
    (1, 2, 1, 8, torch.float32, [9], 0, 4, 10000.0, 1.0),
    (2, 4, 2, 16, torch.float16, [21, 3], 0, 4, 500000.0, 1.0),
    (2, 3, 1, 8, torch.bfloat16, [30, 0], 0, 4, 100.0, 4.0),
    (1, 4, 1, 8, torch.float32, [70001], 3, 16, 10000.0, 1.0),   # positions near 70,000
    (2, 2, 2, 6, torch.float16, [13, 33000], 4, 8, 1000000.0, 2.0),
]


@pytest.mark.parametrize("case", BRUTE_ROPE_CASES)
def test_rotary_matches_mpmath_complex_form(case):
    B, Hq, Hkv, D, dtype, lens, window, ps, theta, rscale = case
    w = W.custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                 context_lens=lens, seed=31 + D + len(lens), window=window, page_size=ps)
    p = W.generate(w, keep_logical=True)
    out, lse = run(p, (theta, rscale))
    bo, bl = brute_rope(p.q, p.logical_k, p.logical_v, lens, p.scale, window, Hq // Hkv,
                        theta, rscale)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = ~np.isinf(bl)
    # Angles near 70,000 rad: the float64 angle carries ~1e-11 rad of rounding,
    # which leaves ~1e-13 in out and lse.
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, bo, rtol=1e-11, atol=1e-12)


def test_shifting_every_position_changes_nothing():
    """Sequence 1 holds c unrelated keys and then sequence 0's n keys; with a
    window of n it sees the same keys, all c positions later, and the query
    moves by c too.  The rotary score depends on the distance only."""
    n, c, D = 200, 777, 128
    w = W.custom(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=torch.float16,
                 context_lens=[n], seed=22, rope=(500000.0, 1.0))
    p = W.generate(w, keep_logical=True)
    gen = torch.Generator().manual_seed(5)
    junk = torch.randn(1, c, 2, D, generator=gen).to(torch.float16)
    lk = torch.cat([junk, p.logical_k[:, :n]], dim=1)
    lv = torch.cat([junk, p.logical_v[:, :n]], dim=1)
    w2 = W.custom(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=D, dtype=torch.float16,
                  context_lens=[n + c], seed=0, window=n)
    p2 = dataclasses.replace(W.paginate(w2, p.q, lk, lv, [n + c], gen), scale=p.scale)
    a = run(p, w.rope)
    b = run(p2, w.rope)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-11, atol=1e-11)
    # ... while without the window the extra keys do change the result.
    w3 = dataclasses.replace(w2, window=0)
    d = run(dataclasses.replace(p2, workload=w3, window=0), w.rope)
    assert np.abs(d[1] - a[1]).max() > 1e-3


@pytest.mark.parametrize("S", [16, 48, 512])
def test_rotary_partitioned_form_gives_the_direct_result(S):
    w = W.custom(batch=3, num_q_heads=6, num_kv_heads=2, head_dim=32, dtype=torch.float16,
                 context_lens=[1, 700, 513], seed=23, window=400)
    p = W.generate(w)
    rope = (10000.0, 1.0)
    a = run(p, rope)
    b = oracle.decode_split(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens, p.scale,
                            S, window=p.window, rotary=rope)
    np.testing.assert_allclose(b[0], a[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-13)


def test_rotary_page_shuffle_is_bitwise_invariant():
    w = W.custom(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype=torch.bfloat16,
                 context_lens=[333, 90], seed=24)
    p = W.generate(w)
    rope = (500000.0, 1.0)
    a = run(p, rope)
    b = run(W.permute_pages(p, seed=7), rope)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rotary_changes_the_result():
    """Guards the pins above against a rotary switch that does nothing."""
    w = W.custom(batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype=torch.float16,
                 context_lens=[300], seed=25)
    p = W.generate(w)
    a = run(p, (10000.0, 1.0))
    b = run(p, None)
    assert np.abs(a[1] - b[1]).max() > 1e-2


def test_invalid_rotary_parameters_are_rejected():
    p = W.generate(W.custom(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=8,
                            dtype=torch.float32, context_lens=[5], seed=26))
    for rope in ((0.0, 1.0), (10000.0, 0.0), (-1.0, 1.0), (float("nan"), 1.0)):
        with pytest.raises(ValueError):
            run(p, rope)
