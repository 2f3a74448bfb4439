"""CPU checks of the output comparison itself (tests/parity.py).

The oracle's own result on the batch-16 ragged workload (lengths 1 .. 4096)
stands in for a GPU output; planted errors must be caught by the per-row
bound even where the whole-tensor rel-L2 lets them through, and rounding the
exact result either way (one output ulp) must not be counted.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from paged_kv_decode_amd import workloads as W


@pytest.fixture(scope="module")
def ragged():
    p = W.generate(W.CONFIGS["llama8b_b16_ragged_f16"])
    out, lse = oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens, p.scale)
    return p, out, lse


def test_ulp_matches_the_dtype_spacing():
    x = torch.tensor([1.0, 1.5, 2.0, 3.0, 1e-3, 65504.0, 2.0 ** -20, 0.0], dtype=torch.float64)
    for dt in (torch.float16, torch.bfloat16, torch.float32):
        u = parity.ulp(x.numpy(), dt)
        v = x.to(dt)
        up = torch.nextafter(v.float(), torch.tensor(float("inf"))) if dt == torch.float32 else None
        for i in range(len(x)):
            if dt == torch.float32:
                assert u[i] == (up[i].double() - v[i].double()).item() or x[i] == 0
            else:
                # v + u is the next representable value above v (not past the range)
                if abs(x[i].item()) < 60000 and x[i] != 0:
                    nxt = torch.tensor(v[i].double().item() + u[i], dtype=torch.float64).to(dt)
                    assert nxt.double().item() == v[i].double().item() + u[i]
                    half = torch.tensor(v[i].double().item() + u[i] / 4, dtype=torch.float64).to(dt)
                    assert half.double().item() == v[i].double().item()
    assert parity.ulp(np.array([0.0]), torch.float16)[0] == 2.0 ** -24


def test_exact_and_rounded_results_pass(ragged):
    p, out, _ = ragged
    g = torch.from_numpy(out).to(torch.float16)
    e = parity.out_errors(g, out, torch.float16)
    assert e["rel_l2"] == 0.0 and e["row_excess"] == 0.0


def test_one_ulp_flips_are_not_counted(ragged):
    """Every element moved to the other neighbouring dtype value of the exact
    result: rel-L2 against the rounded oracle grows, the per-row excess does
    not."""
    p, out, _ = ragged
    for dt in (torch.float16, torch.bfloat16):
        r = torch.from_numpy(out)
        v = r.to(dt).double()
        u = torch.from_numpy(parity.ulp(out, dt))
        other = torch.where(r >= v, v + u, v - u).to(dt)   # the far neighbour of r
        e = parity.out_errors(other, out, dt)
        assert e["row_excess"] == 0.0, e
        assert e["row_rel_l2_max"] > 0.0


def test_error_confined_to_the_longest_sequence_is_caught(ragged):
    """A 4% error on the 4096-token sequence (b = 1) passes the whole-tensor
    rel-L2 but not the per-row bound."""
    p, out, _ = ragged
    bad = out.copy()
    bad[1] *= 1.04
    g = torch.from_numpy(bad).to(torch.float16)
    e = parity.out_errors(g, out, torch.float16)
    assert e["rel_l2"] <= 1e-3          # within the whole-tensor bound
    assert e["row_excess"] > 0.03
    assert e["row_worst"] // p.q.shape[1] == 1


def test_small_error_on_every_long_sequence_is_caught(ragged):
    """0.93% on every sequence longer than 1000 tokens (the split / merge
    paths) passes the whole-tensor rel-L2 but not the per-row bound."""
    p, out, _ = ragged
    bad = out.copy()
    long_rows = [b for b, n in enumerate(p.context_lens.tolist()) if n > 1000]
    assert len(long_rows) >= 8
    bad[long_rows] *= 1.0093
    e = parity.out_errors(torch.from_numpy(bad).to(torch.float16), out, torch.float16)
    assert e["rel_l2"] <= 1e-3          # within the whole-tensor bound
    assert e["row_excess"] > 1e-3


def test_wrong_value_rows_are_caught(ragged):
    """One head of one sequence takes another head's output (a V-side slip
    that leaves lse intact)."""
    p, out, _ = ragged
    bad = out.copy()
    bad[5, 7] = out[5, 6]
    e = parity.out_errors(torch.from_numpy(bad).to(torch.float16), out, torch.float16)
    assert e["row_excess"] > 0.1 and e["row_worst"] == 5 * p.q.shape[1] + 7


def test_empty_rows_must_be_zero():
    ref = np.zeros((1, 2, 8))
    ref[0, 1] = 1.0
    g = torch.zeros(1, 2, 8, dtype=torch.float16)
    g[0, 1] = 1.0
    assert parity.out_errors(g, ref, torch.float16)["row_excess"] == 0.0
    g[0, 0, 3] = 0.01
    e = parity.out_errors(g, ref, torch.float16)
    assert e["row_excess"] > 1e-3 and e["row_worst"] == 0


def test_lse_error_and_inf_pattern():
    ref = np.array([[1.0, -np.inf, 3.0]])
    err, same = parity.lse_error(torch.tensor([[1.00002, -float("inf"), 3.0]], dtype=torch.float64), ref)
    assert same and abs(err - 2e-5) < 1e-9
    _, same = parity.lse_error(torch.tensor([[1.0, 0.0, 3.0]], dtype=torch.float64), ref)
    assert not same
