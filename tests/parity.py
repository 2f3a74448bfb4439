"""Output comparison against the float64 oracle (test infrastructure: used by
the tests, by smoke() and by the benchmark's parity line; it holds no part of
the attention arithmetic).

Two figures for out, both against the exact (float64) oracle result r:

* whole tensor: rel-L2 of the GPU output against r rounded (RNE) to the
  output dtype, ||g - rnd(r)|| / ||rnd(r)|| over [B, Hq, D].  This is the
  tolerance's own definition (rel-L2 <= 1e-3 for f16/bf16, <= 1e-5 for f32).
* per (sequence, query head) row: the part of each element's error beyond
  one unit in the last place of the output dtype at r,
      e_i = max(0, |g_i - r_i| - ulp(r_i)),
  as a fraction of the row's norm, ||e_row|| / ||r_row||, held to the same
  tolerance row by row.  One ulp is the rounding of the result itself: where
  r_i lies near a rounding boundary, a float32 accumulation may land on
  either neighbour, and in a bfloat16 row dominated by a few large elements
  one such flip alone is worth up to 2^-7 of the row norm.  Any error past
  that counts, so a few percent of error confined to one sequence's heads
  fails the row bound even when it is invisible in the whole-tensor norm.
  The plain rel-L2 of every row against rnd(r) is reported as well.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_TOL = {torch.float32: 1e-5, torch.float16: 1e-3, torch.bfloat16: 1e-3}
LSE_TOL = 1e-4

# Significand bits after the leading one, and the smallest positive spacing
# (subnormal step), of each output dtype.
_FRAC_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}
_MIN_STEP = {torch.float32: 2.0 ** -149, torch.float16: 2.0 ** -24, torch.bfloat16: 2.0 ** -133}


def ulp(r: np.ndarray, dtype) -> np.ndarray:
    """Spacing of `dtype` values at |r| (float64 in, float64 out): for r in
    [2^e, 2^(e+1)) it is 2^(e - fraction bits), never below the subnormal
    step."""
    a = np.abs(r)
    _, e = np.frexp(a)            # a = m 2^e, m in [0.5, 1): leading bit at 2^(e-1)
    step = np.where(a > 0, np.ldexp(1.0, e - 1 - _FRAC_BITS[dtype]), 0.0)
    return np.maximum(step, _MIN_STEP[dtype])


def out_errors(out: torch.Tensor, ref_out: np.ndarray, dtype) -> dict:
    """Whole-tensor and per-row errors of out ([B, Hq, D], dtype) against the
    oracle's float64 ref_out (see the module docstring)."""
    g = out.double().cpu().numpy().reshape(-1, out.shape[-1])
    r = np.asarray(ref_out, dtype=np.float64).reshape(g.shape)
    rr = torch.from_numpy(r).to(dtype).double().numpy()
    diff = g - rr
    denom = np.linalg.norm(rr)
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    rows = g.shape[0]
    if rows == 0:
        return {"rel_l2": rel, "row_excess": 0.0, "row_worst": -1, "row_rel_l2_max": 0.0,
                "max_abs": 0.0}
    excess = np.maximum(0.0, np.abs(g - r) - ulp(r, dtype))
    rn = np.linalg.norm(r, axis=1)
    en = np.linalg.norm(excess, axis=1)
    # A row whose exact result is zero (an empty context) must be zero.
    row_ex = np.where(rn > 0, en / np.where(rn > 0, rn, 1.0), en)
    rrn = np.linalg.norm(rr, axis=1)
    dn = np.linalg.norm(diff, axis=1)
    row_rel = np.where(rrn > 0, dn / np.where(rrn > 0, rrn, 1.0), dn)
    worst = int(np.argmax(row_ex))
    return {"rel_l2": rel, "row_excess": float(row_ex[worst]), "row_worst": worst,
            "row_rel_l2_max": float(row_rel.max()), "max_abs": float(np.abs(g - r).max())}


def lse_error(lse: torch.Tensor, ref_lse: np.ndarray):
    """(max abs error over finite oracle entries, whether the -inf entries
    agree)."""
    l = lse.double().cpu().numpy().reshape(-1)
    ref = np.asarray(ref_lse, dtype=np.float64).reshape(-1)
    inf_ref = np.isneginf(ref)
    same_inf = bool(np.array_equal(np.isneginf(l), inf_ref))
    fin = ~inf_ref
    err = float(np.abs(l[fin] - ref[fin]).max()) if fin.any() else 0.0
    return err, same_inf


def describe(e: dict, heads: int) -> str:
    """One line naming the worst (sequence, head) row."""
    w = e["row_worst"]
    where = "b=%d h=%d" % divmod(w, heads) if w >= 0 else "-"
    return ("rel_l2=%.3g worst_row(%s) excess=%.3g row_rel_l2_max=%.3g max_abs=%.3g"
            % (e["rel_l2"], where, e["row_excess"], e["row_rel_l2_max"], e["max_abs"]))
