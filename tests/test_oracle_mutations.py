"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/pa_oracle.c, plants one plausible mistake (a wrong head
map, a dropped scale, a wrong sign, an off-by-one window, transposed strides,
...), compiles the copy with gcc and runs a subset of the pins against it: the
mpmath brute force on the logical K/V, the hand-derived golden cases and the
rotary embedding's complex-form brute force and closed forms.  At
least one pin must fail for every planted mistake; the unmodified source must
pass them all.  This shows the pins constrain every step of the oracle.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as oracle_mod
from paged_kv_decode_amd import workloads as W

from test_oracle_pins import BRUTE_CASES, GOLDEN, _golden_problem, brute
from test_oracle_rotary import (BRUTE_ROPE_CASES, test_two_keys_closed_form,
                                test_window_and_query_position_closed_form, brute_rope)

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "pa_oracle.c")

MUTATIONS = {
    "none": [],
    "head_map_modulo": [("h / (p->Hq / p->Hkv)", "h % p->Hkv")],
    "slot_off_by_one": [("int slot = j % p->page_size;", "int slot = (j + 1) % p->page_size;")],
    "page_row_ignored": [("p->page_table[(int64_t)b * p->pt_stride + j / p->page_size]",
                          "p->page_table[j / p->page_size]")],
    "scale_dropped": [("return p->scale * acc;", "return acc;")],
    "max_sign_flipped": [("double e = exp(s[j - lo] - M);", "double e = exp(M - s[j - lo]);")],
    "lse_without_max": [("    *lse = M + log(L);\n    free(s);", "    *lse = log(L);\n    free(s);")],
    "window_off_by_one": [("*lo = (p->window > 0 && *n > p->window) ? *n - p->window : 0;",
                           "*lo = (p->window > 0 && *n > p->window) ? *n - p->window - 1 : 0;")],
    "normalisation_dropped": [("    for (int d = 0; d < D; ++d)\n        out[d] /= L;\n",
                               "    for (int d = 0; d < D; ++d)\n        out[d] /= 1.0;\n")],
    "strides_transposed": [("(int64_t)g * p->stride_head +\n           (int64_t)slot * p->stride_slot",
                            "(int64_t)slot * p->stride_head +\n           (int64_t)g * p->stride_slot")],
    "query_head_swapped": [("int64_t qo = ((int64_t)b * p->Hq + h) * p->D;",
                            "int64_t qo = ((int64_t)b * p->Hq + (p->Hq - 1 - h)) * p->D;")],
    "last_key_dropped": [("    for (int j = lo; j < n; ++j) {\n        double e",
                          "    for (int j = lo; j < n - 1; ++j) {\n        double e")],
    "f16_exponent_bias": [("ldexp((double)(f + 1024), e - 25)", "ldexp((double)(f + 1024), e - 24)")],
    # rotary embedding
    "rope_turn_reversed": [("return x * cos(angle) - load_elt(base, off + d + half, dtype) * sin(angle);",
                            "return x * cos(angle) + load_elt(base, off + d + half, dtype) * sin(angle);"),
                           ("return x * cos(angle) + load_elt(base, off + d - half, dtype) * sin(angle);",
                            "return x * cos(angle) - load_elt(base, off + d - half, dtype) * sin(angle);")],
    "rope_one_half_sign": [("return x * cos(angle) + load_elt(base, off + d - half, dtype) * sin(angle);",
                            "return x * cos(angle) - load_elt(base, off + d - half, dtype) * sin(angle);")],
    "rope_exponent": [("pow(p->rope_theta, -2.0 * i / p->D)", "pow(p->rope_theta, -1.0 * i / p->D)")],
    "rope_query_at_n": [("p->context_lens[b] - 1.0", "(double)p->context_lens[b]")],
    "rope_key_off_by_one": [("d, (double)j)", "d, (double)(j + 1))")],
    "rope_scale_multiplies": [("pos / p->rope_scale", "pos * p->rope_scale")],
    "rope_query_not_turned": [("qv[d] = p->rotary ?", "qv[d] = 0 ?")],
    "rope_adjacent_pairs": [("int i = d < half ? d : d - half;", "int i = d / 2;"),
                            ("if (d < half)\n        return x * cos(angle) - load_elt(base, off + d + half, dtype) * sin(angle);\n    return x * cos(angle) + load_elt(base, off + d - half, dtype) * sin(angle);",
                             "if (d % 2 == 0)\n        return x * cos(angle) - load_elt(base, off + d + 1, dtype) * sin(angle);\n    return x * cos(angle) + load_elt(base, off + d - 1, dtype) * sin(angle);")],
}


def _build(name, tmp_path):
    src = open(SRC).read()
    for a, b in MUTATIONS[name]:
        assert a in src, "mutation anchor not found: %r" % a
        src = src.replace(a, b)
    c = tmp_path / ("m_%s.c" % name)
    so = tmp_path / ("m_%s.so" % name)
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(c), "-o",
                    str(so), "-lm"], check=True)
    return oracle_mod.load_library(str(so))


def _pins_pass(lib):
    """True when every pin in the subset holds for the library ``lib``."""
    for case in BRUTE_CASES:
        B, Hq, Hkv, D, dtype, lens, window, ps = case
        w = W.custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                     context_lens=lens, seed=11 + len(lens) + D, window=window, page_size=ps,
                     num_pages=sum((n + ps - 1) // ps for n in lens) + 3)
        p = W.generate(w, keep_logical=True)
        try:
            out, lse = oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens,
                                     p.scale, window=p.window, lib=lib)
        except ValueError:
            return False
        bo, bl = brute(p.q, p.logical_k, p.logical_v, lens, p.scale, window, Hq // Hkv)
        fin = ~np.isinf(bl)
        if not (np.array_equal(np.isinf(lse), np.isinf(bl)) and
                np.allclose(lse[fin], bl[fin], rtol=1e-13, atol=1e-13) and
                np.allclose(out, bo, rtol=1e-12, atol=1e-13)):
            return False
    for c in json.load(open(GOLDEN))["cases"]:
        p = _golden_problem(c, page_size=2, seed=2)
        out, lse = oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens,
                                 p.scale, window=p.window, lib=lib)
        if not (np.allclose(out[0], c["out"], rtol=1e-14, atol=1e-14) and
                np.allclose(lse[0], c["lse"], rtol=1e-14, atol=1e-14)):
            return False
    return _rotary_pins_pass(lib)


def _rotary_pins_pass(lib):
    """The rotary pins: complex-form brute force and the closed forms."""
    for case in BRUTE_ROPE_CASES[:3] + BRUTE_ROPE_CASES[4:]:
        B, Hq, Hkv, D, dtype, lens, window, ps, theta, rscale = case
        w = W.custom(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                     context_lens=lens, seed=31 + D + len(lens), window=window, page_size=ps)
        p = W.generate(w, keep_logical=True)
        out, lse = oracle.decode(p.q, p.k_cache, p.v_cache, p.page_table, p.context_lens,
                                 p.scale, window=p.window, lib=lib, rotary=(theta, rscale))
        bo, bl = brute_rope(p.q, p.logical_k, p.logical_v, lens, p.scale, window, Hq // Hkv,
                            theta, rscale)
        fin = ~np.isinf(bl)
        if not (np.array_equal(np.isinf(lse), np.isinf(bl)) and
                np.allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12) and
                np.allclose(out, bo, rtol=1e-11, atol=1e-12)):
            return False
    orig = oracle.decode
    try:
        oracle.decode = lambda *a, **k: orig(*a, lib=lib, **k)
        for fn, args in ((test_two_keys_closed_form, (1.0,)), (test_two_keys_closed_form, (2.0,)),
                         (test_window_and_query_position_closed_form, ())):
            try:
                fn(*args)
            except AssertionError:
                return False
    finally:
        oracle.decode = orig
    return True


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    lib = _build(name, tmp_path)
    if name == "none":
        assert _pins_pass(lib)
    else:
        assert not _pins_pass(lib), "planted mistake %s went unnoticed" % name
