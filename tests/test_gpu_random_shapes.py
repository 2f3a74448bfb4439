"""GPU: parity with the oracle over 48 seeded random problem shapes.

Each case draws, from its own seed:
  * head_dim, dtype, the GQA group and the KV-head count;
  * the batch size and ragged lengths (empty and one-token sequences,
    exact page multiples);
  * a sliding window or none, rotary or none;
  * the planner's partition size or a forced one;
  * the dense or the token-major cache layout.
Every case is compared with the float64 oracle to the standard tolerances.
The draws are fixed by the seeds, so the suite is the same on every run.
"""
import dataclasses
import random

import pytest
import torch

from paged_kv_decode_amd import workloads as W

from helpers import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

GROUPS = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16]


def draw(seed: int):
    r = random.Random(seed)
    D = r.choice([64, 96, 128, 256])
    dtype = r.choice([torch.float16, torch.bfloat16] + ([torch.float32] if D == 64 else []))
    hkv = r.choice([1, 2, 4])
    G = r.choice(GROUPS)
    B = r.choice([1, 1, 2, 3, 5, 8])
    lens = []
    for _ in range(B):
        kind = r.random()
        if kind < 0.1:
            lens.append(0)
        elif kind < 0.2:
            lens.append(1)
        elif kind < 0.3:
            lens.append(16 * r.randint(1, 100))
        else:
            lens.append(r.randint(2, 2500))
    window = r.choice([0, 0, r.randint(1, 1200)])
    rope = None if r.random() < 0.6 else (r.choice([1e4, 5e5]), r.choice([1.0, 2.0]))
    S = r.choice([None, None, 16 * r.randint(1, 40)])
    token_major = r.random() < 0.2
    return D, dtype, hkv, G, lens, window, rope, S, token_major


@pytest.mark.parametrize("seed", range(48))
def test_random_shape(seed):
    D, dtype, hkv, G, lens, window, rope, S, token_major = draw(7000 + seed)
    w = W.custom(batch=len(lens), num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D,
                 dtype=dtype, context_lens=lens, seed=7000 + seed, window=window, rope=rope)
    p = W.generate(w)
    ref_out, ref_lse = run_oracle(p)
    if token_major:
        # [num_pages, ps, Hkv, D] storage viewed as [num_pages, Hkv, ps, D]
        k = p.k_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = p.v_cache.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        p = dataclasses.replace(p, k_cache=k, v_cache=v)
    out, lse, plan = run_gpu(p, partition_size=S)
    what = "seed %d: D=%d %s Hkv=%d G=%d lens=%s window=%d rope=%s S=%s token_major=%s" % (
        seed, D, dtype, hkv, G, lens, window, rope, S, token_major)
    rel, lerr = compare(out, lse, ref_out, ref_lse, dtype, what)
    print("%s plan(S=%d,P=%d) rel_l2=%.3g lse_err=%.3g" % (
        what, plan["partition_size"], plan["num_partitions"], rel, lerr), flush=True)
