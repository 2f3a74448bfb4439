"""GPU parity of the CSR page-table entry point (pa_decode_run_csr).

The CSR form (page_indptr, page_indices, last_page_len) carries the same
page ids as the dense table; the oracle runs on the dense form of the same
problem.  Covered:
  * the five workloads at full size, with the host switch of TVM PR #20426,
    section "Change" (split only when nnz_pages > B * 256 / page_size) and
    with each workload's own partition size;
  * bitwise agreement with the dense entry point under the same forced
    partition size (the same kernels read the same pages);
  * the switch itself: a batch of short contexts runs unsplit, a longer one
    split, both within tolerance;
  * sequences owning no page (out = 0, lse = -inf), last pages holding 1 and
    16 tokens, pages shared between sequences, NaN in every slot the method
    must not read, and max_context_len left to nnz_pages * page_size.
"""
import dataclasses

import torch
import pytest

from paged_kv_decode_amd import workloads as W

from helpers import compare, run_gpu, run_gpu_csr, run_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_workload_full_size_csr(name):
    p = W.generate(W.CONFIGS[name])
    csr = W.to_csr(p)
    ref_out, ref_lse = run_oracle(p)
    for S in sorted({0, p.workload.partition_size}):
        out, lse, plan = run_gpu_csr(p, csr, partition_size=S)
        compare(out, lse, ref_out, ref_lse, p.workload.dtype, "%s csr S=%d" % (name, S))
        if S == 0 and csr.nnz_pages * 16 <= p.q.shape[0] * 256:
            assert plan["split"] == 0


@pytest.mark.parametrize("name", ["llama1b_ctx3060_f16", "llama8b_b16_ragged_f16",
                                  "d256_window4096_bf16"])
def test_csr_matches_dense_bitwise(name):
    p = W.generate(W.CONFIGS[name])
    csr = W.to_csr(p)
    for S in (64, 512):
        a = run_gpu(p, partition_size=S)
        c = run_gpu_csr(p, csr, partition_size=S)
        assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]), (name, S)
        assert a[2] == c[2]


def test_csr_host_switch_unsplit_and_split():
    # 8 sequences averaging < 256 tokens: one partition per context
    short = W.custom(batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                     context_lens=[1, 16, 17, 100, 255, 256, 300, 511], seed=900)
    # the same batch at ~2k tokens: split
    long_ = dataclasses.replace(short, context_lens=[1, 2048, 4000, 17, 3000, 2500, 1024, 999],
                                seed=901)
    for w, split in ((short, 0), (long_, 1)):
        p = W.generate(w)
        csr = W.to_csr(p)
        assert (csr.nnz_pages * 16 > 8 * 256) == bool(split)
        out, lse, plan = run_gpu_csr(p, csr, partition_size=0)
        assert plan["split"] == split
        ref = run_oracle(p)
        compare(out, lse, ref[0], ref[1], torch.float16, "switch split=%d" % split)


def test_csr_edges():
    w = W.custom(batch=5, num_q_heads=12, num_kv_heads=2, head_dim=256, dtype=torch.bfloat16,
                 context_lens=[0, 16, 33, 1, 48], seed=902)
    p = W.generate(w, poison=True, extra_pages=4)
    csr = W.to_csr(p)
    assert csr.last_page_len.tolist() == [0, 16, 1, 1, 16]
    ref_out, ref_lse = run_oracle(p)
    for S, mc in ((0, None), (16, None), (32, 0)):
        out, lse, _ = run_gpu_csr(p, csr, partition_size=S, max_context_len=mc)
        compare(out, lse, ref_out, ref_lse, torch.bfloat16, "csr edges S=%d" % S)
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_csr_shared_pages():
    # two sequences read the same physical pages (aliasing is legal, read-only)
    w = W.custom(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=torch.float16,
                 context_lens=[700, 700], seed=903)
    p = W.generate(w)
    k = -(-700 // 16)
    pt = p.page_table.clone()
    pt[1, :k] = pt[0, :k]
    p2 = dataclasses.replace(p, page_table=pt)
    csr = W.to_csr(p2)
    ref_out, ref_lse = run_oracle(p2)
    for S in (0, 64):
        out, lse, _ = run_gpu_csr(p2, csr, partition_size=S)
        compare(out, lse, ref_out, ref_lse, torch.float16, "csr shared S=%d" % S)


def test_csr_ragged_batch_plans_the_balanced_schedule_itself():
    """partition_size 0 on the CSR path: a batch whose mean page count is
    well below the longest gets the length-balanced schedule from the host's
    page count (one 4096-token sequence among 200-token ones; the batch-16
    ragged workload, mean ~0.53 of the longest, with and without rotary), the
    same plan and bits as asking for it; a batch at a mean of 0.64 (above
    the 5/8 rule) and a batch of equal lengths keep fixed partitions.  All
    match the oracle."""
    skew = W.custom(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                    context_lens=[4096] + [200] * 15, seed=905)
    near = W.custom(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=torch.float16,
                    context_lens=[4096] + [2500] * 15, seed=906)
    cases = [(W.generate(skew), True),
             (W.generate(W.CONFIGS["llama8b_b16_ragged_rope_f16"]), True),
             (W.generate(W.CONFIGS["llama8b_b16_ragged_f16"]), True),
             (W.generate(near), False),
             (W.generate(W.custom(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                  dtype=torch.float16, context_lens=[2171] * 16, seed=904)), False)]
    for p, balanced in cases:
        csr = W.to_csr(p)
        out, lse, plan = run_gpu_csr(p, csr, partition_size=0)
        assert (plan["balanced_waves"] > 0) == balanced, plan
        assert plan["split"] == 1
        ref = run_oracle(p)
        compare(out, lse, ref[0], ref[1], torch.float16, "csr auto balanced=%s" % balanced)
        if balanced:
            out_b, lse_b, plan_b = run_gpu_csr(p, csr, partition_size=W.BALANCED)
            assert plan_b == plan and torch.equal(out_b, out) and torch.equal(lse_b, lse)
