"""Host-side checks of libpa_decode.so (CPU only, no kernel launch).

* the library loads and exports every function include/pa_decode.h declares;
* the status strings;
* pa_decode_create rejects invalid descriptions before touching HIP;
* the planner (pa_decode_plan_query, pure host) covers every context with its
  partitions, keeps the partition size a multiple of the page size, picks the
  unsplit path exactly when one partition covers every context, keeps the
  grid and LDS within limits, and honours a forced partition size (the
  5-th workload's 512-token partitions give 196 of them at 100,000 tokens).
"""
import ctypes
import os
import re

import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pa_decode.h")


def lib():
    return B.load_library()


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(pa_decode_\w+)\s*\(", text, re.M))
    assert declared == set(B.EXPORTED), declared ^ set(B.EXPORTED)
    L = lib()
    for name in declared:
        assert hasattr(L, name) and getattr(L, name) is not None


def test_status_strings():
    assert B.pa_decode_status_string(0) == "ok"
    assert B.pa_decode_status_string(-3) == "workspace too small"
    assert B.pa_decode_status_string(123) == "unknown status"


@pytest.mark.parametrize("fields,status", [
    (dict(num_q_heads=0), B.PA_DECODE_INVALID_ARG),
    (dict(num_q_heads=6, num_kv_heads=4), B.PA_DECODE_INVALID_ARG),
    (dict(head_dim=80), B.PA_DECODE_UNSUPPORTED),
    (dict(dtype=B.PA_DTYPE_F32, head_dim=96), B.PA_DECODE_UNSUPPORTED),
    (dict(page_size=32), B.PA_DECODE_UNSUPPORTED),
    (dict(dtype=7), B.PA_DECODE_UNSUPPORTED),
    (dict(dtype=B.PA_DTYPE_F32, head_dim=128), B.PA_DECODE_UNSUPPORTED),
    (dict(num_q_heads=32, num_kv_heads=1), B.PA_DECODE_UNSUPPORTED),
    (dict(max_batch=-1), B.PA_DECODE_INVALID_ARG),
    (dict(max_batch=65536), B.PA_DECODE_UNSUPPORTED),
    (dict(num_q_heads=65536 * 2, num_kv_heads=65536), B.PA_DECODE_UNSUPPORTED),
    (dict(rotary_mode=2, rope_theta=1e4, rope_scale=1.0), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=-1), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=1, rope_theta=0.0, rope_scale=1.0), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=1, rope_theta=1e4, rope_scale=0.0), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=1, rope_theta=-1e4, rope_scale=1.0), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=1, rope_theta=float("inf"), rope_scale=1.0), B.PA_DECODE_INVALID_ARG),
    (dict(rotary_mode=1, rope_theta=1e4, rope_scale=float("nan")), B.PA_DECODE_INVALID_ARG),
    (dict(debug_checks=2), B.PA_DECODE_INVALID_ARG),
    (dict(debug_checks=-1), B.PA_DECODE_INVALID_ARG),
])
def test_create_rejects_invalid_descriptions(fields, status):
    base = dict(num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                dtype=B.PA_DTYPE_F16, max_batch=4, max_context_len=4096, device=0)
    base.update(fields)
    d = B.PaDecodeDesc(**base)
    h = ctypes.c_void_p()
    assert lib().pa_decode_create(ctypes.byref(d), ctypes.byref(h)) == status
    assert not h.value


def test_read_probe_rejects_bad_arguments_on_the_host():
    # Each case fails before anything touches a device.
    sink = ctypes.c_void_p(256)
    probe = lib().pa_decode_read_probe
    assert probe(ctypes.c_void_p(256), None, 4, 2048, None, None) == B.PA_DECODE_INVALID_ARG
    assert probe(ctypes.c_void_p(256), None, -1, 2048, sink, None) == B.PA_DECODE_INVALID_ARG
    assert probe(ctypes.c_void_p(256), None, 4, 1024, sink, None) == B.PA_DECODE_INVALID_ARG
    assert probe(ctypes.c_void_p(256), None, 4, 16384, sink, None) == B.PA_DECODE_INVALID_ARG
    assert probe(None, None, 4, 2048, sink, None) == B.PA_DECODE_INVALID_ARG
    assert probe(ctypes.c_void_p(264), None, 4, 2048, sink, None) == B.PA_DECODE_INVALID_ARG
    assert probe(ctypes.c_void_p(256), None, 0, 2048, sink, None) == B.PA_DECODE_OK


def test_null_arguments_are_rejected():
    assert lib().pa_decode_debug_status(None, None) == B.PA_DECODE_INVALID_ARG
    assert lib().pa_decode_create(None, None) == B.PA_DECODE_INVALID_ARG
    assert lib().pa_decode_run(None, None, None) == B.PA_DECODE_INVALID_ARG
    assert lib().pa_decode_last_plan(None, None) == B.PA_DECODE_INVALID_ARG
    assert lib().pa_decode_destroy(None) == B.PA_DECODE_OK


def plan(w: W.Workload, num_cus=256, batch=None, max_ctx=None, S=None, window=None,
         waves_per_cu=8):
    d = B.make_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=4096,
                    max_context_len=1 << 20)
    lens = w.context_lens or [4096]
    return B.pa_decode_plan_query(d, num_cus, waves_per_cu, batch or w.batch,
                                  max_ctx or max(lens), w.window if window is None else window,
                                  w.partition_size if S is None else S)


def covered(p, n, window):
    """Partitions [lo/S + i for i < P] cover [lo, n) with the plan's S."""
    lo = n - window if (window > 0 and n > window) else 0
    if n == lo:
        return True
    S = p.partition_size
    first = lo // S
    last = (n + S - 1) // S - 1
    return last - first + 1 <= p.num_partitions


@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_plan_covers_every_context(name):
    w = W.CONFIGS[name]
    for max_ctx in (1, 15, 16, 17, 300, 3060, 4096, 8192, 100000):
        for S in (0, 16, 48, 512):
            p = plan(w, max_ctx=max_ctx, S=S)
            assert p.partition_size % 16 == 0 and p.partition_size > 0
            if S:
                assert p.partition_size == S
            for n in {0, 1, max_ctx // 2, max_ctx - 1, max_ctx}:
                if 0 <= n <= max_ctx:
                    assert covered(p, n, w.window), (name, max_ctx, S, n)
            assert p.split == (1 if p.num_partitions > 1 else 0)
            assert p.waves_per_partition in (1, 2, 4)
            assert p.waves_per_group % p.waves_per_partition == 0
            slots = p.waves_per_group // p.waves_per_partition
            assert p.grid_partial[0] == -(-p.num_partitions // slots)
            assert p.grid_partial[1] == w.num_kv_heads
            assert 64 <= p.block_partial <= 256 and p.block_partial == 64 * p.waves_per_group
            if p.split and p.num_partitions <= 64:
                # one wave per 64-column slice, or per 16-column slice when
                # 64-column slices give fewer than 256 waves
                slices = -(-w.head_dim // 64)
                cw = 16 if w.batch * w.num_q_heads * slices < 256 else 64
                units = w.batch * w.num_q_heads * -(-w.head_dim // cw)
                assert list(p.grid_merge) == [-(-units // 4), 1, 1]
            elif p.split:   # one workgroup per 16-column slice
                assert list(p.grid_merge) == [w.num_q_heads, w.batch, w.head_dim // 16]
            if p.split:
                rows = w.batch * w.num_q_heads * p.num_partitions
                assert p.workspace_bytes >= rows * (w.head_dim + 2) * 4
            else:
                assert p.workspace_bytes == 0


def test_forced_512_partitions_at_100k_give_196():
    p = plan(W.CONFIGS["ctx100k_gqa6_f16"])
    assert p.partition_size == 512 and p.num_partitions == 196 and p.split == 1


@pytest.mark.parametrize("waves_per_cu", [4, 8, 12, 16])
@pytest.mark.parametrize("name", W.CONFIG_ORDER)
def test_waves_per_partition_target_one_round(name, waves_per_cu):
    """The waves sharing a partition bring the grid's wave count closest to
    four per compute unit without exceeding what the device holds at once."""
    w = W.CONFIGS[name]
    p = plan(w, waves_per_cu=waves_per_cu, S=max(w.partition_size, 0))   # fixed partitions
    if not p.split:
        return
    units = w.batch * w.num_kv_heads * p.num_partitions
    capacity, target = 256 * waves_per_cu, min(256 * waves_per_cu, 256 * 4)
    blocks = -(-(p.partition_size // 16 + (1 if w.window else 0)) // p.pages_per_block)
    cands = [c for c in (1, 2, 4) if c == 1 or (c <= blocks and units * c <= capacity
                                                and c <= p.waves_per_group)]
    best = min(cands, key=lambda c: abs(units * c - target))
    assert p.waves_per_partition == best
    assert units * p.waves_per_partition <= max(capacity, units)


def test_long_context_with_512_token_partitions_uses_one_wave_each():
    p = plan(W.CONFIGS["ctx100k_gqa6_f16"], waves_per_cu=8)
    assert p.waves_per_partition == 1 and p.waves_per_group == 4
    assert p.grid_partial[0] == 49  # 196 partitions, 4 per workgroup


def test_unsplit_when_one_partition_covers_the_context():
    w = W.custom(batch=512, num_q_heads=32, num_kv_heads=8, head_dim=128, context_lens=[200] * 512)
    p = plan(w)
    assert p.split == 0 and p.num_partitions == 1 and p.partition_size >= 200
    # long context, small batch: split
    p = plan(W.CONFIGS["llama1b_ctx3060_f16"])
    assert p.split == 1 and p.num_partitions > 1


def test_plan_fills_the_device():
    # at least about one wave per compute unit when the work allows it
    for name in ("llama1b_ctx3060_f16", "llama8b_b16_ragged_f16", "d256_window4096_bf16"):
        w = W.CONFIGS[name]
        p = plan(w)
        waves = p.grid_partial[0] * p.grid_partial[1] * p.grid_partial[2] * p.block_partial // 64
        assert waves >= 256, (name, p.as_dict())


def test_plan_rejects_bad_partition_sizes():
    w = W.CONFIGS["llama1b_ctx3060_f16"]
    with pytest.raises(B.PaDecodeError):
        plan(w, S=24)
    with pytest.raises(B.PaDecodeError):
        plan(w, num_cus=0)


# ---- CSR page-table form ------------------------------------------------

def csr_plan(w: W.Workload, batch, nnz, max_ctx=0, S=0, window=0, num_cus=256, waves_per_cu=8):
    d = B.make_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=4096,
                    max_context_len=1 << 20)
    return B.pa_decode_plan_query_csr(d, num_cus, waves_per_cu, batch, nnz, max_ctx, window, S)


@pytest.mark.parametrize("batch,avg_tokens", [(1, 16), (1, 3060), (8, 100), (8, 256), (8, 272),
                                              (16, 2048), (64, 240), (64, 4096)])
def test_csr_host_switch_follows_the_page_count(batch, avg_tokens):
    """TVM PR #20426, section "Change": the sharded path only when
    nnz_pages > B * 256 / page_size; otherwise one partition per context."""
    w = W.CONFIGS["llama8b_b16_ragged_f16"]
    nnz = batch * (-(-avg_tokens // 16))
    max_ctx = 2 * avg_tokens
    p = csr_plan(w, batch, nnz, max_ctx=max_ctx)
    if nnz * 16 <= batch * 256:
        assert p.split == 0 and p.num_partitions == 1 and p.partition_size >= max_ctx
        assert p.workspace_bytes == 0
    elif 8 <= batch <= 64 and 8 * nnz < 5 * batch * (-(-max_ctx // 16)):
        dense = plan(w, batch=batch, max_ctx=max_ctx, S=B.PA_DECODE_PARTITION_BALANCED)
        assert p.balanced_waves > 0 and p.as_dict() == dense.as_dict()
    else:
        dense = plan(w, batch=batch, max_ctx=max_ctx, S=0)
        assert p.as_dict() == dense.as_dict()


@pytest.mark.parametrize("batch,lens,rope,balanced", [
    (16, [4096] * 16, False, False),                       # uniform
    (16, [4096 - 37 * i for i in range(16)], False, False),  # nearly uniform
    (16, [1 + 273 * i for i in range(16)], False, True),   # mean ~0.53 of the longest: balanced
    (16, [4096] + [2500] * 15, False, False),              # mean 0.64 (just above 5/8): fixed
    (16, [4096] + [2440] * 15, False, True),               # mean 0.62 (just below 5/8): balanced
    (16, [4096] + [200] * 15, False, True),                # one long, many short: balanced
    (16, [1 + 273 * i for i in range(16)], True, True),    # the same with rotary: balanced
    (16, [4096] + [2500] * 15, True, False),               # mean 0.64 with rotary: fixed
    (16, [4096 - 100 * i for i in range(16)], True, False),  # mean 0.82, rotary: fixed
    (4, [4096, 17, 17, 17], False, False),                 # below 8 sequences: fixed
    (8, [4096] + [300] * 7, False, True),                  # 8 sequences, very ragged
    (65, [4096] + [17] * 64, False, False),                # above 64 sequences: fixed
    (4, [8192] * 4, False, False),                         # the windowed workload's batch
])
def test_csr_ragged_rule_picks_the_balanced_schedule(batch, lens, rope, balanced):
    """With partition_size 0 and pages above the single-pass switch, the CSR
    host picks the length-balanced schedule for 8 .. 64 sequences whose mean
    page count is below 5/8 of what max_context_len allows, with or without
    rotary, else fixed partitions (the rule measured in bench.py --probe
    schedule-sweep); the choice uses host counts only."""
    w = W.CONFIGS["llama8b_b16_ragged_f16"]
    d = B.make_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=4096,
                    max_context_len=1 << 20, rope=(500000.0, 1.0) if rope else None)
    nnz = sum(-(-n // 16) for n in lens)
    max_ctx = max(lens)
    p = B.pa_decode_plan_query_csr(d, 256, 8, batch, nnz, max_ctx, 0, 0)
    assert (8 <= batch <= 64 and 8 * nnz < 5 * batch * (-(-max_ctx // 16))) == balanced
    assert (p.balanced_waves > 0) == balanced, p.as_dict()
    fixed = B.pa_decode_plan_query(d, 256, 8, batch, max_ctx, 0, 0)
    if not balanced:
        assert p.as_dict() == fixed.as_dict()


def test_csr_plan_defaults_and_forced_partitions():
    w = W.CONFIGS["ctx100k_gqa6_f16"]
    # forced 512-token partitions over 6250 pages: 196 partitions, as the dense form
    p = csr_plan(w, 1, 6250, max_ctx=100000, S=512)
    assert p.partition_size == 512 and p.num_partitions == 196 and p.split == 1
    # max_context_len 0 stands for nnz_pages * page_size
    p0 = csr_plan(w, 1, 6250, max_ctx=0, S=512)
    assert p0.num_partitions == 196
    # window: partitions cover only the window
    w4 = W.CONFIGS["d256_window4096_bf16"]
    pw = csr_plan(w4, 4, 4 * 512, max_ctx=8192, S=512, window=4096)
    assert pw.num_partitions == 9


@pytest.mark.parametrize("batch,nnz", [(1, -1), (0, 3)])
def test_csr_plan_rejects_bad_counts(batch, nnz):
    with pytest.raises(B.PaDecodeError):
        csr_plan(W.CONFIGS["llama1b_ctx3060_f16"], batch, nnz, max_ctx=64)


def test_csr_null_arguments_are_rejected():
    assert lib().pa_decode_run_csr(None, None, None) == B.PA_DECODE_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib().pa_decode_workspace_size_csr(None, 1, 1, 16, 0, 0, ctypes.byref(n)) == \
        B.PA_DECODE_INVALID_ARG


def test_csr_conversion_round_trips():
    for name in W.CONFIG_ORDER:
        p = W.generate(W.CONFIGS[name])
        c = W.to_csr(p)
        pt, lens = W.from_csr(c)
        assert torch.equal(lens, p.context_lens)
        for b, n in enumerate(lens.tolist()):
            k = -(-n // 16)
            assert torch.equal(pt[b, :k], p.page_table[b, :k])
        assert c.nnz_pages == sum(-(-n // 16) for n in lens.tolist())


@pytest.mark.parametrize("dtype", [B.PA_DTYPE_F16, B.PA_DTYPE_BF16])
def test_head_dim_96_is_planned(dtype):
    """head_dim 96 (12 chunks of 16 bytes per row, TVM PR #20426, "Tests",
    lays out D = 96 too): accepted, one page per block (192-byte rows), the
    merge grid covers a partial 64-column slice, LDS within 64 KiB per
    workgroup."""
    d = B.PaDecodeDesc(num_q_heads=32, num_kv_heads=8, head_dim=96, page_size=16, dtype=dtype,
                       max_batch=64, max_context_len=8192, device=0)
    h = ctypes.c_void_p()
    assert lib().pa_decode_create(ctypes.byref(d), ctypes.byref(h)) in (B.PA_DECODE_OK,
                                                                         B.PA_DECODE_HIP_ERROR)
    for S, P in ((16, 256), (512, 8)):
        p = B.pa_decode_plan_query(d, 256, 8, 2, 4096, 0, S)
        assert p.pages_per_block == 1 and p.num_partitions == P
        if P <= 64:   # 2 x 32 x 2 = 128 waves at 64 columns: 16-column slices
            assert list(p.grid_merge) == [-(-2 * 32 * (96 // 16) // 4), 1, 1]
        else:
            assert list(p.grid_merge) == [32, 2, 96 // 16]
        rows = 2 * 32 * P
        assert p.workspace_bytes >= rows * (96 + 2) * 4


@pytest.mark.parametrize("dtype,head_dim", [(B.PA_DTYPE_F32, 64), (B.PA_DTYPE_F16, 64),
                                            (B.PA_DTYPE_F16, 96), (B.PA_DTYPE_BF16, 128),
                                            (B.PA_DTYPE_F16, 256)])
def test_rotary_descriptions_are_planned(dtype, head_dim):
    """rotary_mode 1 (TVM PR #20426, "Correctness") with a valid base and
    scale is accepted for every built shape.  Its plan aims at twice the
    resident waves (rotary blocks cost about twice the instructions): the
    same or smaller partitions, every context still covered."""
    kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=head_dim, page_size=16, dtype=dtype,
              max_batch=64, max_context_len=1 << 17, device=0)
    d0 = B.PaDecodeDesc(**kw)
    d1 = B.PaDecodeDesc(rotary_mode=1, rope_theta=500000.0, rope_scale=1.0, **kw)
    h = ctypes.c_void_p()
    assert lib().pa_decode_create(ctypes.byref(d1), ctypes.byref(h)) in (B.PA_DECODE_OK,
                                                                          B.PA_DECODE_HIP_ERROR)
    for batch, ctx, window, S in ((1, 100000, 0, 0), (16, 4096, 0, 0), (4, 8192, 4096, 0),
                                  (1, 3060, 0, 512), (2, 17, 0, 0)):
        p0 = B.pa_decode_plan_query(d0, 256, 8, batch, ctx, window, S)
        p1 = B.pa_decode_plan_query(d1, 256, 8, batch, ctx, window, S)
        if S:
            assert p1.partition_size == p0.partition_size == S
            assert p1.num_partitions == p0.num_partitions
        else:
            assert p1.partition_size <= p0.partition_size
            assert p1.num_partitions >= p0.num_partitions
        assert p1.partition_size % 16 == 0
        assert covered(p1, ctx, window)
        assert p1.split == (p1.num_partitions > 1)
        if p1.split:
            assert p1.workspace_bytes >= batch * 32 * p1.num_partitions * (head_dim + 2) * 4



@pytest.mark.parametrize("dtype", [B.PA_DTYPE_F16, B.PA_DTYPE_BF16])
@pytest.mark.parametrize("waves_per_cu", [4, 6, 8])
def test_plans_fill_their_wave_target_with_two_wave_workgroups(dtype, waves_per_cu):
    """head_dim-256 rotary workgroups hold two waves (LDS); partitions are
    sized for those two waves, so a long batch launches the targeted wave
    count (one per resident slot, at most eight per compute unit), not half
    of it."""
    d = B.PaDecodeDesc(num_q_heads=16, num_kv_heads=4, head_dim=256, page_size=16, dtype=dtype,
                       max_batch=64, max_context_len=1 << 17, device=0, rotary_mode=1,
                       rope_theta=500000.0, rope_scale=1.0)
    p = B.pa_decode_plan_query(d, 256, waves_per_cu, 8, 8192, 0, 0)
    assert p.waves_per_group == 2
    waves = p.grid_partial[0] * p.grid_partial[1] * p.grid_partial[2] * p.waves_per_group
    target = 256 * min(waves_per_cu, 8)
    assert target * 0.9 <= waves <= target
    assert covered(p, 8192, 0)


@pytest.mark.parametrize("batch,hq,hkv,D,ctx,win,wpc,old_wgs", [
    (3, 8, 1, 64, 32768, 0, 16, 258),
    (6, 8, 2, 128, 16384, 0, 12, 264),
    (12, 8, 1, 64, 88064, 0, 16, 264),
    (4, 32, 8, 128, 8192, 4096, 12, 288),
    (8, 8, 4, 256, 8192, 4096, 8, 288),
])
def test_default_plans_keep_one_workgroup_per_compute_unit(batch, hq, hkv, D, ctx, win, wpc, old_wgs):
    """Where rounding the partition count up would end the grid a little
    past one 4-wave workgroup per compute unit (old_wgs on 256 units), the
    planner takes a few more pages per wave instead, so that no unit runs
    two: at most 256 workgroups, and the wave count stays near the target."""
    dt = B.PA_DTYPE_BF16 if D == 256 else B.PA_DTYPE_F16
    d = B.PaDecodeDesc(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=16, dtype=dt,
                       max_batch=64, max_context_len=1 << 20, device=0)
    p = B.pa_decode_plan_query(d, 256, wpc, batch, ctx, win, 0)
    wgs = p.grid_partial[0] * p.grid_partial[1] * p.grid_partial[2]
    assert p.split == 1 and p.waves_per_group == 4
    assert 256 * 3 // 4 <= wgs <= 256 < old_wgs
    # every visible page is still covered
    visible = min(ctx, win) if win else ctx
    assert p.num_partitions * p.partition_size >= visible


@pytest.mark.parametrize("name", ["llama1b_ctx3060_f16", "d256_window4096_bf16"])
def test_default_plans_of_the_benchmark_shapes_are_unchanged(name):
    """The 3060-token and windowed head_dim-256 plans (measured best in
    their sweeps) are what the grid rule leaves them."""
    w = W.CONFIGS[name]
    d = B.make_desc(w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, max_batch=64,
                    max_context_len=1 << 20)
    p = B.pa_decode_plan_query(d, 256, 16 if w.head_dim == 64 else 8, w.batch,
                               max(w.context_lens), w.window, 0)
    expect = {"llama1b_ctx3060_f16": (128, 24, [24, 8, 1]),
              "d256_window4096_bf16": (320, 14, [14, 4, 4])}[name]
    assert (p.partition_size, p.num_partitions, list(p.grid_partial)) == expect


@pytest.mark.parametrize("hq,batch,ctx,S,window,dtype,P", [
    (8, 4, 8192, 496, 0, B.PA_DTYPE_BF16, 17),
    (24, 2, 32768, 1008, 0, B.PA_DTYPE_F16, 33),
    (8, 8, 8192, 512, 4096, B.PA_DTYPE_BF16, 9),
])
def test_head_dim_256_fixed_partitions_past_one_workgroup_per_unit(hq, batch, ctx, S, window, dtype, P):
    """head_dim 256 with a caller's partition size whose 4-wave partitions
    would number a little more than the 256 compute units: two waves per
    partition, two partitions per 4-wave workgroup, within one workgroup
    per unit.  The same counts at head_dim 128 keep four waves per
    partition."""
    d = B.PaDecodeDesc(num_q_heads=hq, num_kv_heads=4, head_dim=256, page_size=16, dtype=dtype,
                       max_batch=64, max_context_len=1 << 20, device=0)
    p = B.pa_decode_plan_query(d, 256, 8, batch, ctx, window, S)
    wgs = p.grid_partial[0] * p.grid_partial[1] * p.grid_partial[2]
    assert p.num_partitions == P and 256 < 4 * batch * P < 512
    assert (p.waves_per_partition, p.waves_per_group) == (2, 4) and wgs <= 256
    d128 = B.PaDecodeDesc(num_q_heads=hq, num_kv_heads=4, head_dim=128, page_size=16,
                          dtype=B.PA_DTYPE_F16, max_batch=64, max_context_len=1 << 20, device=0)
    q = B.pa_decode_plan_query(d128, 256, 12, batch, ctx, window, S)
    assert q.num_partitions == P and q.waves_per_partition == 4


def test_plan_invariants_on_random_shapes():
    """Seeded random shapes (head_dim, dtype, heads, batch, context bound,
    window, automatic or fixed partition size, compute units and resident
    waves): every plan covers every context length up to its bound, its
    grid and workgroup sizes are consistent, its partitions are whole pages,
    and an automatic plan never takes more than 256 pages per wave."""
    import random
    r = random.Random(20261203)
    for _ in range(400):
        D = r.choice([64, 96, 128, 256])
        dt = r.choice([B.PA_DTYPE_F16, B.PA_DTYPE_BF16] + ([B.PA_DTYPE_F32] if D == 64 else []))
        hkv = r.choice([1, 2, 4, 8])
        G = r.choice([1, 2, 4, 6, 8])
        batch = r.choice([1, 2, 3, 5, 8, 12, 16, 24, 48])
        max_ctx = r.choice([1, 17, 300, 3060, r.randint(1, 40000), r.randint(40000, 200000)])
        window = r.choice([0, 0, r.randint(1, 5000)])
        S = r.choice([0, 0, 16 * r.randint(1, 64)])
        cus = r.choice([256, 304, 80])
        wpc = r.choice([4, 8, 12, 16])
        d = B.make_desc(G * hkv, hkv, D, dt, max_batch=64, max_context_len=1 << 20)
        p = B.pa_decode_plan_query(d, cus, wpc, batch, max_ctx, window, S)
        what = (D, dt, hkv, G, batch, max_ctx, window, S, cus, wpc, p.as_dict())
        assert p.partition_size > 0 and p.partition_size % 16 == 0, what
        if S:
            assert p.partition_size == S, what
        elif p.split:
            assert p.partition_size <= 4 * 256 * 16, what
        for n in {0, 1, max_ctx // 3, max_ctx - 1, max_ctx}:
            if 0 <= n <= max_ctx:
                assert covered(p, n, window), what
        assert p.split == (1 if p.num_partitions > 1 else 0), what
        assert p.waves_per_partition in (1, 2, 4), what
        assert p.waves_per_group % p.waves_per_partition == 0, what
        slots = p.waves_per_group // p.waves_per_partition
        assert p.grid_partial[0] == -(-p.num_partitions // slots), what
        assert list(p.grid_partial[1:]) == [hkv, batch], what
        assert p.block_partial == 64 * p.waves_per_group, what
        if p.split:
            assert p.workspace_bytes >= batch * G * hkv * p.num_partitions * (D + 2) * 4, what
        else:
            assert p.workspace_bytes == 0, what
