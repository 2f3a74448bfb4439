"""CPU: the length-balanced schedule's plan and range arithmetic.

* pa_decode_plan_query with partition_size PA_DECODE_PARTITION_BALANCED gives
  a whole number of workgroups per KV head, one wave per range, a state-row
  pitch of min(waves, visible pages), room for the per-(sequence, head)
  counts in the workspace, and refuses batches above 64;
* the range arithmetic the kernel and merge use (each sequence with pages is
  charged C start pages in front of its visible pages; wave w takes the
  charged pages [w T / Weff, (w + 1) T / Weff) of the batch, Weff = min(W, T);
  page x lies in wave ((x + 1) Weff - 1) / T; the visible piece of sequence b
  in wave w is state row w - w0(b), w0(b) the wave of its first visible
  page) is written out here in integers and checked on seeded
  ragged batches against the plans: every visible page lies in exactly one
  range, the pieces of a sequence have rows 0 .. count - 1 with no gap, and
  no count passes the plan's row pitch.
"""
import random

import pytest
import torch

from paged_kv_decode_amd import binding as B
from paged_kv_decode_amd import workloads as W

BAL = B.PA_DECODE_PARTITION_BALANCED
PS = 16


def desc(G=4, hkv=8, D=128, dtype=torch.float16, rope=None):
    return B.make_desc(G * hkv, hkv, D, dtype, max_batch=4096, max_context_len=1 << 20, rope=rope)


def visible_pages(n, window):
    lo = n - window if (window > 0 and n > window) else 0
    return (-(-n // PS)) - lo // PS if n > lo else 0


def schedule(lens, window, W_, C):
    """(sequence, wave, first page, end page, row) pieces and row counts, in
    the kernel's integer arithmetic (C pages charged per sequence start)."""
    pages = [visible_pages(n, window) for n in lens]
    charged = [c + C if c else 0 for c in pages]
    incl, acc = [], 0
    for c in charged:
        acc += c
        incl.append(acc)
    T = acc
    Weff = min(W_, T)
    pieces = []
    for w in range(W_):
        if w >= Weff:
            continue
        A, E = w * T // Weff, (w + 1) * T // Weff
        for b, c in enumerate(charged):
            ex, inn = incl[b] - c, incl[b]
            if c == 0 or inn <= A or ex >= E:
                continue
            r0, r1 = max(A, ex + C), min(E, inn)
            if r0 >= r1:
                continue
            w0 = ((ex + C + 1) * Weff - 1) // T
            pieces.append((b, w, r0 - ex - C, r1 - ex - C, w - w0))
    counts = []
    for b, c in enumerate(charged):
        if c == 0:
            counts.append(0)
            continue
        ex, inn = incl[b] - c, incl[b]
        counts.append((inn * Weff - 1) // T - ((ex + C + 1) * Weff - 1) // T + 1)
    return pages, pieces, counts


def test_balanced_plan_shape():
    for (G, hkv, D, dtype) in [(4, 8, 128, torch.float16), (6, 4, 256, torch.float16),
                               (1, 1, 64, torch.float32), (8, 2, 96, torch.bfloat16)]:
        d = desc(G, hkv, D, dtype)
        for batch, ctx, window in [(16, 4096, 0), (4, 8192, 4096), (64, 3000, 0), (1, 100000, 0),
                                   (3, 20, 0), (2, 100, 7)]:
            p = B.pa_decode_plan_query(d, 256, 8, batch, ctx, window, BAL)
            nw = p.waves_per_group
            W_ = p.balanced_waves
            assert W_ > 0 and W_ % nw == 0 and p.grid_partial[0] * nw == W_
            assert list(p.grid_partial[1:]) == [hkv, 1] and p.block_partial == 64 * nw
            assert p.waves_per_partition == 1 and p.split == 1 and p.partition_size == 0
            windowed = 0 < window < ctx
            vis = -(-(window if windowed else ctx) // PS) + (1 if windowed else 0)
            assert p.num_partitions == min(W_, vis)
            # about four waves per compute unit over all KV heads, never
            # more than the batch's pages
            assert W_ <= max(nw, min(1024 // hkv, batch * vis))
            rows = batch * G * hkv * p.num_partitions
            a = lambda x: (x + 255) // 256 * 256
            want = a(rows * D * 4) + 2 * a(rows * 4) + a(batch * G * hkv * 4)
            assert p.workspace_bytes == want
            # one merge wave per (sequence, head, column slice), whatever the pitch
            cw = 16 if batch * G * hkv * (-(-D // 64)) < 256 else 64
            assert list(p.grid_merge) == [-(-batch * G * hkv * (-(-D // cw)) // 4), 1, 1]


def test_balanced_plan_limits():
    d = desc()
    with pytest.raises(B.PaDecodeError) as e:
        B.pa_decode_plan_query(d, 256, 8, 65, 4096, 0, BAL)
    assert e.value.status == B.PA_DECODE_UNSUPPORTED
    with pytest.raises(B.PaDecodeError) as e:
        B.pa_decode_plan_query(d, 256, 8, 64, 1 << 20, 0, -2)
    assert e.value.status == B.PA_DECODE_INVALID_ARG
    p = B.pa_decode_plan_query(d, 256, 8, 0, 4096, 0, BAL)   # empty batch: nothing to launch
    assert p.balanced_waves == 0
    p = B.pa_decode_plan_query_csr(d, 256, 8, 16, 16 * 200, 0, 0, BAL)
    assert p.balanced_waves > 0


@pytest.mark.parametrize("seed", range(40))
def test_ranges_tile_the_visible_pages(seed):
    r = random.Random(seed)
    batch = r.choice([1, 2, 5, 16, 33, 64])
    lens = [r.choice([0, 1, 16, 17, r.randint(2, 9000)]) for _ in range(batch)]
    ctx = max(lens + [1])
    window = r.choice([0, 0, r.randint(1, 2000)])
    hkv = r.choice([1, 2, 8, 32])
    p = B.pa_decode_plan_query(desc(hkv=hkv), 256, 8, batch, ctx, window, BAL)
    C = r.choice([0, 1, 2, 4, 64])
    pages, pieces, counts = schedule(lens, window, p.balanced_waves, C)
    seen = [[0] * c for c in pages]
    rows = [[] for _ in lens]
    for b, w, a, e, row in pieces:
        assert 0 <= a < e <= pages[b]
        for x in range(a, e):
            seen[b][x] += 1
        rows[b].append(row)
    assert all(all(v == 1 for v in s) for s in seen), "a page is missed or read twice"
    for b in range(batch):
        assert sorted(rows[b]) == list(range(counts[b])), (b, rows[b], counts[b])
        assert counts[b] <= p.num_partitions
    # with no start charge, every wave below Weff has at least one page
    T = sum(pages)
    if T and C == 0:
        assert len({w for _, w, _, _, _ in pieces}) == min(p.balanced_waves, T)
