"""Seeded synthetic inputs for paged-KV GQA decode attention.

This module only draws numbers and lays them out in a paged cache; it holds
none of the attention arithmetic, and both the HIP path's tests/benchmark and
the oracle's tests take their inputs from it.

Recipe (every tensor is drawn on the CPU from one ``torch.Generator`` seeded
with the workload's seed, in this order):
  1. context lengths (only for workloads with random lengths),
  2. q       ~ N(0, 1) in float32, shape [B, Hq, D],
  3. logical K ~ N(0, 1) in float32, shape [B, n_max, Hkv, D],
  4. logical V ~ N(0, 1) in float32, same shape,
  5. a random permutation of the physical page pool,
  6. the filler of unused pool pages and tail slots ~ N(0, 1)
     (or NaN in the poison variant, which any read of a masked slot exposes).
Values are then rounded to nearest-even into the workload dtype.  Sequence b
takes the next ceil(n_b / page_size) entries of the permutation as its page
table row, so its pages are scattered across the pool; logical token j of
sequence b lands in page table[b][j // page_size], slot j % page_size.

The workloads mirror the page's decode shapes: a tiny GQA-4 fp32 case, a
Llama-3.2-1B-shaped batch-1 decode at 3060 tokens (the context of the
sequence-sharded nest's measurements, TVM PR #20426 section "Measurements"),
a Llama-3.1-8B-shaped batch of 16 with ragged lengths, head_dim 256 with a
sliding window, and a 100,000-token GQA-6 context cut into 512-token
partitions (the paged_attention_v2_pytorch.py commit page's 100K example).
The ``*_rope_f16`` variants are the same inputs with the rotary embedding
switched on (rope_theta 500000, rope_scale 1): the cache holds keys before the
embedding, which the kernel applies as it reads them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    context_lens: Optional[List[int]]   # None: drawn (see random_lens)
    num_pages: int                      # size of the physical page pool
    seed: int
    window: int = 0                     # <= 0: no sliding window
    partition_size: int = 0             # 0: the library chooses; BALANCED: the
                                        # length-balanced schedule
    page_size: int = PAGE_SIZE
    random_lens: Optional[tuple] = None  # (lo, hi, forced{index: len}) for drawn lengths
    rope: Optional[tuple] = None        # (rope_theta, rope_scale): rotary_mode 1; None: off

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim) rounded to float32 (the value both sides use)."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


# partition_size of the length-balanced schedule (PA_DECODE_PARTITION_BALANCED):
# the ragged batches below run with it, as a caller who knows its batch is
# ragged would (the planner's automatic choice keeps fixed partitions, which
# suit batches of equal lengths better).
BALANCED = -1

CONFIGS = {
    "tiny_gqa4_f32": Workload(
        name="tiny_gqa4_f32", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
        dtype=torch.float32, context_lens=[300], num_pages=19, seed=1),
    "llama1b_ctx3060_f16": Workload(
        name="llama1b_ctx3060_f16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=64,
        dtype=torch.float16, context_lens=[3060], num_pages=4096, seed=2),
    "llama8b_b16_ragged_f16": Workload(
        name="llama8b_b16_ragged_f16", batch=16, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype=torch.float16, context_lens=None, num_pages=4096, seed=3,
        random_lens=(1, 4096, {0: 1, 1: 4096, 2: 17}), partition_size=BALANCED),
    "d256_window4096_bf16": Workload(
        name="d256_window4096_bf16", batch=4, num_q_heads=8, num_kv_heads=4, head_dim=256,
        dtype=torch.bfloat16, context_lens=[8192] * 4, num_pages=2048, seed=4,
        window=4096),
    "ctx100k_gqa6_f16": Workload(
        name="ctx100k_gqa6_f16", batch=1, num_q_heads=24, num_kv_heads=4, head_dim=256,
        dtype=torch.float16, context_lens=[100000], num_pages=6250, seed=5,
        partition_size=512),
    # head_dim 96 (not one of the five; measures the 12-chunk-row path)
    "d96_b16_ragged_f16": Workload(
        name="d96_b16_ragged_f16", batch=16, num_q_heads=32, num_kv_heads=8, head_dim=96,
        dtype=torch.float16, context_lens=None, num_pages=4096, seed=6,
        random_lens=(1, 4096, {0: 1, 1: 4096, 2: 17}), partition_size=BALANCED),
    "d96_ctx32k_f16": Workload(
        name="d96_ctx32k_f16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=96,
        dtype=torch.float16, context_lens=[32768], num_pages=2048, seed=7),
}

# head_dim 128 at one long context (Llama-3.1-8B heads, 32768 tokens).
CONFIGS["llama8b_ctx32k_f16"] = Workload(
    name="llama8b_ctx32k_f16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
    dtype=torch.float16, context_lens=[32768], num_pages=2048, seed=8)

# The windowed head_dim-256 shape at batch 8 (a window's partitions sit on
# multiples of S, so the planner sizes them with one partition to spare).
CONFIGS["d256_window4096_b8_bf16"] = dataclasses.replace(
    CONFIGS["d256_window4096_bf16"], name="d256_window4096_b8_bf16", batch=8,
    context_lens=[8192] * 8, num_pages=4096, seed=9)

# Uniform serving-style batches of Llama-3.1-8B heads (fixed partitions).
CONFIGS["llama8b_b64_ctx1000_f16"] = Workload(
    name="llama8b_b64_ctx1000_f16", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
    dtype=torch.float16, context_lens=[1000] * 64, num_pages=64 * 63, seed=10)
CONFIGS["llama8b_b32_ctx2048_f16"] = Workload(
    name="llama8b_b32_ctx2048_f16", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
    dtype=torch.float16, context_lens=[2048] * 32, num_pages=32 * 128, seed=11)

# Rotary embedding in the kernel (rotary_mode 1; TVM PR #20426, "Correctness"),
# with the frequency base 500000 of the Llama 3.x models the PR measures.
for _base in ("llama1b_ctx3060_f16", "llama8b_b16_ragged_f16", "ctx100k_gqa6_f16",
              "llama8b_ctx32k_f16"):
    _w = CONFIGS[_base]
    _name = _base[:-len("_f16")] + "_rope_f16"
    CONFIGS[_name] = dataclasses.replace(_w, name=_name, rope=(500000.0, 1.0))

# The five workloads in the order they are usually listed.
CONFIG_ORDER = ["tiny_gqa4_f32", "llama1b_ctx3060_f16", "llama8b_b16_ragged_f16",
                "d256_window4096_bf16", "ctx100k_gqa6_f16"]
# Further shapes (head_dim 96; rotary embedding; a larger windowed batch; uniform
# serving batches), measured but not part of the five.
EXTRA_ORDER = ["d96_b16_ragged_f16", "d96_ctx32k_f16", "llama8b_ctx32k_f16",
               "llama1b_ctx3060_rope_f16", "llama8b_b16_ragged_rope_f16",
               "ctx100k_gqa6_rope_f16", "llama8b_ctx32k_rope_f16", "d256_window4096_b8_bf16",
               "llama8b_b64_ctx1000_f16", "llama8b_b32_ctx2048_f16"]


@dataclasses.dataclass
class Problem:
    """One decode-attention problem in CPU memory."""
    workload: Workload
    q: torch.Tensor             # [B, Hq, D]
    k_cache: torch.Tensor       # [num_pages, Hkv, page_size, D]
    v_cache: torch.Tensor       # [num_pages, Hkv, page_size, D]
    page_table: torch.Tensor    # int32 [B, pt_stride]
    context_lens: torch.Tensor  # int32 [B]
    scale: float
    window: int
    logical_k: Optional[torch.Tensor] = None  # [B, n_max, Hkv, D], workload dtype
    logical_v: Optional[torch.Tensor] = None

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.context_lens.numel() else 0

    def visible_tokens(self) -> int:
        """Sum over sequences of the number of keys attended to."""
        tot = 0
        for n in self.context_lens.tolist():
            lo = n - self.window if (self.window > 0 and n > self.window) else 0
            tot += n - lo
        return tot

    def kv_bytes(self) -> int:
        """K and V bytes of the visible keys: the algorithmic HBM traffic of a step."""
        w = self.workload
        return self.visible_tokens() * w.num_kv_heads * w.head_dim * \
            torch.tensor([], dtype=w.dtype).element_size() * 2


def draw_lengths(w: Workload, gen: torch.Generator) -> List[int]:
    if w.context_lens is not None:
        return list(w.context_lens)
    lo, hi, forced = w.random_lens
    lens = torch.randint(lo, hi + 1, (w.batch,), generator=gen).tolist()
    for i, n in forced.items():
        lens[i] = n
    return lens


def generate(w: Workload, seed: Optional[int] = None, poison: bool = False,
             keep_logical: bool = False, context_lens: Optional[List[int]] = None,
             extra_pages: int = 0) -> Problem:
    """Draw one problem for workload ``w``.

    ``poison`` fills every slot the method must not read (tail slots of the last
    page, keys before the sliding window, unused pool pages) with NaN, and points
    the page-table padding at a NaN page.  ``context_lens`` overrides the
    workload's lengths (the pool grows if needed).  ``extra_pages`` adds unused
    pages to the pool.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    lens = list(context_lens) if context_lens is not None else draw_lengths(w, gen)
    B, Hq, Hkv, D = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    assert len(lens) == B
    n_max = max(lens) if lens else 0
    q = torch.randn((B, Hq, D), generator=gen, dtype=torch.float32)
    lk = torch.randn((B, n_max, Hkv, D), generator=gen, dtype=torch.float32)
    lv = torch.randn((B, n_max, Hkv, D), generator=gen, dtype=torch.float32)
    return paginate(w, q.to(w.dtype), lk.to(w.dtype), lv.to(w.dtype), lens, gen,
                    poison=poison, keep_logical=keep_logical, extra_pages=extra_pages)


def paginate(w: Workload, q: torch.Tensor, lk: torch.Tensor, lv: torch.Tensor,
             lens: List[int], gen: torch.Generator, poison: bool = False,
             keep_logical: bool = False, extra_pages: int = 0) -> Problem:
    """Scatter logical K/V [B, n_max, Hkv, D] into a shuffled page pool.

    Draws the page permutation, then the filler of unused slots (N(0, 1), or
    NaN when ``poison``), from ``gen``.
    """
    B, Hkv, D, ps = w.batch, w.num_kv_heads, w.head_dim, w.page_size
    pages_per_seq = [(n + ps - 1) // ps for n in lens]
    used = sum(pages_per_seq)
    num_pages = max(w.num_pages, used) + extra_pages
    if poison and num_pages == used:
        num_pages += 1  # a NaN page for the page-table padding to point at
    perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
    if poison:
        k_cache = torch.full((num_pages, Hkv, ps, D), float("nan")).to(w.dtype)
        v_cache = torch.full((num_pages, Hkv, ps, D), float("nan")).to(w.dtype)
    else:
        k_cache = torch.randn((num_pages, Hkv, ps, D), generator=gen).to(w.dtype)
        v_cache = torch.randn((num_pages, Hkv, ps, D), generator=gen).to(w.dtype)

    pt_stride = max(1, max(pages_per_seq) if pages_per_seq else 1)
    page_table = torch.zeros((B, pt_stride), dtype=torch.int32)
    off = 0
    for b in range(B):
        k = pages_per_seq[b]
        page_table[b, :k] = perm[off:off + k]
        off += k
    # Padding entries point at a page no sequence uses when there is one.
    pad_page = int(perm[used]) if used < num_pages else 0
    for b in range(B):
        page_table[b, pages_per_seq[b]:] = pad_page

    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        j = torch.arange(n)
        pages = page_table[b, j // ps].long()
        slots = (j % ps).long()
        # k_cache[page, :, slot, :] = logical[b, j, :, :]
        k_cache[pages, :, slots, :] = lk[b, :n]
        v_cache[pages, :, slots, :] = lv[b, :n]
        if poison and w.window > 0 and n > w.window:
            hidden = torch.arange(n - w.window)
            hp = page_table[b, hidden // ps].long()
            hs = (hidden % ps).long()
            k_cache[hp, :, hs, :] = float("nan")
            v_cache[hp, :, hs, :] = float("nan")
    return Problem(
        workload=w, q=q.contiguous(), k_cache=k_cache, v_cache=v_cache,
        page_table=page_table, context_lens=torch.tensor(lens, dtype=torch.int32),
        scale=w.scale, window=w.window,
        logical_k=lk if keep_logical else None, logical_v=lv if keep_logical else None)


def custom(name="custom", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
           dtype=torch.float16, context_lens=(100,), num_pages=0, seed=0, window=0,
           partition_size=0, page_size=PAGE_SIZE, rope=None) -> Workload:
    """A workload with explicit sizes (used for parity sweeps and edge cases)."""
    lens = list(context_lens)
    assert len(lens) == batch
    need = sum((n + page_size - 1) // page_size for n in lens)
    return Workload(name=name, batch=batch, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, dtype=dtype,
                    context_lens=lens, num_pages=max(num_pages, need, 1), seed=seed,
                    window=window, partition_size=partition_size, page_size=page_size,
                    rope=rope)


def permute_pages(p: Problem, seed: int) -> Problem:
    """The same logical problem with its physical pages moved to new slots.

    Page i of the pool moves to slot perm[i] and the page table is remapped, so
    every sequence still sees the same keys in the same order.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    num_pages = p.k_cache.shape[0]
    perm = torch.randperm(num_pages, generator=gen)
    k = torch.empty_like(p.k_cache)
    v = torch.empty_like(p.v_cache)
    k[perm] = p.k_cache
    v[perm] = p.v_cache
    pt = perm.to(torch.int32)[p.page_table.long()]
    return dataclasses.replace(p, k_cache=k, v_cache=v, page_table=pt)


@dataclasses.dataclass
class CsrTable:
    """A page table in CSR form: sequence b owns pages
    indices[indptr[b]:indptr[b+1]] in token order, the last holding
    last_page_len[b] tokens."""
    indptr: torch.Tensor         # int32 [B + 1]
    indices: torch.Tensor        # int32 [nnz_pages]
    last_page_len: torch.Tensor  # int32 [B]

    @property
    def nnz_pages(self) -> int:
        return int(self.indptr[-1].item())


def to_csr(p: Problem, page_size: int = 16) -> CsrTable:
    """The CSR form of a problem's dense page table (rows cut to
    ceil(n_b / page_size) pages)."""
    lens = p.context_lens.tolist()
    counts = [(n + page_size - 1) // page_size for n in lens]
    indptr = [0]
    for c in counts:
        indptr.append(indptr[-1] + c)
    indices = [int(x) for b, c in enumerate(counts) for x in p.page_table[b, :c].tolist()]
    last = [n - (c - 1) * page_size if c > 0 else 0 for n, c in zip(lens, counts)]
    return CsrTable(torch.tensor(indptr, dtype=torch.int32),
                    torch.tensor(indices, dtype=torch.int32),
                    torch.tensor(last, dtype=torch.int32))


def from_csr(csr: CsrTable, page_size: int = 16):
    """(page_table [B, max_pages] int32, context_lens [B] int32) of a CSR table."""
    ip = csr.indptr.tolist()
    counts = [ip[b + 1] - ip[b] for b in range(len(ip) - 1)]
    width = max(1, max(counts) if counts else 1)
    pt = torch.zeros((len(counts), width), dtype=torch.int32)
    lens = []
    for b, c in enumerate(counts):
        pt[b, :c] = csr.indices[ip[b]:ip[b + 1]]
        last = min(max(int(csr.last_page_len[b]), 0), page_size)
        lens.append((c - 1) * page_size + last if c > 0 else 0)
    return pt, torch.tensor(lens, dtype=torch.int32)
