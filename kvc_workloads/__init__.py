"""Seeded synthetic decode-step inputs shared by the GPU tests, the oracle
tests and the benchmark.

This module holds workload shapes and random-number plumbing only: it draws
q, K, V and the new token's K/V, lays caches out contiguously or in a paged
pool, and builds block tables.  It contains none of the attention arithmetic
and imports neither the oracle nor the GPU library.

Recipe (every workload): values are drawn in float32 from N(0, 1) with a
``torch.Generator`` seeded per workload, then cast once to the workload dtype
(round-to-nearest-even for bf16), so the oracle and the GPU see identical
bits.  Cache slots at or beyond a sequence's length are filled with
``fill`` (0 by default; NaN or a large finite value in the masking tests).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import torch

BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h: int
    g: int
    d: int
    dtype: str                     # "f32" or "bf16"
    T: Optional[int] = None        # cached length before the step (uniform lengths)
    T_range: Optional[Tuple[int, int]] = None  # inclusive range for per-sequence lengths
    paged: bool = False
    block_size: int = BLOCK_SIZE
    cap_pad: int = 16              # contiguous capacity = T + cap_pad
    num_splits: int = 0            # 0 = library chooses
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def m(self) -> int:
        return self.h // self.g

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five decode workloads.  T is the cached length before the step; one new
# token is appended, so every sequence attends to T + 1 positions.
WORKLOADS = {
    "tiny_gqa_f32": Workload("tiny_gqa_f32", B=1, h=4, g=2, d=16, dtype="f32", T=32, seed=1000),
    "mha_7b_bf16": Workload("mha_7b_bf16", B=8, h=32, g=32, d=128, dtype="bf16", T=2048,
                            seed=1001),
    "gqa_70b_bf16": Workload("gqa_70b_bf16", B=32, h=64, g=8, d=128, dtype="bf16", T=4096,
                             seed=1002),
    "paged_gqa_bf16": Workload("paged_gqa_bf16", B=64, h=32, g=8, d=128, dtype="bf16",
                               T_range=(128, 8192), paged=True, seed=2000),
    "long_mqa_bf16": Workload("long_mqa_bf16", B=4, h=32, g=1, d=128, dtype="bf16", T=131072,
                              num_splits=64, seed=1004),
}

# The d = 1 hand-computed example: prefilled K = [1, 2], V = [10, 20]; the
# third token has q = 1, k = 0, v = 30; scale 1.
D1_EXAMPLE = dict(k_prefill=[1.0, 2.0], v_prefill=[10.0, 20.0], q=1.0, k_new=0.0, v_new=30.0,
                  scale=1.0)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def randn(shape, dtype, gen: torch.Generator) -> torch.Tensor:
    """float32 N(0,1) draw cast once to ``dtype`` (CPU)."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def seq_lengths(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """Cached lengths before the step, int32 [B]."""
    if w.T_range is None:
        return torch.full((w.B,), w.T, dtype=torch.int32)
    lo, hi = w.T_range
    return torch.randint(lo, hi + 1, (w.B,), generator=_gen(w.seed if seed is None else seed),
                         dtype=torch.int64).to(torch.int32)


def make_contiguous(w: Workload, seed: Optional[int] = None, lengths: Optional[torch.Tensor] = None,
                    t_cap: Optional[int] = None, fill: float = 0.0) -> dict:
    """Host tensors for one decode step on a contiguous [B, g, t_cap, d] cache.

    Returns q [B,h,d], k_cache/v_cache [B,g,t_cap,d] (positions < len filled),
    k_new/v_new [B,g,d], seq_lens_before (int32 [B]), seq_lens_after = +1,
    scale, t_cap."""
    gen = _gen(w.seed if seed is None else seed)
    dt = w.torch_dtype
    lens = seq_lengths(w, seed) if lengths is None else lengths.to(torch.int32)
    max_len = int(lens.max().item()) if lens.numel() else 0
    cap = (max_len + w.cap_pad) if t_cap is None else t_cap
    q = randn((w.B, w.h, w.d), dt, gen)
    k_cache = randn((w.B, w.g, cap, w.d), dt, gen)
    v_cache = randn((w.B, w.g, cap, w.d), dt, gen)
    k_new = randn((w.B, w.g, w.d), dt, gen)
    v_new = randn((w.B, w.g, w.d), dt, gen)
    pos = torch.arange(cap).view(1, 1, cap, 1)
    unwritten = pos >= lens.view(-1, 1, 1, 1).to(torch.int64)
    k_cache.masked_fill_(unwritten, fill)
    v_cache.masked_fill_(unwritten, fill)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                seq_lens_before=lens.clone(), seq_lens_after=(lens + 1).to(torch.int32),
                scale=w.scale, t_cap=cap)


def block_counts(lengths: torch.Tensor, block_size: int) -> torch.Tensor:
    """Blocks each sequence owns so that it can hold ``lengths`` tokens."""
    return (lengths.to(torch.int64) + block_size - 1) // block_size


def make_block_table(capacity_lens: torch.Tensor, block_size: int, perm_seed: int,
                     max_blocks: Optional[int] = None, extra_blocks: int = 0):
    """Random physical placement: NB = sum of per-sequence block counts
    (+ extra unused blocks); physical ids are a seeded random permutation of
    range(NB), handed out in (sequence, logical block) order.  Unused table
    entries are -1.  Returns (block_table int32 [B, max_blocks], NB)."""
    n = block_counts(capacity_lens, block_size)
    nb = int(n.sum().item()) + extra_blocks
    mb = int(n.max().item()) if max_blocks is None else max_blocks
    mb = max(mb, 1)
    perm = torch.randperm(nb, generator=_gen(perm_seed)).to(torch.int32)
    table = torch.full((capacity_lens.numel(), mb), -1, dtype=torch.int32)
    nxt = 0
    for b in range(capacity_lens.numel()):
        cnt = int(n[b].item())
        table[b, :cnt] = perm[nxt:nxt + cnt]
        nxt += cnt
    return table, nb


def scatter_to_pool(cache: torch.Tensor, lengths: torch.Tensor, block_table: torch.Tensor,
                    num_blocks: int, block_size: int, fill: float = 0.0) -> torch.Tensor:
    """Copy positions < lengths[b] of a contiguous cache [B, g, T, d] into a
    pool [num_blocks, g, block_size, d] laid out by ``block_table``; all other
    pool slots hold ``fill``."""
    B, g, _, d = cache.shape
    pool = torch.full((num_blocks, g, block_size, d), fill, dtype=cache.dtype)
    for b in range(B):
        L = int(lengths[b].item())
        for lb in range((L + block_size - 1) // block_size):
            p0 = lb * block_size
            p1 = min(p0 + block_size, L)
            phys = int(block_table[b, lb].item())
            pool[phys, :, : p1 - p0, :] = cache[b, :, p0:p1, :]
    return pool


def make_paged(w: Workload, seed: Optional[int] = None, lengths: Optional[torch.Tensor] = None,
               fill: float = 0.0, max_blocks: Optional[int] = None, new_tokens: int = 1) -> dict:
    """Host tensors for one decode step on a paged pool.

    Lengths before the step are ``lengths`` (or drawn from w.T_range with
    w.seed); every sequence owns ceil((len + new_tokens) / block_size) blocks
    so that the appended tokens have slots (k_new / v_new below hold one).
    Physical blocks are a random permutation (seed w.seed + 1).  Pool slots
    at positions >= len hold ``fill``.
    Returns q, k_pool, v_pool [NB,g,bs,d], block_table [B,max_blocks],
    k_new, v_new, seq_lens_before, seq_lens_after, scale, num_blocks."""
    s = w.seed if seed is None else seed
    gen = _gen(s + 7)
    dt = w.torch_dtype
    bs = w.block_size
    lens = seq_lengths(w, s) if lengths is None else lengths.to(torch.int32)
    table, nb = make_block_table(lens + new_tokens, bs, perm_seed=s + 1, max_blocks=max_blocks)
    q = randn((w.B, w.h, w.d), dt, gen)
    k_pool = randn((nb, w.g, bs, w.d), dt, gen)
    v_pool = randn((nb, w.g, bs, w.d), dt, gen)
    k_new = randn((w.B, w.g, w.d), dt, gen)
    v_new = randn((w.B, w.g, w.d), dt, gen)
    # Blank the unwritten tail slots of each sequence's last block(s).
    for b in range(w.B):
        L = int(lens[b].item())
        nblk = int(((L + new_tokens + bs - 1) // bs))
        for lb in range(L // bs, nblk):
            phys = int(table[b, lb].item())
            first = max(L - lb * bs, 0)
            k_pool[phys, :, first:, :] = fill
            v_pool[phys, :, first:, :] = fill
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, k_new=k_new, v_new=v_new,
                seq_lens_before=lens.clone(), seq_lens_after=(lens + 1).to(torch.int32),
                scale=w.scale, num_blocks=nb, block_size=bs)
