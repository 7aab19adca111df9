"""Helpers for the GPU parity tests: device upload, the tolerance of the
parity bar, and structured-input builders (needles, ramps)."""
from __future__ import annotations

import math

import numpy as np
import torch

# Parity bar for attention outputs on bf16 (or fp32) inputs with fp32
# accumulation: max |out - oracle| <= OUT_RTOL * max|V| over the attended
# V entries of the batch, and |lse - oracle| <= LSE_ATOL.
OUT_RTOL = 2e-3
LSE_ATOL = 1e-4


def have_gpu() -> bool:
    return torch.cuda.is_available()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")


def attended_vmax_contig(v_cache: torch.Tensor, lengths) -> float:
    """max |V| over positions < length of each sequence (contiguous cache)."""
    B = v_cache.shape[0]
    m = 0.0
    for b in range(B):
        L = int(lengths[b])
        if L > 0:
            m = max(m, float(v_cache[b, :, :L].float().abs().max()))
    return m


def attended_vmax_paged(v_pool: torch.Tensor, block_table: torch.Tensor, lengths, bs: int) -> float:
    m = 0.0
    for b in range(block_table.shape[0]):
        L = int(lengths[b])
        nblk = (L + bs - 1) // bs
        for lb in range(nblk):
            n = min(bs, L - lb * bs)
            phys = int(block_table[b, lb])
            m = max(m, float(v_pool[phys, :, :n].float().abs().max()))
    return m


def check_parity(out, lse, ref_out, ref_lse, vmax: float, what: str = ""):
    """Assert the parity bar; returns (max out error / vmax, max lse error)."""
    o = out.detach().cpu().double().numpy()
    l = lse.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(l)), f"{what}: lse finiteness differs"
    assert np.all(l[~fin] == ref_lse[~fin]), f"{what}: lse of empty rows must be -inf"
    err_o = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    err_l = float(np.max(np.abs(l[fin] - ref_lse[fin]))) if fin.any() else 0.0
    bar = OUT_RTOL * max(vmax, 1e-30)
    assert err_o <= bar, f"{what}: max|out err| {err_o:.3e} > {bar:.3e} (vmax {vmax:.3g})"
    assert err_l <= LSE_ATOL, f"{what}: max|lse err| {err_l:.3e} > {LSE_ATOL}"
    return err_o / max(vmax, 1e-30), err_l


def plant_needles_contig(x: dict, positions, alpha: float = 60.0):
    """Make K[b, j, positions[b][j]] point along the sum of the group's
    queries with length alpha, so that this one position dominates every
    query head of the group.  Modifies x['k_cache'] in place (host)."""
    q = x["q"].float()
    B, h, _ = q.shape
    g = x["k_cache"].shape[1]
    m = h // g
    for b in range(B):
        for j in range(g):
            u = q[b, j * m:(j + 1) * m].sum(0)
            u = u / u.norm()
            x["k_cache"][b, j, positions[b][j]] = (alpha * u).to(x["k_cache"].dtype)


def needle_positions(lengths, g: int, special, seed: int):
    """One position per (b, j): cycle through `special` positions (clipped to
    the sequence) and random ones."""
    rng = np.random.default_rng(seed)
    out = []
    k = 0
    for b in range(len(lengths)):
        L = int(lengths[b])
        row = []
        for _ in range(g):
            if k % 2 == 0 and special:
                p = special[(k // 2) % len(special)]
                p = p if p >= 0 else L + p
                p = min(max(p, 0), L - 1)
            else:
                p = int(rng.integers(0, L))
            row.append(p)
            k += 1
        out.append(row)
    return out


def scale_f32(scale: float) -> float:
    return float(np.float32(scale))


def inv_sqrt(d: int) -> float:
    return 1.0 / math.sqrt(d)
