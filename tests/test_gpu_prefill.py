"""GPU parity of the multi-row kernel (more than 32 query rows per KV head,
bf16, head_dim 128): many new tokens per sequence attending to a cached
prefix and to each other with the bottom-right causal mask (a prefill chunk
after a prefix hit, or draft tokens checked at once), and more than 32
query heads per KV head.

* Ragged batches (length 0, 1, tile edges, lengths past one LDS table
  window) on all three work-group shapes (16 rows per wavefront with four
  wavefronts; 32 with four; 256-row blocks of eight wavefronts, with a
  last block only partly filled), contiguous and paged, automatic and
  fixed splits, with NaN in every unwritten slot: every output row against
  the oracle's multi-token definition (itself pinned to a full causal
  forward).
* Sliding windows and ring caches with many new tokens.
* The 70B GQA shape (B = 32, h = 64, g = 8, 4096 cached positions) with
  n = 128 and n = 512 new tokens per sequence, in the launch the benchmark
  times: the cache bytes in full, and attention rows of sampled sequences
  and tokens against the oracle, each computed alone.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import attended_vmax_contig, attended_vmax_paged, check_parity, dev

pytestmark = pytest.mark.gpu

BEFORE = [0, 1, 31, 33, 200, 1000, 4100]


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _to_torch(a: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    if like.dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def _raw(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# (id, h, g, n): rows per KV head (h / g) * n pick the work-group shape
SHAPES = [
    ("rows40_w4", 8, 1, 5),        # 16 rows per wavefront, 4 wavefronts, one block of 64
    ("rows64_w4", 16, 2, 8),       # exactly 64 rows
    ("rows100_nqt2", 4, 4, 100),   # 32 rows per wavefront, 4 wavefronts (128-row block)
    ("rows264_w8", 64, 8, 33),     # 256-row blocks of 8 wavefronts: a second block of 8 rows
    ("rows1024_w8", 16, 2, 128),   # four full 256-row blocks
    ("mqa_heads48", 48, 1, 1),     # one token, 48 query heads per KV head
]


def _case(h, g, n, paged, seed, before=BEFORE, bs=16):
    lens = torch.tensor(before, dtype=torch.int32)
    B = len(before)
    w = W.Workload("pf", B=B, h=h, g=g, d=128, dtype="bf16", seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    q = W.randn((B, h, n, 128), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, 128), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, 128), torch.bfloat16, gen)
    x = W.make_contiguous(w, lengths=lens, t_cap=max(before) + n + 3, fill=float("nan"))
    if paged:
        table, nb = W.make_block_table(lens + n, bs, perm_seed=seed + 2, extra_blocks=2)
        kc = W.scatter_to_pool(x["k_cache"], lens, table, nb, bs, fill=float("nan"))
        vc = W.scatter_to_pool(x["v_cache"], lens, table, nb, bs, fill=float("nan"))
    else:
        table, kc, vc = None, x["k_cache"], x["v_cache"]
    return w, lens, q, k_new, v_new, kc, vc, table


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_append_decode_multi_rows(shape, paged, num_splits):
    name, h, g, n = shape
    _log(f"case prefill {name} n={n} paged={paged} splits={num_splits}")
    bs = 16
    w, before, q, k_new, v_new, kc, vc, table = _case(h, g, n, paged, 1300, bs=bs)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       block_table=dev(table) if paged else None, scale=w.scale,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before, block_table=table)
    assert np.array_equal(_raw(kd), ek) and np.array_equal(_raw(vd), ev), f"{name}: cache"
    k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, w.scale, block_table=table,
                                 block_size=bs)
    after = before + n
    vmax = attended_vmax_paged(v_host, table, after, bs) if paged else \
        attended_vmax_contig(v_host, after)
    e = check_parity(out, lse, ro, rl, vmax, name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[3], SHAPES[5]],
                         ids=[SHAPES[0][0], SHAPES[3][0], SHAPES[5][0]])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_multi_rows_over_filled_cache(shape, paged):
    """The new tokens are already in the cache; seq_lens counts them."""
    name, h, g, n = shape
    _log(f"case prefill_filled {name} paged={paged}")
    w, before, q, k_new, v_new, kc, vc, table = _case(h, g, n, paged, 1310)
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before, block_table=table)
    k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    out, lse = kvc.decode_multi(dev(q), dev(k_host), dev(v_host), dev(before + n),
                                block_table=dev(table) if paged else None, scale=w.scale)
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, w.scale, block_table=table,
                                 block_size=16)
    after = before + n
    vmax = attended_vmax_paged(v_host, table, after, 16) if paged else \
        attended_vmax_contig(v_host, after)
    check_parity(out, lse, ro, rl, vmax, name)


@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
@pytest.mark.parametrize("window", [1, 40, 700])
def test_window_many_tokens(layout, window):
    """64 new tokens per sequence under a sliding window (rows of 2 heads x
    64 tokens = 128 per KV head)."""
    ring, paged = layout == "ring", layout == "paged"
    h, g, n, bs = 4, 2, 64, 16
    _log(f"case prefill_window {layout} W={window}")
    before = torch.tensor([0, 5, 64, 700, 3000], dtype=torch.int32)
    B = len(before)
    gen = torch.Generator().manual_seed(1320 + window)
    q = W.randn((B, h, n, 128), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, 128), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, 128), torch.bfloat16, gen)
    nan = float("nan")
    if ring:
        t_cap = window + n - 1 + 5
        k = W.randn((B, g, t_cap, 128), torch.bfloat16, gen)
        v = W.randn((B, g, t_cap, 128), torch.bfloat16, gen)
        table = None
    else:
        t_cap = int(before.max()) + n + 3
        k = torch.full((B, g, t_cap, 128), nan, dtype=torch.bfloat16)
        v = k.clone()
        for b in range(B):  # only positions some token of b sees are written
            lo = max(0, int(before[b]) + 1 - window)
            k[b, :, lo:int(before[b])] = W.randn((g, int(before[b]) - lo, 128), torch.bfloat16, gen)
            v[b, :, lo:int(before[b])] = W.randn((g, int(before[b]) - lo, 128), torch.bfloat16, gen)
        table = None
        if paged:
            table, nb = W.make_block_table(before + n, bs, perm_seed=1330, extra_blocks=2)
            kp = W.scatter_to_pool(k, before, table, nb, bs, fill=nan)
            vp = W.scatter_to_pool(v, before, table, nb, bs, fill=nan)
            for b in range(B):
                lo = max(0, int(before[b]) + 1 - window)
                table[b, : lo // bs] = -1
            k, v = kp, vp
    kd, vd = dev(k), dev(v)
    out, lse = kvc.decode_window(dev(q), kd, vd, dev(before), window, ring=ring,
                                 block_table=dev(table) if paged else None,
                                 k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    ek, ev = oracle.append_window(k_new, v_new, k, v, before, ring=ring, block_table=table)
    assert np.array_equal(_raw(kd), ek.view(np.uint16)) and np.array_equal(_raw(vd), ev.view(np.uint16))
    k_host, v_host = _to_torch(ek, k), _to_torch(ev, v)
    ro, rl = oracle.decode_window(q, k_host, v_host, before, 128 ** -0.5, window, ring=ring,
                                  block_table=table)
    vmax = 0.0
    for b in range(B):
        hi = int(before[b]) + n
        for p in range(max(0, int(before[b]) + 1 - window), hi):
            if paged:
                row = v_host[int(table[b, p // bs]), :, p % bs]
            else:
                row = v_host[b, :, p % t_cap if ring else p]
            vmax = max(vmax, float(row.float().abs().max()))
    e = check_parity(out, lse, ro, rl, vmax, f"window {layout}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("n", [128, 512])
def test_full_size_70b_many_tokens(n):
    """The 70B GQA shape with n new tokens per sequence (a prefill chunk
    after a 4096-position prefix), in the benchmark's launch: the whole
    cache after the step, and the attention rows of sampled sequences and
    tokens against the oracle, each computed alone."""
    _log(f"case prefill_full_70b n={n}")
    w = W.WORKLOADS["gqa_70b_bf16"]
    x = W.make_contiguous(w, t_cap=w.T + n + w.cap_pad)
    gen = torch.Generator().manual_seed(1340 + n)
    q = W.randn((w.B, w.h, n, w.d), w.torch_dtype, gen)
    k_new = W.randn((w.B, w.g, n, w.d), w.torch_dtype, gen)
    v_new = W.randn((w.B, w.g, n, w.d), w.torch_dtype, gen)
    before = x["seq_lens_before"]
    kd, vd = dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       scale=x["scale"])
    torch.cuda.synchronize()
    # the append: the n new rows at positions T .. T+n-1, nothing else touched
    k_host, v_host = x["k_cache"].clone(), x["v_cache"].clone()
    k_host[:, :, w.T:w.T + n] = k_new
    v_host[:, :, w.T:w.T + n] = v_new
    assert torch.equal(kd.cpu().view(torch.int16), k_host.view(torch.int16))
    assert torch.equal(vd.cpu().view(torch.int16), v_host.view(torch.int16))
    out_h, lse_h = out.cpu(), lse.cpu()
    seqs = [0, 13, 31]
    tokens = sorted({0, 1, 31, 32, n // 2, n - 2, n - 1})
    for t in tokens:
        vis = before[seqs] + t + 1
        ro, rl = oracle.decode(q[seqs, :, t].contiguous(), k_host[seqs], v_host[seqs], vis,
                               x["scale"])
        e = check_parity(out_h[seqs, :, t], lse_h[seqs, :, t], ro, rl,
                         attended_vmax_contig(v_host[seqs], vis), f"70b n={n} t={t}")
    _log(f"  last sampled token err/vmax {e[0]:.2e} lse {e[1]:.2e}")
    assert torch.isfinite(out_h).all() and torch.isfinite(lse_h).all()
