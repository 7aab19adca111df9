"""GPU parity of bf16 caches with head dimension 64, 80, 96 and 256, which run
on the multi-row matrix-core kernel for every row count (one K/V read per KV head;
rows = query heads per KV head x new tokens):

* one query row (MHA) up to 320 rows per KV head (the four work-group
  shapes), one and several new tokens, appended in the same call, over
  ragged batches (length 0, 1, tile edges, past one LDS table window), with
  NaN in every unwritten slot, contiguous and paged, automatic and fixed
  splits: every output row against the oracle's multi-token definition;
* sliding windows over linear, ring and paged caches.
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
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)


def _raw(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# (id, h, g, n): rows per KV head = (h / g) * n
SHAPES = [
    ("mha_rows1", 4, 4, 1),
    ("gqa_rows4", 8, 2, 1),
    ("gqa_rows8_n2", 8, 2, 2),
    ("rows40", 8, 1, 5),
    ("rows96", 4, 2, 48),
    ("rows320", 32, 2, 20),
]


def _case(h, g, n, d, paged, seed, before=BEFORE, bs=16):
    lens = torch.tensor(before, dtype=torch.int32)
    B = len(before)
    w = W.Workload("hd", B=B, h=h, g=g, d=d, dtype="bf16", seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    x = W.make_contiguous(w, lengths=lens, t_cap=max(before) + n + 3, fill=float("nan"))
    if paged:
        table, nb = W.make_block_table(lens + n, bs, perm_seed=seed + 2, extra_blocks=2)
        kc = W.scatter_to_pool(x["k_cache"], lens, table, nb, bs, fill=float("nan"))
        vc = W.scatter_to_pool(x["v_cache"], lens, table, nb, bs, fill=float("nan"))
    else:
        table, kc, vc = None, x["k_cache"], x["v_cache"]
    return w, lens, q, k_new, v_new, kc, vc, table


@pytest.mark.parametrize("d", [64, 80, 96, 256])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_append_decode_head_dims(d, shape, paged, num_splits):
    name, h, g, n = shape
    _log(f"case headdim d={d} {name} paged={paged} splits={num_splits}")
    bs = 16
    w, before, q, k_new, v_new, kc, vc, table = _case(h, g, n, d, paged, 1600 + d, bs=bs)
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
    e = check_parity(out, lse, ro, rl, vmax, f"d={d} {name}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("d", [64, 80, 96, 256])
@pytest.mark.parametrize("shape", [SHAPES[1], SHAPES[4]], ids=[SHAPES[1][0], SHAPES[4][0]])
def test_decode_head_dims_over_filled_cache(d, shape):
    """The new tokens already in the cache; seq_lens counts them.  One token:
    the two-call form (kvc_append, then the decode call); several: the cache
    filled on the host."""
    name, h, g, n = shape
    _log(f"case headdim_filled d={d} {name}")
    w, before, q, k_new, v_new, kc, vc, table = _case(h, g, n, d, False, 1610 + d)
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before)
    k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    if n == 1:
        kd, vd = dev(kc), dev(vc)
        kvc.append(dev(k_new[:, :, 0].contiguous()), dev(v_new[:, :, 0].contiguous()), kd, vd,
                   dev(before))
    else:
        kd, vd = dev(k_host), dev(v_host)
    out, lse = kvc.decode_multi(dev(q), kd, vd, dev(before + n), scale=w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(_raw(kd), ek) and np.array_equal(_raw(vd), ev)
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, w.scale)
    check_parity(out, lse, ro, rl, attended_vmax_contig(v_host, before + n), f"d={d} {name}")


@pytest.mark.parametrize("d", [64, 80, 96, 256])
@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
@pytest.mark.parametrize("window,n", [(1, 1), (40, 4), (300, 33)])
def test_window_head_dims(d, layout, window, n):
    ring, paged = layout == "ring", layout == "paged"
    h, g, bs = 4, 2, 16
    _log(f"case headdim_window d={d} {layout} W={window} n={n}")
    before = torch.tensor([0, 5, 64, 700, 3000], dtype=torch.int32)
    B = len(before)
    gen = torch.Generator().manual_seed(1620 + window + d)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    nan = float("nan")
    if ring:
        t_cap = window + n - 1 + 5
        k = W.randn((B, g, t_cap, d), torch.bfloat16, gen)
        v = W.randn((B, g, t_cap, d), torch.bfloat16, gen)
        table = None
    else:
        t_cap = int(before.max()) + n + 3
        k = torch.full((B, g, t_cap, d), nan, dtype=torch.bfloat16)
        v = k.clone()
        for b in range(B):  # only positions some token of b sees are written
            lo = max(0, int(before[b]) + 1 - window)
            k[b, :, lo:int(before[b])] = W.randn((g, int(before[b]) - lo, d), torch.bfloat16, gen)
            v[b, :, lo:int(before[b])] = W.randn((g, int(before[b]) - lo, d), torch.bfloat16, gen)
        table = None
        if paged:
            table, nb = W.make_block_table(before + n, bs, perm_seed=1630, extra_blocks=2)
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
    ro, rl = oracle.decode_window(q, k_host, v_host, before, d ** -0.5, window, ring=ring,
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
    e = check_parity(out, lse, ro, rl, vmax, f"window d={d} {layout}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


def test_head_dims_route_to_the_multi_row_kernel():
    """bf16 caches with d = 64, 80, 96 and 256 launch the multi-row kernel (a
    work-group of four or eight wavefronts), not the generic one (one
    wavefront per query row of a KV head; four rows here, eight below)."""
    for d in (64, 80, 96, 256):
        for h, g, n in [(8, 8, 1), (32, 8, 1), (64, 8, 64)]:
            waves = kvc.launch_shape(B=4, h=h * n, g=g, d=d, max_seq_len=2048)[0]
            assert waves in (4, 8), (d, h, n, waves)
    # fp32 stays on the generic kernel: one work-group per KV head with one
    # wavefront per query row of its group (h / g = 4 here)
    assert kvc.launch_shape(B=4, h=8, g=2, d=64, max_seq_len=2048, dtype=torch.float32)[0] == 4
    assert kvc.launch_shape(B=4, h=16, g=2, d=112, max_seq_len=2048, dtype="fp8")[0] == 8


# Head dims outside 64, 80, 96, 128 and 256, and fp32 caches, run on the
# generic kernel: four dims per lane and 64 / LP positions per wavefront pass
# when d is a multiple of 4 (d = 20: LP = 8 with three idle lanes per group;
# 100 and 112: LP = 32; 200: LP = 64), one dim per lane otherwise (d = 6).
# bf16 caches with d = 96 take the multi-row kernel here, fp32 ones the
# generic kernel.
GENERIC_DIMS = [6, 20, 96, 100, 112, 200]


def _host_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.int32) if a.dtype == np.float32 else a


def _device_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("d", GENERIC_DIMS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_append_decode_generic_head_dims(d, dtype, paged, num_splits):
    """Two new tokens per sequence, three query heads per KV head, appended
    in the same call over ragged lengths with NaN in every unwritten slot:
    the cache bytes and every output row against the oracle."""
    h, g, n, bs = 12, 4, 2, 16
    _log(f"case generic_headdim d={d} {dtype} paged={paged} splits={num_splits}")
    seed = 1700 + d
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lens = torch.tensor(BEFORE, dtype=torch.int32)
    B = len(BEFORE)
    w = W.Workload("gen", B=B, h=h, g=g, d=d, dtype=dtype, seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    q = W.randn((B, h, n, d), tdt, gen)
    k_new = W.randn((B, g, n, d), tdt, gen)
    v_new = W.randn((B, g, n, d), tdt, gen)
    x = W.make_contiguous(w, lengths=lens, t_cap=max(BEFORE) + n + 3, fill=float("nan"))
    if paged:
        table, nb = W.make_block_table(lens + n, bs, perm_seed=seed + 2, extra_blocks=2)
        kc = W.scatter_to_pool(x["k_cache"], lens, table, nb, bs, fill=float("nan"))
        vc = W.scatter_to_pool(x["v_cache"], lens, table, nb, bs, fill=float("nan"))
    else:
        table, kc, vc = None, x["k_cache"], x["v_cache"]
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(lens),
                                       block_table=dev(table) if paged else None, scale=w.scale,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, lens, block_table=table)
    assert np.array_equal(_device_bits(kd), _host_bits(ek)), "K cache"
    assert np.array_equal(_device_bits(vd), _host_bits(ev)), "V cache"
    if dtype == "bf16":
        k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    else:
        k_host, v_host = torch.from_numpy(ek.copy()), torch.from_numpy(ev.copy())
    ro, rl = oracle.decode_multi(q, k_host, v_host, lens, w.scale, block_table=table,
                                 block_size=bs)
    after = lens + n
    vmax = attended_vmax_paged(v_host, table, after, bs) if paged else \
        attended_vmax_contig(v_host, after)
    e = check_parity(out, lse, ro, rl, vmax, f"generic d={d} {dtype}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


def test_paged_multi_row_plans_take_short_chunks():
    """Over a paged bf16 pool (ragged lengths) the multi-row kernel's row
    groups that fill the device take chunks of at most 2816 positions
    instead of whole units; FP8 pools and contiguous caches keep whole
    units there.  (Launch shapes depend on the device's resident slots:
    these hold on a 256-CU MI355X, where the 128-row work-group keeps two
    per CU.)"""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"slot counts assume 256 compute units (this device has {cus})")
    L = 8208  # a 513-entry table of 16-position blocks
    for d, h in ((96, 32), (128, 32 * 32)):
        waves, wgs, cl, nc = kvc.launch_shape(64, h, 8, d, L, 0, paged=True)
        assert (nc, cl) == (3, 2752), (d, h, waves, wgs, cl, nc)
        waves, wgs, cl, nc = kvc.launch_shape(64, h, 8, d, L, 0, paged=False)
        assert nc == 1, (d, h, nc)
    waves, wgs, cl, nc = kvc.launch_shape(64, 32 * 32, 8, 128, L, 0, dtype="fp8", paged=True)
    assert nc == 1, nc
    # the FP8 decode kernel with two new tokens per sequence over the same
    # pool: chunks (not the stream grid), 3 of 2752 positions; the bf16 one
    # streams (chunk fields 0)
    assert kvc.launch_shape_multi(64, 32, 8, 128, 2, L, dtype="fp8", paged=True)[2:] == (2752, 3)
    assert kvc.launch_shape_multi(64, 32, 8, 128, 2, L, paged=True)[2:] == (0, 0)
