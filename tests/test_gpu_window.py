"""GPU parity of sliding-window decode (kvc_*_window): the token at position x
sees positions max(0, x + 1 - W) .. x.  Linear caches hold NaN outside every
window (and paged tables hold -1 for blocks wholly before it), so a read
outside the window shows up as NaN; ring caches (position p in slot p mod
t_cap) wrap many times.  Checked against the oracle's windowed reference."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import check_parity, dev

pytestmark = pytest.mark.gpu

SHAPES = [
    ("valu_m1", dict(h=4, g=4, d=128, dtype="bf16"), 1),
    ("valu_rows2", dict(h=8, g=4, d=128, dtype="bf16"), 1),
    ("mfma_m8", dict(h=16, g=2, d=128, dtype="bf16"), 1),
    ("mfma_rows32", dict(h=16, g=2, d=128, dtype="bf16"), 4),
    ("mfma_slices_64", dict(h=16, g=2, d=128, dtype="bf16"), 8),
    ("generic_f32_d16", dict(h=4, g=2, d=16, dtype="f32"), 2),
    # more than 32 new tokens per KV head: the new positions span two tiles
    ("mfma_mha_n33", dict(h=2, g=2, d=128, dtype="bf16"), 33),
    ("mfma_mha_n64", dict(h=1, g=1, d=128, dtype="bf16"), 64),
]
BEFORE = [0, 1, 5, 31, 32, 33, 100, 1000, 4095, 5000]


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.view(torch.int32).numpy().view(np.uint32)


def _to_torch(a: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    if like.dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def _vmax(v_host, before, n, window, ring, table=None, bs=16):
    """max |V| over every position some token sees."""
    m = 0.0
    for b in range(len(before)):
        hi = int(before[b]) + n
        lo = max(0, int(before[b]) + 1 - window)
        for p in range(lo, hi):
            if table is not None:
                row = v_host[int(table[b, p // bs]), :, p % bs]
            else:
                row = v_host[b, :, p % v_host.shape[2] if ring else p]
            m = max(m, float(row.float().abs().max()))
    return m


def _case(name, s, n, window, ring, paged, seed, bs=16):
    before = torch.tensor(BEFORE, dtype=torch.int32)
    B = len(BEFORE)
    w = W.Workload(name, B=B, seed=seed, **s)
    gen = torch.Generator().manual_seed(seed)
    dt = w.torch_dtype
    q = W.randn((B, w.h, n, w.d), dt, gen)
    k_new = W.randn((B, w.g, n, w.d), dt, gen)
    v_new = W.randn((B, w.g, n, w.d), dt, gen)
    nan = float("nan")
    table = None
    if ring:
        t_cap = window + n - 1 + 3
        k = W.randn((B, w.g, t_cap, w.d), dt, gen)
        v = W.randn((B, w.g, t_cap, w.d), dt, gen)
        for b in range(B):      # slots no position has reached yet stay unwritten
            if BEFORE[b] < t_cap:
                k[b, :, BEFORE[b]:] = nan
                v[b, :, BEFORE[b]:] = nan
    else:
        t_cap = max(BEFORE) + n + 5
        k = torch.full((B, w.g, t_cap, w.d), nan, dtype=dt)
        v = torch.full((B, w.g, t_cap, w.d), nan, dtype=dt)
        for b in range(B):      # only positions some token of b sees are written
            lo = max(0, BEFORE[b] + 1 - window)
            k[b, :, lo:BEFORE[b]] = W.randn((w.g, BEFORE[b] - lo, w.d), dt, gen)
            v[b, :, lo:BEFORE[b]] = W.randn((w.g, BEFORE[b] - lo, w.d), dt, gen)
        if paged:
            table, nb = W.make_block_table(before + n, bs, perm_seed=seed + 1, extra_blocks=2)
            kp = W.scatter_to_pool(k, before, table, nb, bs, fill=nan)
            vp = W.scatter_to_pool(v, before, table, nb, bs, fill=nan)
            for b in range(B):  # blocks wholly before every window are unmapped
                lo = max(0, BEFORE[b] + 1 - window)
                table[b, : lo // bs] = -1
            k, v = kp, vp
    return w, before, q, k_new, v_new, k, v, table, t_cap


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("window", [1, 37, 4096])
@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
@pytest.mark.parametrize("num_splits", [0, 3, -1])
def test_append_decode_window(shape, window, layout, num_splits):
    name, s, n = shape
    ring, paged = layout == "ring", layout == "paged"
    _log(f"case window {name} n={n} W={window} {layout} splits={num_splits}")
    w, before, q, k_new, v_new, k, v, table, t_cap = _case(name, s, n, window, ring, paged, 1000)
    kd, vd = dev(k), dev(v)
    out, lse = kvc.decode_window(dev(q), kd, vd, dev(before), window, ring=ring,
                                 block_table=dev(table) if paged else None, scale=w.scale,
                                 num_splits=num_splits, k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    ek, ev = oracle.append_window(k_new, v_new, k, v, before, ring=ring,
                                  block_table=table if paged else None)
    assert np.array_equal(_raw(kd), ek.view(_raw(kd).dtype)), f"{name}: cache after the step"
    assert np.array_equal(_raw(vd), ev.view(_raw(vd).dtype)), f"{name}: cache after the step"
    k_host, v_host = _to_torch(ek, k), _to_torch(ev, v)
    ro, rl = oracle.decode_window(q, k_host, v_host, before, w.scale, window, ring=ring,
                                  block_table=table if paged else None)
    vmax = _vmax(v_host, before, n, window, ring, table if paged else None)
    e = check_parity(out, lse, ro, rl, vmax, name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2], SHAPES[3]], ids=["valu_m1", "mfma_m8",
                                                                          "mfma_rows32"])
@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
def test_decode_window_over_filled_cache(shape, layout):
    """The tokens are already in the cache; seq_lens counts them."""
    name, s, n = shape
    ring, paged = layout == "ring", layout == "paged"
    window = 37
    _log(f"case window_filled {name} {layout}")
    w, before, q, k_new, v_new, k, v, table, t_cap = _case(name, s, n, window, ring, paged, 1010)
    ek, ev = oracle.append_window(k_new, v_new, k, v, before, ring=ring,
                                  block_table=table if paged else None)
    k_host, v_host = _to_torch(ek, k), _to_torch(ev, v)
    out, lse = kvc.decode_window(dev(q), dev(k_host), dev(v_host), dev(before + n), window,
                                 ring=ring, block_table=dev(table) if paged else None,
                                 scale=w.scale, num_splits=2)
    ro, rl = oracle.decode_window(q, k_host, v_host, before, w.scale, window, ring=ring,
                                  block_table=table if paged else None)
    check_parity(out, lse, ro, rl, _vmax(v_host, before, n, window, ring,
                                         table if paged else None), name)


def test_ring_incremental_many_wraps():
    """60 one-call steps of 3 tokens into a ring of 12 slots with a window of
    10: the ring wraps 15 times; every step matches the oracle."""
    _log("case ring_incremental")
    B, h, g, d, n, window = 3, 16, 2, 128, 3, 10
    t_cap = window + n - 1
    gen = torch.Generator().manual_seed(1020)
    k_host = torch.full((B, g, t_cap, d), float("nan"), dtype=torch.bfloat16)
    v_host = k_host.clone()
    kd, vd = dev(k_host), dev(v_host)
    lengths = torch.tensor([0, 4, 11], dtype=torch.int32)
    for step in range(60):
        q = W.randn((B, h, n, d), torch.bfloat16, gen)
        kn = W.randn((B, g, n, d), torch.bfloat16, gen)
        vn = W.randn((B, g, n, d), torch.bfloat16, gen)
        if step == 0:  # the prefix of sequences 1 and 2 is already there
            for b in (1, 2):
                for p in range(int(lengths[b])):
                    k_host[b, :, p % t_cap] = W.randn((g, d), torch.bfloat16, gen)
                    v_host[b, :, p % t_cap] = W.randn((g, d), torch.bfloat16, gen)
            kd.copy_(k_host.cuda())
            vd.copy_(v_host.cuda())
        out, lse = kvc.decode_window(dev(q), kd, vd, dev(lengths), window, ring=True,
                                     k_new=dev(kn), v_new=dev(vn))
        ek, ev = oracle.append_window(kn, vn, k_host, v_host, lengths, ring=True)
        k_host, v_host = _to_torch(ek, k_host), _to_torch(ev, v_host)
        assert torch.equal(kd.cpu().view(torch.int16), k_host.view(torch.int16)), f"step {step}"
        ro, rl = oracle.decode_window(q, k_host, v_host, lengths, 1.0 / math.sqrt(d), window,
                                      ring=True)
        vmax = _vmax(v_host, lengths, n, window, True)
        check_parity(out, lse, ro, rl, vmax, f"ring step {step}")
        lengths = lengths + n


@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
def test_window_full_size(layout):
    """A window of 1024 at the 70B GQA shape (linear cache, or a ring of
    1039 slots) and on the paged GQA workload, one token per sequence, in
    the launch configuration the benchmark times."""
    window = 1024
    ring, paged = layout == "ring", layout == "paged"
    _log(f"case window_full {layout}")
    if paged:
        w = W.WORKLOADS["paged_gqa_bf16"]
        x = W.make_paged(w)
        k, v, table = x["k_pool"], x["v_pool"], x["block_table"]
    else:
        w = W.WORKLOADS["gqa_70b_bf16"]
        x = W.make_contiguous(w, t_cap=window + 15 if ring else None)
        k, v, table = x["k_cache"], x["v_cache"], None
    before = x["seq_lens_before"]
    q = x["q"].view(w.B, w.h, 1, w.d)
    kn, vn = x["k_new"].view(w.B, w.g, 1, w.d), x["v_new"].view(w.B, w.g, 1, w.d)
    kd, vd = dev(k), dev(v)
    out, lse = kvc.decode_window(dev(q), kd, vd, dev(before), window, ring=ring,
                                 block_table=dev(table) if paged else None, scale=x["scale"],
                                 num_splits=w.num_splits, k_new=dev(kn), v_new=dev(vn))
    torch.cuda.synchronize()
    ek, ev = oracle.append_window(kn, vn, k, v, before, ring=ring, block_table=table)
    assert np.array_equal(_raw(kd), ek.view(_raw(kd).dtype)), f"{layout}: cache after the step"
    assert np.array_equal(_raw(vd), ev.view(_raw(vd).dtype)), f"{layout}: cache after the step"
    k_host, v_host = _to_torch(ek, k), _to_torch(ev, v)
    ro, rl = oracle.decode_window(q, k_host, v_host, before, x["scale"], window, ring=ring,
                                  block_table=table)
    vmax = 0.0
    for b in range(w.B):  # max |V| over the window of the new token
        hi = int(before[b]) + 1
        pos = torch.arange(max(0, hi - window), hi)
        if paged:
            rows = v_host[table[b, pos // 16].long(), :, pos % 16]
        else:
            rows = v_host[b][:, pos % v_host.shape[2] if ring else pos]
        vmax = max(vmax, float(rows.float().abs().max()))
    e = check_parity(out, lse, ro, rl, vmax, f"window full {layout}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")
