"""GPU parity: libkvc (through the C ABI, via the ctypes binding) against the
CPU fp64 oracle on identical seeded inputs.

Bar: append and block-table gathers are bit-exact (whole-cache byte
compare); attention outputs satisfy max|out - oracle| <= 2e-3 * max|V| over
the attended V entries and |lse - oracle| <= 1e-4.  Random N(0,1) data alone
is a weak check (near-flat softmax), so structured inputs are added: needles
at boundary positions, scale 0, edge lengths, NaN-poisoned unwritten slots.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import (attended_vmax_contig, attended_vmax_paged, check_parity, dev,
                      needle_positions, plant_needles_contig)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _u16(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def _raw_np(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


# ----------------------------------------------------------------------------
def test_d1_worked_example():
    """zwjcode.cn 'KV Cache 的增量解码' section 04: K=[1,2]+[0], V=[10,20]+[30],
    q=1, scale 1 -> o ~ 18.45 (exactly 18.453021...)."""
    _log("case d1_worked_example")
    k = torch.zeros(1, 1, 4, 1)
    v = torch.zeros(1, 1, 4, 1)
    k[0, 0, :2, 0] = torch.tensor([1.0, 2.0])
    v[0, 0, :2, 0] = torch.tensor([10.0, 20.0])
    kd, vd = dev(k), dev(v)
    kvc.append(dev(torch.zeros(1, 1, 1)), dev(torch.full((1, 1, 1), 30.0)), kd, vd,
               dev(torch.tensor([2], dtype=torch.int32)))
    assert kd.cpu()[0, 0, :3, 0].tolist() == [1.0, 2.0, 0.0]
    assert vd.cpu()[0, 0, :3, 0].tolist() == [10.0, 20.0, 30.0]
    q = torch.ones(1, 1, 1)
    out, lse = kvc.decode(dev(q), kd, vd, dev(torch.tensor([3], dtype=torch.int32)), scale=1.0)
    ro, rl = oracle.decode(q, kd.cpu(), vd.cpu(), [3], 1.0)
    check_parity(out, lse, ro, rl, 30.0, "d1")
    assert abs(float(out[0, 0, 0]) - 18.45) <= 0.005


# ----------------------------------------------------------------------------
def _run_contig(w: W.Workload, x: dict, num_splits: int, what: str):
    """GPU append + decode on a contiguous workload; returns errors."""
    q, kc, vc = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"])
    sl_before, sl_after = dev(x["seq_lens_before"]), dev(x["seq_lens_after"])
    kvc.append(dev(x["k_new"]), dev(x["v_new"]), kc, vc, sl_before)
    ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["seq_lens_before"])
    assert np.array_equal(_u16(kc), _raw_np(ek)), f"{what}: K cache after append differs"
    assert np.array_equal(_u16(vc), _raw_np(ev)), f"{what}: V cache after append differs"
    out, lse = kvc.decode(q, kc, vc, sl_after, scale=x["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    k_host, v_host = kc.cpu(), vc.cpu()
    ro, rl = oracle.decode(x["q"], k_host, v_host, x["seq_lens_after"], x["scale"])
    vmax = attended_vmax_contig(v_host, x["seq_lens_after"])
    return check_parity(out, lse, ro, rl, vmax, what)


def _run_paged(w: W.Workload, x: dict, num_splits: int, what: str):
    q, kp, vp = dev(x["q"]), dev(x["k_pool"]), dev(x["v_pool"])
    bt = dev(x["block_table"])
    sl_before, sl_after = dev(x["seq_lens_before"]), dev(x["seq_lens_after"])
    kvc.append(dev(x["k_new"]), dev(x["v_new"]), kp, vp, sl_before, block_table=bt)
    ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_pool"], x["v_pool"], x["seq_lens_before"],
                           block_table=x["block_table"])
    assert np.array_equal(_u16(kp), _raw_np(ek)), f"{what}: K pool after append differs"
    assert np.array_equal(_u16(vp), _raw_np(ev)), f"{what}: V pool after append differs"
    out, lse = kvc.decode_paged(q, kp, vp, bt, sl_after, scale=x["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    k_host, v_host = kp.cpu(), vp.cpu()
    ro, rl = oracle.decode(x["q"], k_host, v_host, x["seq_lens_after"], x["scale"],
                           block_table=x["block_table"], block_size=x["block_size"])
    vmax = attended_vmax_paged(v_host, x["block_table"], x["seq_lens_after"], x["block_size"])
    return check_parity(out, lse, ro, rl, vmax, what)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name):
    """Every workload at its full size, in the launch configuration the
    benchmark times (num_splits as the workload states, else automatic)."""
    w = W.WORKLOADS[name]
    _log(f"case full_size {name}")
    if w.paged:
        x = W.make_paged(w)
        e = _run_paged(w, x, w.num_splits, name)
    else:
        x = W.make_contiguous(w)
        e = _run_contig(w, x, w.num_splits, name)
    _log(f"  {name}: out err/vmax {e[0]:.2e}, lse err {e[1]:.2e}")


@pytest.mark.parametrize("name", ["mha_7b_bf16", "gqa_70b_bf16", "paged_gqa_bf16", "long_mqa_bf16"])
def test_workload_needles(name):
    """One dominant key per (sequence, KV head) at first/last/tile/page/chunk
    boundary positions: a skipped or shifted position moves out by ~|V|."""
    w = W.WORKLOADS[name]
    _log(f"case needles {name}")
    B = min(w.B, 8)
    w = W.Workload(w.name, B=B, h=w.h, g=w.g, d=w.d, dtype=w.dtype, T=w.T, T_range=w.T_range,
                   paged=w.paged, num_splits=w.num_splits, seed=w.seed + 500)
    lengths = W.seq_lengths(w)
    x = W.make_contiguous(w, lengths=lengths)
    Lafter = x["seq_lens_after"]
    max_len = int(x["t_cap"]) if not w.paged else int(W.block_counts(Lafter, 16).max()) * 16
    _, cl, _ = kvc.plan(w.B, w.h, w.g, w.d, max_len, w.num_splits)
    cl = cl or 2049  # stream mode cuts anywhere: probe odd offsets too
    special = [0, -1, -2, 15, 16, 31, 32, 33, 127, 128, cl - 1, cl, 2 * cl - 1, 2 * cl, 3 * cl + 16]
    pos = needle_positions(lengths, w.g, special, seed=w.seed)
    plant_needles_contig(x, pos)
    if not w.paged:
        _run_contig(w, x, w.num_splits, name + "/needles")
    else:
        table, nb = W.make_block_table(Lafter, 16, perm_seed=w.seed + 1)
        xp = dict(x)
        xp["k_pool"] = W.scatter_to_pool(x["k_cache"], lengths, table, nb, 16)
        xp["v_pool"] = W.scatter_to_pool(x["v_cache"], lengths, table, nb, 16)
        xp["block_table"] = table
        xp["block_size"] = 16
        _run_paged(w, xp, w.num_splits, name + "/needles")


# ----------------------------------------------------------------------------
# Kernel coverage: VALU (m <= 3), MFMA (4 <= m <= 32), generic (fp32, other d).
KERNEL_SHAPES = [
    ("valu_m1", dict(h=4, g=4, d=128, dtype="bf16")),
    ("valu_m2", dict(h=8, g=4, d=128, dtype="bf16")),
    ("valu_m3", dict(h=6, g=2, d=128, dtype="bf16")),
    ("mfma_m4", dict(h=8, g=2, d=128, dtype="bf16")),
    ("mfma_m8", dict(h=16, g=2, d=128, dtype="bf16")),
    ("mfma_m16", dict(h=16, g=1, d=128, dtype="bf16")),
    ("mfma_m12", dict(h=24, g=2, d=128, dtype="bf16")),
    ("mfma_m32", dict(h=32, g=1, d=128, dtype="bf16")),
    ("generic_m64", dict(h=64, g=1, d=128, dtype="bf16")),
    ("generic_f32_d16", dict(h=4, g=2, d=16, dtype="f32")),
    ("generic_bf16_d64", dict(h=8, g=2, d=64, dtype="bf16")),
    ("generic_f32_d128", dict(h=8, g=2, d=128, dtype="f32")),
]
EDGE_LENGTHS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000]


@pytest.mark.parametrize("shape", KERNEL_SHAPES, ids=[s[0] for s in KERNEL_SHAPES])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_edge_lengths_contiguous(shape, num_splits):
    """Edge lengths (including 0) with NaN in every unwritten slot: the
    kernels must never let a position >= length reach the result."""
    name, s = shape
    _log(f"case edge_contig {name} splits={num_splits}")
    w = W.Workload(name, B=len(EDGE_LENGTHS), seed=300, **s)
    lengths = torch.tensor(EDGE_LENGTHS, dtype=torch.int32)
    x = W.make_contiguous(w, lengths=lengths, fill=float("nan"))
    q, kc, vc = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.decode(q, kc, vc, dev(lengths), scale=x["scale"], num_splits=num_splits)
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], lengths, x["scale"])
    check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], lengths), name)
    o = out.cpu()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse.cpu()[0]))


@pytest.mark.parametrize("shape", KERNEL_SHAPES, ids=[s[0] for s in KERNEL_SHAPES])
@pytest.mark.parametrize("block_size", [16, 8, 32])
def test_edge_lengths_paged(shape, block_size):
    name, s = shape
    _log(f"case edge_paged {name} bs={block_size}")
    w = W.Workload(name, B=len(EDGE_LENGTHS), seed=301, block_size=block_size, paged=True, **s)
    lengths = torch.tensor(EDGE_LENGTHS, dtype=torch.int32)
    x = W.make_paged(w, lengths=lengths, fill=float("nan"))
    out, lse = kvc.decode_paged(dev(x["q"]), dev(x["k_pool"]), dev(x["v_pool"]),
                                dev(x["block_table"]), dev(lengths), scale=x["scale"], num_splits=2)
    ro, rl = oracle.decode(x["q"], x["k_pool"], x["v_pool"], lengths, x["scale"],
                           block_table=x["block_table"], block_size=block_size)
    vmax = attended_vmax_paged(x["v_pool"], x["block_table"], lengths, block_size)
    check_parity(out, lse, ro, rl, vmax, name)


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[0], KERNEL_SHAPES[4], KERNEL_SHAPES[7]],
                         ids=["valu_m1", "mfma_m8", "mfma_m32"])
def test_split_counts_agree(shape):
    name, s = shape
    w = W.Workload(name, B=2, T=1500, seed=302, **s)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    q, kc, vc, sl = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L)
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    vmax = attended_vmax_contig(x["v_cache"], L)
    for ns in [1, 2, 3, 5, 7, 16, 31, 47, 64]:
        _log(f"case splits {name} {ns}")
        out, lse = kvc.decode(q, kc, vc, sl, scale=x["scale"], num_splits=ns)
        check_parity(out, lse, ro, rl, vmax, f"{name}/splits={ns}")


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[1], KERNEL_SHAPES[4]], ids=["valu_m2", "mfma_m8"])
def test_scale_zero_and_equal_rows(shape):
    """scale 0 gives the mean of the attended V rows and lse = ln L."""
    name, s = shape
    _log(f"case scale0 {name}")
    w = W.Workload(name, B=4, T_range=(1, 3000), seed=303, **s)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L), scale=0.0)
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, 0.0)
    check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], L), name + "/scale0")
    assert np.max(np.abs(lse.cpu().double().numpy() - np.log(L.double().numpy())[:, None])) < 1e-4


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[0], KERNEL_SHAPES[4], KERNEL_SHAPES[9]],
                         ids=["valu_m1", "mfma_m8", "generic_f32_d16"])
def test_paged_equals_contiguous_on_gpu(shape):
    """Same logical cache, two layouts, one chunk each: identical tiling, so
    the GPU results are bit-identical."""
    name, s = shape
    _log(f"case paged_vs_contig {name}")
    w = W.Workload(name, B=5, T_range=(1, 700), seed=304, **s)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    table, nb = W.make_block_table(L, 16, perm_seed=305, extra_blocks=7)
    kp = W.scatter_to_pool(x["k_cache"], L, table, nb, 16)
    vp = W.scatter_to_pool(x["v_cache"], L, table, nb, 16)
    o1, l1 = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L), num_splits=1)
    o2, l2 = kvc.decode_paged(dev(x["q"]), dev(kp), dev(vp), dev(table), dev(L), num_splits=1)
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[0], KERNEL_SHAPES[4]], ids=["valu_m1", "mfma_m8"])
@pytest.mark.parametrize("paged", [False, True])
def test_incremental_decode_40_steps(shape, paged):
    """zwjcode.cn 'KV Cache 的增量解码' section 07 and 12: append + decode for
    40 steps; every step matches the oracle on the same cache, and the cache
    grows by exactly one slot per step."""
    name, s = shape
    _log(f"case incremental {name} paged={paged}")
    steps, prefix, B = 40, 100, 3
    w = W.Workload(name, B=B, T=prefix, seed=306, **s)
    x = W.make_contiguous(w, t_cap=prefix + steps + 8)
    gen = torch.Generator().manual_seed(307)
    knew = W.randn((steps, B, w.g, w.d), w.torch_dtype, gen)
    vnew = W.randn((steps, B, w.g, w.d), w.torch_dtype, gen)
    qs = W.randn((steps, B, w.h, w.d), w.torch_dtype, gen)
    k_host, v_host = x["k_cache"].clone(), x["v_cache"].clone()
    lengths = torch.full((B,), prefix, dtype=torch.int32)
    if paged:
        table, nb = W.make_block_table(torch.full((B,), prefix + steps, dtype=torch.int32), 16,
                                       perm_seed=308)
        k_host = W.scatter_to_pool(x["k_cache"], lengths, table, nb, 16)
        v_host = W.scatter_to_pool(x["v_cache"], lengths, table, nb, 16)
        bt = dev(table)
    kd, vd = dev(k_host), dev(v_host)
    for t in range(steps):
        before = lengths.clone()
        after = before + 1
        kvc.append(dev(knew[t]), dev(vnew[t]), kd, vd, dev(before),
                   block_table=bt if paged else None)
        if paged:
            out, lse = kvc.decode_paged(dev(qs[t]), kd, vd, bt, dev(after))
            ek, ev = oracle.append(knew[t], vnew[t], k_host, v_host, before, block_table=table)
        else:
            out, lse = kvc.decode(dev(qs[t]), kd, vd, dev(after))
            ek, ev = oracle.append(knew[t], vnew[t], k_host, v_host, before)
        k_host = torch.from_numpy(ek.view(np.int16).copy()).view(w.torch_dtype) \
            if w.dtype == "bf16" else torch.from_numpy(ek.copy())
        v_host = torch.from_numpy(ev.view(np.int16).copy()).view(w.torch_dtype) \
            if w.dtype == "bf16" else torch.from_numpy(ev.copy())
        assert torch.equal(kd.cpu(), k_host) and torch.equal(vd.cpu(), v_host), f"step {t}"
        if paged:
            ro, rl = oracle.decode(qs[t], k_host, v_host, after, w.scale, block_table=table)
            vmax = attended_vmax_paged(v_host, table, after, 16)
        else:
            ro, rl = oracle.decode(qs[t], k_host, v_host, after, w.scale)
            vmax = attended_vmax_contig(v_host, after)
        check_parity(out, lse, ro, rl, vmax, f"{name}/step{t}")
        lengths = after


def test_device_values_are_clamped_not_faulting():
    """A length above the capacity is clamped to it; an append slot outside
    the capacity is skipped."""
    _log("case clamp")
    w = W.Workload("c", B=2, h=8, g=2, d=128, dtype="bf16", T=40, seed=309)
    x = W.make_contiguous(w, t_cap=48)
    kc, vc = dev(x["k_cache"]), dev(x["v_cache"])
    out1, lse1 = kvc.decode(dev(x["q"]), kc, vc, dev(torch.tensor([48, 48], dtype=torch.int32)),
                            num_splits=1)
    out2, lse2 = kvc.decode(dev(x["q"]), kc, vc, dev(torch.tensor([1000, 48], dtype=torch.int32)),
                            num_splits=1)
    assert torch.equal(out1.cpu(), out2.cpu()) and torch.equal(lse1.cpu(), lse2.cpu())
    before = kc.cpu().clone()
    kvc.append(dev(x["k_new"]), dev(x["v_new"]), kc, vc,
               dev(torch.tensor([48, -1], dtype=torch.int32)))
    assert torch.equal(kc.cpu(), before)


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[0], KERNEL_SHAPES[4], KERNEL_SHAPES[7],
                                   KERNEL_SHAPES[8]],
                         ids=["valu_m1", "mfma_m8", "mfma_m32", "generic_m64"])
@pytest.mark.parametrize("num_splits", [0, 3, -1])
@pytest.mark.parametrize("paged", [False, True])
def test_position_ramp(shape, num_splits, paged):
    """V[p] = p mod 64 in every dim (exact in bf16).  With scale 0 every
    attended position has the same weight, so out equals the mean of
    (p mod 64) over exactly the attended positions (a dropped, repeated or
    shifted position moves it) and lse = ln L; with the usual scale the
    result matches the oracle."""
    name, s = shape
    _log(f"case ramp {name} splits={num_splits} paged={paged}")
    lengths = torch.tensor([1, 17, 33, 64, 255, 1000, 4097, 0], dtype=torch.int32)
    B = len(lengths)
    w = W.Workload(name, B=B, seed=330, **s)
    x = W.make_contiguous(w, lengths=lengths, fill=float("nan"))
    T = x["v_cache"].shape[2]
    ramp = (torch.arange(T) % 64).to(torch.float32)
    vr = ramp.view(1, 1, T, 1).expand(B, w.g, T, w.d).to(x["v_cache"].dtype).clone()
    vr[torch.arange(T).view(1, 1, T, 1).expand(B, w.g, T, w.d) >= lengths.view(-1, 1, 1, 1)] = \
        float("nan")
    x["v_cache"] = vr
    if paged:
        table, nb = W.make_block_table(lengths, 16, perm_seed=331, extra_blocks=3)
        kp = W.scatter_to_pool(x["k_cache"], lengths, table, nb, 16, fill=float("nan"))
        vp = W.scatter_to_pool(x["v_cache"], lengths, table, nb, 16, fill=float("nan"))
        call = lambda sc: kvc.decode_paged(dev(x["q"]), dev(kp), dev(vp), dev(table),  # noqa: E731
                                           dev(lengths), scale=sc, num_splits=num_splits)
    else:
        call = lambda sc: kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]),  # noqa: E731
                                     dev(lengths), scale=sc, num_splits=num_splits)
    out, lse = call(0.0)
    for b in range(B):
        L = int(lengths[b])
        o, l = out[b].cpu().double(), lse[b].cpu().double()
        if L == 0:
            assert torch.all(o == 0) and torch.all(torch.isinf(l) & (l < 0)), name
            continue
        # every weight is exactly 1 and the sums are integers below 2^24: the
        # mean is exact up to float32 rounding, so one dropped position (which
        # moves it by |ramp[p] - mean| / L) shows
        mean = float(ramp[:L].double().mean())
        assert float((o - mean).abs().max()) <= 1e-4, (name, b, L, float((o - mean).abs().max()))
        assert float((l - np.log(L)).abs().max()) <= 1e-4, (name, b, L)
    out, lse = call(x["scale"])
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], lengths, x["scale"])
    check_parity(out, lse, ro, rl, 63.0, name + "/ramp")


@pytest.mark.parametrize("shape", [KERNEL_SHAPES[0], KERNEL_SHAPES[4], KERNEL_SHAPES[7],
                                   KERNEL_SHAPES[8]],
                         ids=["valu_m1", "mfma_m8", "mfma_m32", "mfma_m64"])
@pytest.mark.parametrize("num_splits", [0, -1])
@pytest.mark.parametrize("paged", [False, True])
def test_score_staircase(shape, num_splits, paged):
    """Scores that climb in steps along the sequence: K[p] = 0.5 *
    min(floor(p / 37), 16) in every dim and q row i = 1 + (i mod 8)/8, so
    each of the 16 steps raises row i's score by 8.2 (1 + (i mod 8)/8) in
    log2 units, at positions that do not line up with the tiles, by a
    different amount per query row.  The running maximum of every row moves
    again and again mid-sequence; the softmax weight of the positions before
    a step drops by 2^-8 or more.  (The cap keeps lse below about 170, where
    float32 still resolves the 1e-4 bar.)  Checked against the oracle."""
    name, s = shape
    _log(f"case staircase {name} splits={num_splits} paged={paged}")
    lengths = torch.tensor([1, 37, 38, 100, 1000, 4097], dtype=torch.int32)
    B = len(lengths)
    w = W.Workload(name, B=B, seed=340, **s)
    x = W.make_contiguous(w, lengths=lengths, fill=float("nan"))
    T = x["k_cache"].shape[2]
    level = 0.5 * torch.clamp(torch.div(torch.arange(T), 37, rounding_mode="floor"), max=16).to(torch.float32)
    kr = level.view(1, 1, T, 1).expand(B, w.g, T, w.d).to(x["k_cache"].dtype).clone()
    kr[torch.arange(T).view(1, 1, T, 1).expand(B, w.g, T, w.d) >= lengths.view(-1, 1, 1, 1)] = \
        float("nan")
    x["k_cache"] = kr
    qrow = 1.0 + (torch.arange(w.h) % 8).to(torch.float32) / 8.0  # exact in bf16
    x["q"] = qrow.view(1, w.h, 1).expand(B, w.h, w.d).to(x["q"].dtype).clone()
    if paged:
        table, nb = W.make_block_table(lengths, 16, perm_seed=341, extra_blocks=3)
        kp = W.scatter_to_pool(x["k_cache"], lengths, table, nb, 16, fill=float("nan"))
        vp = W.scatter_to_pool(x["v_cache"], lengths, table, nb, 16, fill=float("nan"))
        out, lse = kvc.decode_paged(dev(x["q"]), dev(kp), dev(vp), dev(table), dev(lengths),
                                    scale=x["scale"], num_splits=num_splits)
        vmax = attended_vmax_paged(vp, table, lengths, 16)
    else:
        out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(lengths),
                              scale=x["scale"], num_splits=num_splits)
        vmax = attended_vmax_contig(x["v_cache"], lengths)
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], lengths, x["scale"])
    check_parity(out, lse, ro, rl, vmax, name + "/staircase")
