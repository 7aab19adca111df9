"""GPU parity of FP8 E4M3 caches (kvc_*_fp8): the quantising append is
bit-exact against the oracle's encoder (nearest code, ties to even,
saturation, signed zero, NaN), and attention over the codes matches the
oracle's dequantise-then-exact reference for every kernel family, layout and
split mode.  Unwritten slots hold the NaN code."""
from __future__ import annotations

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
    ("valu_m1", dict(h=4, g=4, d=128)),
    ("valu_m2", dict(h=8, g=4, d=128)),
    ("valu_m3", dict(h=6, g=2, d=128)),
    ("mfma_m4", dict(h=8, g=2, d=128)),
    ("mfma_m8", dict(h=16, g=2, d=128)),
    ("mfma_m16", dict(h=16, g=1, d=128)),
    ("mfma_m32", dict(h=32, g=1, d=128)),
    ("generic_d64", dict(h=8, g=2, d=64)),
    ("generic_m64", dict(h=64, g=1, d=128)),
]
EDGE = [0, 1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 1000, 4095, 4097]
NAN_CODE = 0x7F


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _scales(g, gen):
    ks = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    vs = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    return ks, vs


def _codes(B, g, T, d, lengths, gen):
    """Random codes below each length (finite, every finite code), NaN code above."""
    c = torch.randint(0, 256, (B, g, T, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes in written slots
    pos = torch.arange(T).view(1, 1, T, 1)
    c[pos.expand(B, g, T, d) >= torch.as_tensor(lengths).view(-1, 1, 1, 1)] = NAN_CODE
    return c


def _vmax(vc, vs, lengths, table=None, bs=16):
    vals = torch.from_numpy(oracle.e4m3_values())
    m = 0.0
    for b, L in enumerate(lengths):
        L = int(L)
        if L == 0:
            continue
        if table is None:
            rows = vc[b, :, :L]
        else:
            rows = torch.cat([vc[int(table[b, p // bs]), :, p % bs].unsqueeze(1)
                              for p in range(L)], 1)
        deq = vals[rows.long()] * vs.double().view(-1, 1, 1)
        m = max(m, float(deq.abs().max()))
    return m


def test_quantising_append_bit_exact():
    """Special values: midpoints between neighbouring codes (ties), values
    past 448 and infinities (saturation), values below half the smallest
    subnormal (signed zero), NaN, and random magnitudes over 2^-12 .. 2^10."""
    _log("case fp8_append")
    gen = torch.Generator().manual_seed(1200)
    B, g, d, T = 6, 4, 128, 40
    v = oracle.e4m3_values()
    mids = torch.from_numpy(((v[:126] + v[1:127]) / 2).astype(np.float32))
    special = torch.cat([mids, -mids, torch.tensor([500.0, -1e4, float("inf"), float("-inf"),
                                                    1e-9, -1e-9, 0.0, -0.0, float("nan")])])
    rnd = torch.randn(B * g * d, generator=gen) * torch.exp2(torch.randint(-12, 10, (B * g * d,),
                                                                         generator=gen).float())
    x = rnd.clone()
    x[: special.numel()] = special
    k_new = x.view(B, g, d).to(torch.bfloat16)
    v_new = (-x).view(B, g, d).to(torch.bfloat16)
    ks = torch.tensor([1.0, 0.5, 0.03125, 3.0], dtype=torch.float32)  # exact and inexact quotients
    vs = torch.tensor([2.0, 1.0, 0.1, 0.7], dtype=torch.float32)
    kc = torch.full((B, g, T, d), 0x55, dtype=torch.uint8)
    vc = kc.clone()
    before = torch.tensor([0, 1, 17, 38, 39, 40], dtype=torch.int32)  # 40: past the capacity, skipped
    kd, vd = dev(kc), dev(vc)
    kvc.append_fp8(dev(k_new), dev(v_new), kd, vd, dev(ks), dev(vs), dev(before))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(k_new[:5].unsqueeze(2), v_new[:5].unsqueeze(2), kc[:5].numpy(),
                               vc[:5].numpy(), ks.numpy(), vs.numpy(), before[:5])
    assert np.array_equal(kd.cpu()[:5].numpy(), ek) and np.array_equal(vd.cpu()[:5].numpy(), ev)
    assert torch.equal(kd.cpu()[5], kc[5])  # nothing written past the capacity


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("num_splits", [0, 1, 3, -1])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_fp8(shape, num_splits, paged):
    name, s = shape
    _log(f"case fp8_decode {name} splits={num_splits} paged={paged}")
    gen = torch.Generator().manual_seed(1201)
    B, g, h, d = len(EDGE), s["g"], s["h"], s["d"]
    T = max(EDGE) + 15
    lengths = torch.tensor(EDGE, dtype=torch.int32)
    kc = _codes(B, g, T, d, lengths, gen)
    vc = _codes(B, g, T, d, lengths, gen)
    ks, vs = _scales(g, gen)
    q = W.randn((B, h, d), torch.bfloat16, gen)
    sc = float(d) ** -0.5
    table = None
    if paged:
        table, nb = W.make_block_table(lengths, 16, perm_seed=1202, extra_blocks=2)
        kc = W.scatter_to_pool(kc, lengths, table, nb, 16, fill=NAN_CODE)
        vc = W.scatter_to_pool(vc, lengths, table, nb, 16, fill=NAN_CODE)
    out, lse = kvc.decode_fp8(dev(q), dev(kc), dev(vc), dev(ks), dev(vs), dev(lengths),
                              block_table=dev(table) if paged else None, scale=sc,
                              num_splits=num_splits)
    ro, rl = oracle.decode_fp8(q, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), lengths, sc,
                               block_table=table)
    e = check_parity(out, lse, ro, rl, _vmax(vc, vs, lengths, table), name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[4], SHAPES[6], SHAPES[7]],
                         ids=["valu_m1", "mfma_m8", "mfma_m32", "generic_d64"])
@pytest.mark.parametrize("paged", [False, True])
def test_append_decode_fp8(shape, paged):
    """One call: the new token is quantised, written, and attended to as its
    code (what the cache now holds)."""
    name, s = shape
    _log(f"case fp8_fused {name} paged={paged}")
    gen = torch.Generator().manual_seed(1203)
    B, g, h, d = len(EDGE), s["g"], s["h"], s["d"]
    T = max(EDGE) + 16
    before = torch.tensor(EDGE, dtype=torch.int32)
    kc = _codes(B, g, T, d, before, gen)
    vc = _codes(B, g, T, d, before, gen)
    ks, vs = _scales(g, gen)
    q = W.randn((B, h, d), torch.bfloat16, gen)
    kn = W.randn((B, g, d), torch.bfloat16, gen)
    vn = W.randn((B, g, d), torch.bfloat16, gen)
    table = None
    if paged:
        table, nb = W.make_block_table(before + 1, 16, perm_seed=1204, extra_blocks=2)
        kc = W.scatter_to_pool(kc, before, table, nb, 16, fill=NAN_CODE)
        vc = W.scatter_to_pool(vc, before, table, nb, 16, fill=NAN_CODE)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8(dev(q), kd, vd, dev(ks), dev(vs), dev(before),
                              block_table=dev(table) if paged else None, k_new=dev(kn),
                              v_new=dev(vn))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(kn.unsqueeze(2), vn.unsqueeze(2), kc.numpy(), vc.numpy(),
                               ks.numpy(), vs.numpy(), before, block_table=table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev)
    after = before + 1
    ro, rl = oracle.decode_fp8(q, ek, ev, ks.numpy(), vs.numpy(), after, d ** -0.5,
                               block_table=table)
    check_parity(out, lse, ro, rl, _vmax(torch.from_numpy(ev), vs, after, table), name)


def test_fp8_full_size_70b():
    """The 70B GQA shape with an FP8 cache, one-call step, in the launch the
    benchmark times; cache bytes bit-exact and attention within the bar."""
    _log("case fp8_full_70b")
    w = W.WORKLOADS["gqa_70b_bf16"]
    gen = torch.Generator().manual_seed(1205)
    before = torch.full((w.B,), w.T, dtype=torch.int32)
    T = w.T + 16
    kc = _codes(w.B, w.g, T, w.d, before, gen)
    vc = _codes(w.B, w.g, T, w.d, before, gen)
    ks, vs = _scales(w.g, gen)
    q = W.randn((w.B, w.h, w.d), torch.bfloat16, gen)
    kn = W.randn((w.B, w.g, w.d), torch.bfloat16, gen)
    vn = W.randn((w.B, w.g, w.d), torch.bfloat16, gen)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8(dev(q), kd, vd, dev(ks), dev(vs), dev(before), k_new=dev(kn),
                              v_new=dev(vn))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(kn.unsqueeze(2), vn.unsqueeze(2), kc.numpy(), vc.numpy(),
                               ks.numpy(), vs.numpy(), before)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev)
    ro, rl = oracle.decode_fp8(q, ek, ev, ks.numpy(), vs.numpy(), before + 1, w.scale)
    e = check_parity(out, lse, ro, rl, _vmax(torch.from_numpy(ev), vs, before + 1), "fp8 70b")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


def test_fp8_full_size_paged():
    """The paged GQA workload (64 sequences of 128..8192 positions, blocks
    of 16 in a seeded permutation) with an FP8 cache, one-call step, in the
    launch the benchmark times; the pools hold seeded random codes."""
    _log("case fp8_full_paged")
    w = W.WORKLOADS["paged_gqa_bf16"]
    x = W.make_paged(w)
    gen = torch.Generator().manual_seed(1206)
    shape = x["k_pool"].shape
    kc = torch.randint(0, 256, shape, generator=gen, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, shape, generator=gen, dtype=torch.int32).to(torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    ks, vs = _scales(w.g, gen)
    before, after, table = x["seq_lens_before"], x["seq_lens_after"], x["block_table"]
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8(dev(x["q"]), kd, vd, dev(ks), dev(vs), dev(before),
                              block_table=dev(table), scale=x["scale"], num_splits=w.num_splits,
                              k_new=dev(x["k_new"]), v_new=dev(x["v_new"]))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(x["k_new"].unsqueeze(2), x["v_new"].unsqueeze(2), kc.numpy(),
                               vc.numpy(), ks.numpy(), vs.numpy(), before, block_table=table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev)
    ro, rl = oracle.decode_fp8(x["q"], ek, ev, ks.numpy(), vs.numpy(), after, x["scale"],
                               block_table=table)
    vals = torch.from_numpy(oracle.e4m3_values())
    evt = torch.from_numpy(ev)
    vmax = 0.0
    for b in range(w.B):
        L = int(after[b])
        nb = (L + 15) // 16
        rows = evt[table[b, :nb].long()].permute(1, 0, 2, 3).reshape(w.g, nb * 16, w.d)[:, :L]
        vmax = max(vmax, float((vals[rows.long()] * vs.double().view(-1, 1, 1)).abs().max()))
    e = check_parity(out, lse, ro, rl, vmax, "fp8 paged")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


def test_fp8_launch_shape_70b():
    """The 70B GQA shape with an FP8 cache runs two chunks of about 2080
    positions per (sequence, KV head) on 4-wavefront work-groups on a
    256-CU device (measured faster than one 8-wavefront work-group per
    unit), merged afterwards."""
    w = W.WORKLOADS["gqa_70b_bf16"]
    waves, wgs, cl, nc = kvc.launch_shape(w.B, w.h, w.g, w.d, w.T + 16, 0, dtype="fp8")
    _log(f"case fp8_launch_shape waves={waves} wgs={wgs} chunks={nc}")
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (waves, wgs, nc) == (4, 2 * w.B * w.g, 2)


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[4], SHAPES[6]],
                         ids=["valu_m1", "mfma_m8", "mfma_m32"])
@pytest.mark.parametrize("num_splits", [0, -1])
@pytest.mark.parametrize("paged", [False, True])
def test_score_staircase_fp8(shape, num_splits, paged):
    """K codes of 0.5 * min(floor(p / 37), 16) (exact in E4M3) with K scale 1
    and q row i = 1 + (i mod 8)/8: the scores climb by 8.2 (1 + (i mod 8)/8)
    log2 units at each of 16 steps that do not line up with the tiles, so
    the running maximum moves again and again mid-sequence."""
    name, s = shape
    _log(f"case fp8_staircase {name} splits={num_splits} paged={paged}")
    gen = torch.Generator().manual_seed(1210)
    lengths = torch.tensor([1, 37, 38, 100, 1000, 4097], dtype=torch.int32)
    B, g, h, d = len(lengths), s["g"], s["h"], s["d"]
    T = int(lengths.max()) + 15
    vals = oracle.e4m3_values()
    level = 0.5 * np.minimum(np.arange(T) // 37, 16)
    code_of = {float(vals[c]): c for c in range(0x7F)}  # non-negative codes
    kcode = torch.tensor([code_of[float(x)] for x in level], dtype=torch.uint8)
    kc = kcode.view(1, 1, T, 1).expand(B, g, T, d).clone()
    kc[torch.arange(T).view(1, 1, T, 1).expand(B, g, T, d) >= lengths.view(-1, 1, 1, 1)] = NAN_CODE
    vc = _codes(B, g, T, d, lengths, gen)
    ks = torch.ones(g, dtype=torch.float32)
    _, vs = _scales(g, gen)
    q = (1.0 + (torch.arange(h) % 8).to(torch.float32) / 8.0).view(1, h, 1).expand(B, h, d)
    q = q.to(torch.bfloat16).contiguous()
    sc = float(d) ** -0.5
    table = None
    if paged:
        table, nb = W.make_block_table(lengths, 16, perm_seed=1211, extra_blocks=2)
        kc = W.scatter_to_pool(kc, lengths, table, nb, 16, fill=NAN_CODE)
        vc = W.scatter_to_pool(vc, lengths, table, nb, 16, fill=NAN_CODE)
    out, lse = kvc.decode_fp8(dev(q), dev(kc), dev(vc), dev(ks), dev(vs), dev(lengths),
                              block_table=dev(table) if paged else None, scale=sc,
                              num_splits=num_splits)
    ro, rl = oracle.decode_fp8(q, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), lengths, sc,
                               block_table=table)
    check_parity(out, lse, ro, rl, _vmax(vc, vs, lengths, table), name + "/staircase")
