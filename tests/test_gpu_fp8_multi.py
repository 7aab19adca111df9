"""GPU parity of FP8 E4M3 caches with several new tokens per sequence and
with sliding windows (kvc_*_fp8_multi, kvc_*_fp8_window): the n new tokens'
codes written by the one-call step are bit-exact against the oracle's
quantising append, and attention matches the oracle's dequantise-then-exact
window reference (pinned to torch SDPA over torch's dequantisation), for
every kernel family (rows per KV head: 1-3 vector ALUs, 4-32 matrix cores,
more as 32-row slices), layout (contiguous, ring, paged) and split mode.
Unwritten slots hold the NaN code."""
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

NAN_CODE = 0x7F
# (id, h, g, n); head dim 128 unless the id says d64 / d80 / d96 / d256.
# Rows per KV head (h / g) * n: 1-3 the VALU kernel, 4-32 the matrix-core
# decode kernel, more (and every row count at d = 64, 80, 96, 256) the
# multi-row kernel.
SHAPES = [
    ("valu_rows2", 4, 4, 2),
    ("valu_rows3", 6, 2, 1),
    ("mfma_rows8", 8, 2, 2),
    ("mfma_rows32", 16, 2, 4),
    ("multirow_rows40", 8, 1, 5),
    ("multirow_mha_n33", 2, 2, 33),
    ("multirow_rows96", 4, 2, 48),
    ("multirow_rows320", 32, 2, 20),
    ("multirow_d64_rows6", 6, 2, 2),
    ("multirow_d80_rows6", 6, 2, 2),
    ("multirow_d80_rows160", 16, 2, 20),
    ("multirow_d96_rows6", 6, 2, 2),
    ("multirow_d96_rows160", 16, 2, 20),
    ("multirow_d256_rows4", 8, 2, 1),
    ("multirow_d256_rows160", 16, 2, 20),
]


def _head_dim(name):
    for d in (64, 80, 96, 256):
        if f"d{d}_" in name:
            return d
    return 128
BEFORE = [0, 1, 15, 33, 500, 4096]


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(h, g, n, d, layout, window, seed, bs=16):
    gen = torch.Generator().manual_seed(seed)
    before = torch.tensor(BEFORE, dtype=torch.int32)
    B = len(BEFORE)
    ks = (torch.rand(g, generator=gen) * 0.4 + 0.02).to(torch.float32)
    vs = (torch.rand(g, generator=gen) * 0.4 + 0.02).to(torch.float32)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    v_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    ring = layout == "ring"
    t_cap = (window + n - 1 + 4) if ring else max(BEFORE) + n + 3
    kc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    if not ring:
        pos = torch.arange(t_cap).view(1, 1, t_cap, 1)
        unwritten = pos.expand(B, g, t_cap, d) >= before.view(-1, 1, 1, 1)
        kc[unwritten] = NAN_CODE
        vc[unwritten] = NAN_CODE
    table = None
    if layout == "paged":
        table, nb = W.make_block_table(before + n, bs, perm_seed=seed + 1, extra_blocks=2)
        kc = W.scatter_to_pool(kc, before, table, nb, bs, fill=NAN_CODE)
        vc = W.scatter_to_pool(vc, before, table, nb, bs, fill=NAN_CODE)
    return before, q, k_new, v_new, kc, vc, ks, vs, table, t_cap


def _vmax(vc, vs, before, n, window, layout, table, t_cap, bs=16):
    vals = torch.from_numpy(oracle.e4m3_values())
    m = 0.0
    for b in range(len(before)):
        hi = int(before[b]) + n
        lo = max(0, int(before[b]) + 1 - window) if window else 0
        for p in range(lo, hi):
            if layout == "paged":
                row = vc[int(table[b, p // bs]), :, p % bs]
            else:
                row = vc[b, :, p % t_cap if layout == "ring" else p]
            m = max(m, float((vals[row.long()] * vs.double().view(-1, 1)).abs().max()))
    return m


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("layout", ["linear", "ring", "paged"])
@pytest.mark.parametrize("window", [0, 37])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_append_decode_fp8_multi_window(shape, layout, window, num_splits):
    name, h, g, n = shape
    if layout == "ring" and window == 0:
        pytest.skip("a ring cache needs a window")
    d = _head_dim(name)
    _log(f"case fp8_multi {name} n={n} {layout} W={window} splits={num_splits}")
    before, q, k_new, v_new, kc, vc, ks, vs, table, t_cap = _case(h, g, n, d, layout, window, 1400)
    ring, paged = layout == "ring", layout == "paged"
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8_window(dev(q), kd, vd, dev(ks), dev(vs), dev(before), window=window,
                                     ring=ring, block_table=dev(table) if paged else None,
                                     num_splits=num_splits, k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(k_new, v_new, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), before,
                               block_table=table, ring=ring)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev), \
        f"{name}: codes after the step differ from the oracle's quantising append"
    ro, rl = oracle.decode_fp8_window(q, ek, ev, ks.numpy(), vs.numpy(), before, d ** -0.5, window,
                                      ring=ring, block_table=table)
    vmax = _vmax(torch.from_numpy(ev), vs, before, n, window, layout, table, t_cap)
    e = check_parity(out, lse, ro, rl, vmax, name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[3], SHAPES[4], SHAPES[6], SHAPES[10]],
                         ids=[SHAPES[0][0], SHAPES[3][0], SHAPES[4][0], SHAPES[6][0], SHAPES[10][0]])
@pytest.mark.parametrize("layout", ["linear", "paged"])
def test_decode_fp8_multi_over_filled_cache(shape, layout):
    """The tokens' codes are already in the cache; seq_lens counts them."""
    name, h, g, n = shape
    d = _head_dim(name)
    _log(f"case fp8_multi_filled {name} {layout}")
    before, q, k_new, v_new, kc, vc, ks, vs, table, t_cap = _case(h, g, n, d, layout, 0, 1410)
    ek, ev = oracle.append_fp8(k_new, v_new, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), before,
                               block_table=table)
    out, lse = kvc.decode_fp8_window(dev(q), dev(torch.from_numpy(ek)), dev(torch.from_numpy(ev)),
                                     dev(ks), dev(vs), dev(before + n),
                                     block_table=dev(table) if layout == "paged" else None,
                                     num_splits=2)
    ro, rl = oracle.decode_fp8_window(q, ek, ev, ks.numpy(), vs.numpy(), before, d ** -0.5, 0,
                                      block_table=table)
    check_parity(out, lse, ro, rl,
                 _vmax(torch.from_numpy(ev), vs, before, n, 0, layout, table, t_cap), name)


@pytest.mark.parametrize("n,window", [(4, 0), (1, 1024)])
def test_fp8_multi_window_full_size_70b(n, window):
    """The 70B GQA cache as FP8 codes (per-KV-head scales amax / 448) with 4
    tokens per sequence, and one token under a window of 1024, in the
    launch the benchmark times; attention rows of sampled sequences against
    the oracle."""
    _log(f"case fp8_full_70b n={n} W={window}")
    w = W.WORKLOADS["gqa_70b_bf16"]
    x = W.make_contiguous(w)
    gen = torch.Generator().manual_seed(1420 + n)

    def quantise(t):
        sc = (t.float().abs().amax(dim=(0, 2, 3)) / 448.0).clamp(min=1e-12)
        return (t.float() / sc.view(1, -1, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8), sc
    kc, ks = quantise(x["k_cache"])
    vc, vs = quantise(x["v_cache"])
    q = W.randn((w.B, w.h, n, w.d), torch.bfloat16, gen)
    k_new = W.randn((w.B, w.g, n, w.d), torch.bfloat16, gen)
    v_new = W.randn((w.B, w.g, n, w.d), torch.bfloat16, gen)
    before = x["seq_lens_before"]
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8_window(dev(q), kd, vd, dev(ks), dev(vs), dev(before), window=window,
                                     k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    seqs = [0, 17, 31]
    ek, ev = oracle.append_fp8(k_new[seqs], v_new[seqs], kc[seqs].numpy(), vc[seqs].numpy(),
                               ks.numpy(), vs.numpy(), before[seqs])
    assert np.array_equal(kd.cpu()[seqs].numpy(), ek) and np.array_equal(vd.cpu()[seqs].numpy(), ev)
    ro, rl = oracle.decode_fp8_window(q[seqs], ek, ev, ks.numpy(), vs.numpy(), before[seqs],
                                      x["scale"], window)
    vmax = _vmax(torch.from_numpy(ev), vs, before[seqs], n, window, "linear", None, ek.shape[2])
    e = check_parity(out[seqs], lse[seqs], ro, rl, vmax, f"70b fp8 n={n} W={window}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("n", [128])
def test_fp8_many_tokens_full_size_70b(n):
    """The 70B GQA cache as FP8 codes with 128 new tokens per sequence (1024
    query rows per KV head: the multi-row kernel, codes widened to bf16 as
    they are staged), in the launch the benchmark times: the new codes of
    sampled sequences against the quantising append, and attention rows of
    sampled tokens against the oracle, each computed alone."""
    _log(f"case fp8_full_70b_many n={n}")
    w = W.WORKLOADS["gqa_70b_bf16"]
    x = W.make_contiguous(w, t_cap=w.T + n + w.cap_pad)
    gen = torch.Generator().manual_seed(1430 + n)

    def quantise(t):
        sc = (t.float().abs().amax(dim=(0, 2, 3)) / 448.0).clamp(min=1e-12)
        return (t.float() / sc.view(1, -1, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8), sc
    kc, ks = quantise(x["k_cache"])
    vc, vs = quantise(x["v_cache"])
    q = W.randn((w.B, w.h, n, w.d), torch.bfloat16, gen)
    k_new = W.randn((w.B, w.g, n, w.d), torch.bfloat16, gen)
    v_new = W.randn((w.B, w.g, n, w.d), torch.bfloat16, gen)
    before = x["seq_lens_before"]
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8_window(dev(q), kd, vd, dev(ks), dev(vs), dev(before),
                                     k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    seqs = [0, 31]
    ek, ev = oracle.append_fp8(k_new[seqs], v_new[seqs], kc[seqs].numpy(), vc[seqs].numpy(),
                               ks.numpy(), vs.numpy(), before[seqs])
    assert np.array_equal(kd.cpu()[seqs].numpy(), ek) and np.array_equal(vd.cpu()[seqs].numpy(), ev)
    out_h, lse_h = out.cpu()[seqs], lse.cpu()[seqs]
    for t in [0, 1, 64, n - 1]:
        vis = before[seqs] + t  # token t sees before + t + 1 positions: a single token after before + t
        ro, rl = oracle.decode_fp8(q[seqs, :, t].contiguous(), ek, ev, ks.numpy(), vs.numpy(),
                                   vis + 1, x["scale"])
        vmax = _vmax(torch.from_numpy(ev), vs, vis, 1, 0, "linear", None, ek.shape[2])
        e = check_parity(out_h[:, :, t], lse_h[:, :, t], ro, rl, vmax, f"70b fp8 n={n} t={t}")
    _log(f"  last sampled token err/vmax {e[0]:.2e} lse {e[1]:.2e}")
