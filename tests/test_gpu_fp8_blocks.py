"""GPU parity of paged FP8 pools with a scale per (physical block, KV head)
(kvc_append_fp8_paged_block_scaled, kvc_decode_attention_fp8_paged_block_scaled):
the quantising appends are bit-exact against the oracle (each new code made
with its target block's scale), and attention matches the oracle's
dequantise-then-exact reference (pinned to torch SDPA over torch's per-block
dequantisation) for every kernel family, one and several tokens per
sequence, windows, split modes, and the paged GQA workload at full size."""
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
# (id, h, g, n, d): rows per KV head pick the kernel family
SHAPES = [
    ("valu_m1", 4, 4, 1, 128),
    ("valu_rows3", 6, 2, 1, 128),
    ("valu_rows2_n2", 4, 4, 2, 128),
    ("mfma_m4", 8, 2, 1, 128),
    ("mfma_m8_n3", 16, 2, 3, 128),
    ("mfma_m32", 32, 1, 1, 128),
    ("mfma_slices40", 8, 1, 5, 128),
    ("generic_d64", 8, 2, 2, 64),
]
BEFORE = [0, 1, 15, 16, 17, 100, 2000]


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(h, g, n, d, seed, bs):
    gen = torch.Generator().manual_seed(seed)
    before = torch.tensor(BEFORE, dtype=torch.int32)
    B = len(BEFORE)
    table, nb = W.make_block_table(before + n, bs, perm_seed=seed + 1, extra_blocks=2)
    kc = torch.randint(0, 256, (nb, g, bs, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (nb, g, bs, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    for b in range(B):  # slots at or past each length hold the NaN code
        for p in range(int(before[b]), (int(before[b]) + n + bs - 1) // bs * bs):
            blk = int(table[b, p // bs])
            kc[blk, :, p % bs] = NAN_CODE
            vc[blk, :, p % bs] = NAN_CODE
    ks = (torch.rand(nb, g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    vs = (torch.rand(nb, g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    v_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    return before, q, k_new, v_new, kc, vc, ks, vs, table


def _vmax(vc, vs, table, before, n, window, bs):
    vals = oracle.e4m3_values()
    m = 0.0
    for b in range(len(before)):
        hi = int(before[b]) + n
        lo = max(0, int(before[b]) + 1 - window) if window else 0
        for p in range(lo, hi):
            blk = int(table[b, p // bs])
            m = max(m, float(np.max(np.abs(vals[vc[blk, :, p % bs]] * vs[blk].reshape(-1, 1)))))
    return m


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("window", [0, 37])
@pytest.mark.parametrize("num_splits", [0, 3, kvc.SPLITS_STREAM])
@pytest.mark.parametrize("bs", [8, 16])
def test_append_decode_block_scaled(shape, window, num_splits, bs):
    """Every kernel family; the stream grid where asked for (up to 16 rows
    per KV head: with two query tiles a request for it takes chunks)."""
    name, h, g, n, d = shape
    _log(f"case fp8_blocks {name} n={n} W={window} splits={num_splits} bs={bs}")
    before, q, k_new, v_new, kc, vc, ks, vs, table = _case(h, g, n, d, 1500, bs)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8_block_scaled(dev(q), kd, vd, dev(ks), dev(vs), dev(before),
                                           dev(table), window=window, num_splits=num_splits,
                                           k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8_block_scaled(k_new, v_new, kc.numpy(), vc.numpy(), ks.numpy(),
                                            vs.numpy(), before, table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev), \
        f"{name}: pools after the step differ from the oracle's append"
    ro, rl = oracle.decode_fp8_block_scaled(q, ek, ev, ks.numpy(), vs.numpy(), before, d ** -0.5,
                                            table, bs, window=window)
    e = check_parity(out, lse, ro, rl, _vmax(ev, vs.numpy(), table, before, n, window, bs), name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[4], SHAPES[6]],
                         ids=[SHAPES[0][0], SHAPES[4][0], SHAPES[6][0]])
def test_standalone_append_then_decode(shape):
    """kvc_append_fp8_paged_block_scaled, then the attention over the filled
    pool (seq_lens counting the new tokens): the same as the one-call step."""
    name, h, g, n, d = shape
    _log(f"case fp8_blocks_two_calls {name}")
    bs = 16
    before, q, k_new, v_new, kc, vc, ks, vs, table = _case(h, g, n, d, 1510, bs)
    kd, vd = dev(kc), dev(vc)
    kvc.append_fp8_block_scaled(dev(k_new), dev(v_new), kd, vd, dev(ks), dev(vs), dev(before),
                                dev(table))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8_block_scaled(k_new, v_new, kc.numpy(), vc.numpy(), ks.numpy(),
                                            vs.numpy(), before, table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev)
    out, lse = kvc.decode_fp8_block_scaled(dev(q), kd, vd, dev(ks), dev(vs), dev(before + n),
                                           dev(table), num_splits=2)
    ro, rl = oracle.decode_fp8_block_scaled(q, ek, ev, ks.numpy(), vs.numpy(), before, d ** -0.5,
                                            table, bs)
    check_parity(out, lse, ro, rl, _vmax(ev, vs.numpy(), table, before, n, 0, bs), name)


def test_block_scaled_full_size_paged():
    """The paged GQA workload (B = 64, h = 32, g = 8, lengths U[128, 8192],
    pages of 16) as FP8 codes with per-(block, KV head) scales amax / 448,
    one new token per sequence, in the launch the benchmark times; the
    pools in full, and the attention rows of sampled sequences against the
    oracle over a pool holding just their blocks."""
    _log("case fp8_blocks_full_paged")
    w = W.WORKLOADS["paged_gqa_bf16"]
    x = W.make_paged(w)
    bs = x["block_size"]
    nb = x["num_blocks"]

    def quantise(pool):
        sc = (pool.float().abs().amax(dim=(2, 3)) / 448.0).clamp(min=1e-12)  # [NB, g]
        codes = (pool.float() / sc.view(nb, -1, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes, sc
    kc, ks = quantise(x["k_pool"])
    vc, vs = quantise(x["v_pool"])
    before, table = x["seq_lens_before"], x["block_table"]
    kn = x["k_new"].view(w.B, w.g, 1, w.d)
    vn = x["v_new"].view(w.B, w.g, 1, w.d)
    q = x["q"].view(w.B, w.h, 1, w.d)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.decode_fp8_block_scaled(dev(q), kd, vd, dev(ks), dev(vs), dev(before),
                                           dev(table), scale=x["scale"], k_new=dev(kn),
                                           v_new=dev(vn))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8_block_scaled(kn, vn, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(),
                                            before, table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev)
    seqs = [0, 21, 63]
    rows = [int(bl) for b in seqs for bl in table[b] if int(bl) >= 0]
    remap = {bl: i for i, bl in enumerate(rows)}
    sub_table = torch.full((len(seqs), table.shape[1]), -1, dtype=torch.int32)
    for i, b in enumerate(seqs):
        for c in range(table.shape[1]):
            if int(table[b, c]) >= 0:
                sub_table[i, c] = remap[int(table[b, c])]
    ro, rl = oracle.decode_fp8_block_scaled(q[seqs], ek[rows], ev[rows], ks.numpy()[rows],
                                            vs.numpy()[rows], before[seqs], x["scale"], sub_table,
                                            bs)
    vmax = _vmax(ev[rows], vs.numpy()[rows], sub_table, before[seqs], 1, 0, bs)
    e = check_parity(out[seqs], lse[seqs], ro, rl, vmax, "paged fp8 block scales")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")
