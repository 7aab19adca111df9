"""GPU parity at byte offsets past 2^32: a contiguous cache and paged pools
of more than 4 GB each, so that the rows of the later sequences (and of the
high physical blocks) sit beyond 32-bit byte offsets.  The caches are filled
on the GPU from a seeded generator; sampled sequences are copied back and
checked against the oracle (the paged ones after gathering their rows
through the block table with torch indexing).  The decode kernels and the
multi-row kernel (many new tokens per sequence) are both covered."""
from __future__ import annotations

import sys

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import check_parity, dev

pytestmark = pytest.mark.gpu

GiB = 2 ** 30


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _randn_gpu(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, device="cuda", dtype=torch.bfloat16, generator=g)


def _vmax(rows_v: torch.Tensor) -> float:
    return float(rows_v.float().abs().max())


@pytest.mark.parametrize("num_splits", [0, -1])
def test_contiguous_cache_past_4gb(num_splits):
    _log(f"case large contiguous splits={num_splits}")
    B, h, g, d, t_cap = 64, 64, 8, 128, 40000
    # sequence 63 starts 5.2 GB into each cache
    assert (B - 1) * g * t_cap * d * 2 > 4 * GiB
    gen = torch.Generator().manual_seed(1500)
    lengths = torch.randint(1, t_cap + 1, (B,), generator=gen, dtype=torch.int32)
    lengths[-3:] = torch.tensor([39000, 39999, 40000], dtype=torch.int32)
    k = _randn_gpu((B, g, t_cap, d), 1501)
    v = _randn_gpu((B, g, t_cap, d), 1502)
    q = W.randn((B, h, d), torch.bfloat16, gen)
    scale = d ** -0.5
    out, lse = kvc.decode(dev(q), k, v, dev(lengths), scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    pick = [0, 40, B - 1]
    L = [int(lengths[b]) for b in pick]
    ks = k[pick, :, : max(L)].cpu()
    vs = v[pick, :, : max(L)].cpu()
    ro, rl = oracle.decode(q[pick], ks, vs, lengths[pick], scale)
    vmax = max(_vmax(vs[i, :, : L[i]]) for i in range(len(pick)))
    check_parity(out[pick], lse[pick], ro, rl, vmax, "large contiguous")
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h", [32, 8], ids=["mfma_m4", "valu_m1"])
@pytest.mark.parametrize("num_splits", [0, 4])
def test_paged_pools_past_4gb(h, num_splits):
    _log(f"case large paged h={h} splits={num_splits}")
    B, g, d, bs = 32, 8, 128, 16
    gen = torch.Generator().manual_seed(1510)
    lengths = torch.randint(1, 8193, (B,), generator=gen, dtype=torch.int32)
    lengths[-1] = 8192
    used = int(((lengths.to(torch.int64) + bs - 1) // bs).sum())
    nb = 140000  # 140000 * 8 * 16 * 128 * 2 B = 4.6 GB per pool
    assert nb * g * bs * d * 2 > 4 * GiB
    table, nb_out = W.make_block_table(lengths, bs, perm_seed=1511, extra_blocks=nb - used)
    assert nb_out == nb and int(table.max()) * g * bs * d * 2 > 4 * GiB
    kp = _randn_gpu((nb, g, bs, d), 1512)
    vp = _randn_gpu((nb, g, bs, d), 1513)
    q = W.randn((B, h, d), torch.bfloat16, gen)
    scale = d ** -0.5
    bt = dev(table)
    out, lse = kvc.decode_paged(dev(q), kp, vp, bt, dev(lengths), scale=scale,
                                num_splits=num_splits)
    torch.cuda.synchronize()
    # reference rows of the sampled sequences: gathered through the table
    pick = [int(torch.argmax(table.max(dim=1).values)), B - 1]
    for b in pick:
        Lb = int(lengths[b])
        pos = torch.arange(Lb, device="cuda")
        blk = bt[b, pos // bs].long()
        kr = kp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).cpu()  # [1, g, L, d]
        vr = vp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).cpu()
        ro, rl = oracle.decode(q[b:b + 1], kr.contiguous(), vr.contiguous(),
                               lengths[b:b + 1], scale)
        check_parity(out[b:b + 1], lse[b:b + 1], ro, rl, _vmax(vr), f"large paged b={b}")
    del kp, vp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h", [32, 8], ids=["mfma_m4", "valu_m1"])
def test_paged_fp8_pools_past_4gb(h):
    _log(f"case large paged fp8 h={h}")
    B, g, d, bs = 32, 8, 128, 16
    gen = torch.Generator().manual_seed(1520)
    lengths = torch.randint(1, 8193, (B,), generator=gen, dtype=torch.int32)
    used = int(((lengths.to(torch.int64) + bs - 1) // bs).sum())
    nb = 280000  # 280000 * 8 * 16 * 128 B = 4.6 GB per pool of one-byte codes
    table, _ = W.make_block_table(lengths, bs, perm_seed=1521, extra_blocks=nb - used)
    assert int(table.max()) * g * bs * d > 4 * GiB
    gg = torch.Generator(device="cuda").manual_seed(1522)
    pools = []
    for _ in range(2):
        c = torch.randint(0, 256, (nb, g, bs, d), device="cuda", dtype=torch.uint8, generator=gg)
        c[(c & 0x7F) == 0x7F] = 0x3C  # finite codes only
        pools.append(c)
    kp, vp = pools
    ks = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    vs = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
    q = W.randn((B, h, d), torch.bfloat16, gen)
    scale = d ** -0.5
    bt = dev(table)
    out, lse = kvc.decode_fp8(dev(q), kp, vp, dev(ks), dev(vs), dev(lengths), block_table=bt,
                              scale=scale)
    torch.cuda.synchronize()
    vals = torch.from_numpy(oracle.e4m3_values())
    for b in [int(torch.argmax(table.max(dim=1).values)), B - 1]:
        Lb = int(lengths[b])
        pos = torch.arange(Lb, device="cuda")
        blk = bt[b, pos // bs].long()
        kr = kp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).contiguous().cpu()
        vr = vp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).contiguous().cpu()
        ro, rl = oracle.decode_fp8(q[b:b + 1], kr.numpy(), vr.numpy(), ks.numpy(), vs.numpy(),
                                   lengths[b:b + 1], scale)
        vmax = float((vals[vr.long()] * vs.double().view(1, -1, 1, 1)).abs().max())
        check_parity(out[b:b + 1], lse[b:b + 1], ro, rl, vmax, f"large paged fp8 b={b}")
    del kp, vp, pools
    torch.cuda.empty_cache()


def test_multi_rows_contiguous_past_4gb():
    """The multi-row kernel (80 new tokens x 2 query heads per KV head = 160
    rows: 256-row work-groups of eight wavefronts) over a contiguous cache of
    5.2 GB per K and V, the sampled last sequence starting past 4 GB."""
    _log("case large multi-row contiguous")
    B, h, g, d, n, t_cap = 64, 16, 8, 128, 80, 40000
    assert (B - 1) * g * t_cap * d * 2 > 4 * GiB
    gen = torch.Generator().manual_seed(1530)
    lengths = torch.randint(n, t_cap + 1, (B,), generator=gen, dtype=torch.int32)
    lengths[-1] = t_cap
    k = _randn_gpu((B, g, t_cap, d), 1531)
    v = _randn_gpu((B, g, t_cap, d), 1532)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    scale = d ** -0.5
    out, lse = kvc.decode_multi(dev(q), k, v, dev(lengths), scale=scale)
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu(), lse.cpu()
    for b in [0, B - 1]:
        Lb = int(lengths[b])
        ks = k[b:b + 1, :, :Lb].cpu()
        vs = v[b:b + 1, :, :Lb].cpu()
        ro, rl = oracle.decode_multi(q[b:b + 1], ks, vs, lengths[b:b + 1] - n, scale)
        check_parity(out_h[b:b + 1], lse_h[b:b + 1], ro, rl, _vmax(vs), f"large multi-row b={b}")
    del k, v
    torch.cuda.empty_cache()


def test_multi_rows_paged_past_4gb():
    """The multi-row kernel over paged pools of 4.6 GB, the sampled sequences
    holding blocks past 4 GB; the reference gathers their rows through the
    table."""
    _log("case large multi-row paged")
    B, h, g, d, n, bs = 32, 16, 8, 128, 80, 16
    gen = torch.Generator().manual_seed(1540)
    lengths = torch.randint(n, 8193, (B,), generator=gen, dtype=torch.int32)
    lengths[-1] = 8192
    used = int(((lengths.to(torch.int64) + bs - 1) // bs).sum())
    nb = 140000
    table, _ = W.make_block_table(lengths, bs, perm_seed=1541, extra_blocks=nb - used)
    assert int(table.max()) * g * bs * d * 2 > 4 * GiB
    kp = _randn_gpu((nb, g, bs, d), 1542)
    vp = _randn_gpu((nb, g, bs, d), 1543)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    scale = d ** -0.5
    bt = dev(table)
    out, lse = kvc.decode_multi(dev(q), kp, vp, dev(lengths), block_table=bt, scale=scale)
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu(), lse.cpu()
    for b in [int(torch.argmax(table.max(dim=1).values)), B - 1]:
        Lb = int(lengths[b])
        pos = torch.arange(Lb, device="cuda")
        blk = bt[b, pos // bs].long()
        kr = kp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).contiguous().cpu()
        vr = vp[blk, :, pos % bs].permute(1, 0, 2).unsqueeze(0).contiguous().cpu()
        ro, rl = oracle.decode_multi(q[b:b + 1], kr, vr, lengths[b:b + 1] - n, scale)
        check_parity(out_h[b:b + 1], lse_h[b:b + 1], ro, rl, _vmax(vr), f"large multi-row paged b={b}")
    del kp, vp
    torch.cuda.empty_cache()
