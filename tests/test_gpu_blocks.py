"""GPU block operations (copy-on-write block copies, block-table forks,
beam re-ranking of contiguous caches) against the oracle: bit-exact, and an
end-to-end shared-prompt scenario whose attention must equal attention over
private caches."""
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


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.view(torch.int32).numpy().view(np.uint32)


def _same(t: torch.Tensor, a: np.ndarray) -> bool:
    r = _raw(t)
    return np.array_equal(r, a.view(r.dtype))


@pytest.mark.parametrize("g,bs,d,dt", [(8, 16, 128, torch.bfloat16), (2, 8, 16, torch.float32),
                                       (1, 32, 64, torch.bfloat16), (3, 16, 1, torch.float32),
                                       (2, 8, 3, torch.bfloat16)])
def test_copy_blocks(g, bs, d, dt):
    _log(f"case copy_blocks g={g} bs={bs} d={d} {dt}")
    gen = torch.Generator().manual_seed(1100)
    nb = 40
    kp = W.randn((nb, g, bs, d), dt, gen)
    vp = W.randn((nb, g, bs, d), dt, gen)
    pairs = torch.tensor([[0, 5], [7, 3], [12, 39], [39, 39], [-1, 2], [6, nb], [20, 21]],
                         dtype=torch.int32)
    ek, ev = oracle.copy_blocks(kp, vp, pairs)
    kd, vd = dev(kp), dev(vp)
    kvc.copy_blocks(kd, vd, dev(pairs))
    torch.cuda.synchronize()
    assert _same(kd, ek) and _same(vd, ev)
    kvc.copy_blocks(kd, vd, dev(torch.zeros((0, 2), dtype=torch.int32)))   # nothing to do
    assert _same(kd, ek)


def test_fork_block_tables():
    _log("case fork_tables")
    gen = torch.Generator().manual_seed(1101)
    tables = torch.randint(-1, 500, (5, 7), generator=gen, dtype=torch.int32)
    lens = torch.randint(0, 112, (5,), generator=gen, dtype=torch.int32)
    parent = torch.tensor([4, 4, 0, 2, 1, 3, 0], dtype=torch.int32)
    et, el = oracle.fork_tables(tables, lens, parent)
    ot, ol = kvc.fork_block_tables(dev(tables), dev(lens), dev(parent))
    assert np.array_equal(ot.cpu().numpy(), et) and np.array_equal(ol.cpu().numpy(), el)
    # a parent outside [0, B_src) gives a row of -1 and length 0
    bad = torch.tensor([1, -1, 5, 2], dtype=torch.int32)
    ot, ol = kvc.fork_block_tables(dev(tables), dev(lens), dev(bad))
    assert torch.equal(ot.cpu()[0], tables[1]) and torch.equal(ot.cpu()[3], tables[2])
    assert torch.all(ot.cpu()[1:3] == -1) and ol.cpu().tolist() == [int(lens[1]), 0, 0, int(lens[2])]


@pytest.mark.parametrize("dt,d", [(torch.bfloat16, 128), (torch.float32, 16), (torch.bfloat16, 3)])
def test_gather_cache(dt, d):
    _log(f"case gather_cache {dt} d={d}")
    gen = torch.Generator().manual_seed(1102)
    B_src, g, t_cap = 4, 2, 300
    ks = W.randn((B_src, g, t_cap, d), dt, gen)
    vs = W.randn((B_src, g, t_cap, d), dt, gen)
    lens = torch.tensor([300, 65, 0, 1000], dtype=torch.int32)  # 1000: clamped to t_cap
    parent = torch.tensor([3, 1, 1, 0, 2, 3], dtype=torch.int32)
    kd0 = W.randn((6, g, t_cap, d), dt, gen)
    vd0 = W.randn((6, g, t_cap, d), dt, gen)
    kd, vd = dev(kd0), dev(vd0)
    kvc.gather_cache(dev(ks), dev(vs), dev(lens), dev(parent), kd, vd)
    torch.cuda.synchronize()
    ek, ev = oracle.gather_cache(ks, vs, parent, torch.clamp(lens, max=t_cap), k_dst=kd0, v_dst=vd0)
    assert _same(kd, ek) and _same(vd, ev)


def test_shared_prompt_copy_on_write_isolation():
    """Three requests fork one 40-token prompt (bs = 16: blocks 0, 1 full,
    block 2 partial), copy the shared partial block before writing, and each
    runs 5 one-call decode steps: every step equals attention over the
    request's private contiguous cache; the full prompt blocks stay shared
    and unchanged."""
    _log("case cow_isolation")
    gen = torch.Generator().manual_seed(1103)
    g, h, d, bs, P, steps, R = 2, 16, 128, 16, 40, 5, 3
    dt = torch.bfloat16
    nb = 32
    prompt_k = W.randn((g, P, d), dt, gen)
    prompt_v = W.randn((g, P, d), dt, gen)
    kp = torch.zeros((nb, g, bs, d), dtype=dt)
    vp = torch.zeros((nb, g, bs, d), dtype=dt)
    for lb in range(3):
        n = min(bs, P - lb * bs)
        kp[lb, :, :n] = prompt_k[:, lb * bs: lb * bs + n]
        vp[lb, :, :n] = prompt_v[:, lb * bs: lb * bs + n]
    table0 = torch.full((1, 8), -1, dtype=torch.int32)
    table0[0, :3] = torch.tensor([0, 1, 2])
    kd, vd = dev(kp), dev(vp)
    tables, lens = kvc.fork_block_tables(dev(table0), dev(torch.tensor([P], dtype=torch.int32)),
                                         dev(torch.zeros(R, dtype=torch.int32)))
    # copy-on-write of the shared partial block for requests 1 and 2
    kvc.copy_blocks(kd, vd, dev(torch.tensor([[2, 3], [2, 4]], dtype=torch.int32)))
    tables[1, 2], tables[2, 2] = 3, 4
    tables[:, 3] = torch.tensor([5, 6, 7], dtype=torch.int32, device="cuda")  # next blocks, private
    private_k = [prompt_k.clone() for _ in range(R)]
    private_v = [prompt_v.clone() for _ in range(R)]
    for step in range(steps):
        q = W.randn((R, h, d), dt, gen)
        kn = W.randn((R, g, d), dt, gen)
        vn = W.randn((R, g, d), dt, gen)
        out, lse = kvc.append_decode(dev(q), dev(kn), dev(vn), kd, vd, lens, block_table=tables)
        lens = lens + 1
        for r in range(R):
            private_k[r] = torch.cat([private_k[r], kn[r].unsqueeze(1)], 1)
            private_v[r] = torch.cat([private_v[r], vn[r].unsqueeze(1)], 1)
            L = private_k[r].shape[1]
            ro, rl = oracle.decode(q[r:r + 1], private_k[r].unsqueeze(0).contiguous(),
                                   private_v[r].unsqueeze(0).contiguous(), [L], 1.0 / d ** 0.5)
            vmax = float(private_v[r].float().abs().max())
            check_parity(out[r:r + 1], lse[r:r + 1], ro, rl, vmax, f"step {step} request {r}")
    pool_k = kd.cpu()
    for lb in range(2):
        assert torch.equal(pool_k[lb], prompt_k[:, lb * bs:(lb + 1) * bs]), "shared block changed"


def test_beam_rerank_then_decode():
    """Beams re-ranked by parent attend to their parents' histories, both by
    gathering contiguous caches and by forking paged tables."""
    _log("case beam_rerank")
    gen = torch.Generator().manual_seed(1104)
    B, g, h, d, t_cap = 4, 2, 16, 128, 700
    dt = torch.bfloat16
    w = W.Workload("beam", B=B, h=h, g=g, d=d, dtype="bf16", T_range=(1, 680), seed=1105)
    x = W.make_contiguous(w, t_cap=t_cap)
    lens = x["seq_lens_before"]
    parent = torch.tensor([2, 2, 0, 3], dtype=torch.int32)
    kd = torch.zeros((B, g, t_cap, d), dtype=dt, device="cuda")
    vd = torch.zeros_like(kd)
    kvc.gather_cache(dev(x["k_cache"]), dev(x["v_cache"]), dev(lens), dev(parent), kd, vd)
    q = W.randn((B, h, d), dt, gen)
    plens = lens[parent.long()]
    out, lse = kvc.decode(dev(q), kd, vd, dev(plens))
    ek, ev = oracle.gather_cache(x["k_cache"], x["v_cache"], parent, lens)
    kh = torch.from_numpy(ek.view(np.int16)).view(dt)
    vh = torch.from_numpy(ev.view(np.int16)).view(dt)
    ro, rl = oracle.decode(q, kh, vh, plens, 1.0 / d ** 0.5)
    vmax = max(float(vh[b, :, :int(plens[b])].float().abs().max()) for b in range(B)
               if int(plens[b]) > 0)
    check_parity(out, lse, ro, rl, vmax, "gathered beams")
    # paged: fork the tables instead of moving data
    table, nb = W.make_block_table(lens, 16, perm_seed=1106)
    kp = W.scatter_to_pool(x["k_cache"], lens, table, nb, 16)
    vp = W.scatter_to_pool(x["v_cache"], lens, table, nb, 16)
    ft, fl = kvc.fork_block_tables(dev(table), dev(lens), dev(parent))
    out2, lse2 = kvc.decode_paged(dev(q), dev(kp), dev(vp), ft, fl)
    check_parity(out2, lse2, ro, rl, vmax, "forked paged beams")
