"""GPU parity of the one-call decode step (kvc_append_decode_attention[_paged]):
the cache afterwards is byte-identical to the oracle's append, and out / lse
meet the parity bar against the oracle on that cache.  Unwritten slots hold
NaN, the new token's slot included, so a kernel that read the new token from
the cache instead of from k_new / v_new would give NaN."""
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

SHAPES = [
    ("valu_m1", dict(h=4, g=4, d=128, dtype="bf16")),
    ("valu_m2", dict(h=8, g=4, d=128, dtype="bf16")),
    ("valu_m3", dict(h=6, g=2, d=128, dtype="bf16")),
    ("mfma_m4", dict(h=8, g=2, d=128, dtype="bf16")),
    ("mfma_m8", dict(h=16, g=2, d=128, dtype="bf16")),
    ("mfma_m12", dict(h=24, g=2, d=128, dtype="bf16")),
    ("mfma_m32", dict(h=32, g=1, d=128, dtype="bf16")),
    ("generic_m64", dict(h=64, g=1, d=128, dtype="bf16")),
    ("generic_f32_d16", dict(h=4, g=2, d=16, dtype="f32")),
]
# lengths before the step: 0 (the new token alone), tile / page / window
# edges, and the last slot of the capacity
BEFORE = [0, 1, 15, 16, 31, 32, 33, 127, 128, 1000, 4095, 4096, 4200]
T_CAP = 4201


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.view(torch.int32).numpy().view(np.uint32)


def _raw_np(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def _to_torch(a: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    if like.dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("num_splits", [0, 1, 3, -1])
def test_fused_contiguous(shape, num_splits):
    name, s = shape
    _log(f"case fused_contig {name} splits={num_splits}")
    before = torch.tensor(BEFORE, dtype=torch.int32)
    w = W.Workload(name, B=len(BEFORE), seed=800, **s)
    x = W.make_contiguous(w, lengths=before, t_cap=T_CAP, fill=float("nan"))
    kc, vc = dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.append_decode(dev(x["q"]), dev(x["k_new"]), dev(x["v_new"]), kc, vc, dev(before),
                                 scale=x["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], before)
    assert np.array_equal(_raw(kc), _raw_np(ek)) and np.array_equal(_raw(vc), _raw_np(ev)), \
        f"{name}: cache after the fused step differs from the oracle's append"
    k_host, v_host = _to_torch(ek, x["k_cache"]), _to_torch(ev, x["v_cache"])
    after = before + 1
    ro, rl = oracle.decode(x["q"], k_host, v_host, after, x["scale"])
    e = check_parity(out, lse, ro, rl, attended_vmax_contig(v_host, after), name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("num_splits,block_size", [(0, 16), (2, 16), (-1, 8), (1, 32)])
def test_fused_paged(shape, num_splits, block_size):
    name, s = shape
    _log(f"case fused_paged {name} splits={num_splits} bs={block_size}")
    before = torch.tensor(BEFORE, dtype=torch.int32)
    w = W.Workload(name, B=len(BEFORE), seed=801, block_size=block_size, paged=True, **s)
    x = W.make_paged(w, lengths=before, fill=float("nan"))
    kp, vp = dev(x["k_pool"]), dev(x["v_pool"])
    out, lse = kvc.append_decode(dev(x["q"]), dev(x["k_new"]), dev(x["v_new"]), kp, vp, dev(before),
                                 block_table=dev(x["block_table"]), scale=x["scale"],
                                 num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_pool"], x["v_pool"], before,
                           block_table=x["block_table"])
    assert np.array_equal(_raw(kp), _raw_np(ek)) and np.array_equal(_raw(vp), _raw_np(ev)), \
        f"{name}: pool after the fused step differs from the oracle's append"
    k_host, v_host = _to_torch(ek, x["k_pool"]), _to_torch(ev, x["v_pool"])
    after = before + 1
    ro, rl = oracle.decode(x["q"], k_host, v_host, after, x["scale"], block_table=x["block_table"],
                           block_size=block_size)
    check_parity(out, lse, ro, rl, attended_vmax_paged(v_host, x["block_table"], after, block_size),
                 name)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_fused_workload_full_size(name):
    """Every workload at full size through the one-call step, in the launch
    configuration the benchmark times."""
    w = W.WORKLOADS[name]
    _log(f"case fused_full {name}")
    if w.paged:
        x = W.make_paged(w)
        kc, vc, bt = dev(x["k_pool"]), dev(x["v_pool"]), dev(x["block_table"])
    else:
        x = W.make_contiguous(w)
        kc, vc, bt = dev(x["k_cache"]), dev(x["v_cache"]), None
    before, after = x["seq_lens_before"], x["seq_lens_after"]
    out, lse = kvc.append_decode(dev(x["q"]), dev(x["k_new"]), dev(x["v_new"]), kc, vc, dev(before),
                                 block_table=bt, scale=x["scale"], num_splits=w.num_splits)
    torch.cuda.synchronize()
    if w.paged:
        ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_pool"], x["v_pool"], before,
                               block_table=x["block_table"])
    else:
        ek, ev = oracle.append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], before)
    assert np.array_equal(_raw(kc), _raw_np(ek)) and np.array_equal(_raw(vc), _raw_np(ev)), name
    like = x["k_pool"] if w.paged else x["k_cache"]
    k_host, v_host = _to_torch(ek, like), _to_torch(ev, like)
    if w.paged:
        ro, rl = oracle.decode(x["q"], k_host, v_host, after, x["scale"],
                               block_table=x["block_table"], block_size=x["block_size"])
        vmax = attended_vmax_paged(v_host, x["block_table"], after, x["block_size"])
    else:
        ro, rl = oracle.decode(x["q"], k_host, v_host, after, x["scale"])
        vmax = attended_vmax_contig(v_host, after)
    e = check_parity(out, lse, ro, rl, vmax, name)
    _log(f"  {name}: out err/vmax {e[0]:.2e}, lse err {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[4]], ids=["valu_m1", "mfma_m8"])
@pytest.mark.parametrize("paged", [False, True])
def test_fused_incremental_40_steps(shape, paged):
    """zwjcode.cn 'KV Cache 的增量解码' section 07: 40 one-call steps; the
    cache grows by one slot per step and every step matches the oracle."""
    name, s = shape
    _log(f"case fused_incremental {name} paged={paged}")
    steps, prefix, B = 40, 100, 3
    w = W.Workload(name, B=B, T=prefix, seed=802, **s)
    x = W.make_contiguous(w, t_cap=prefix + steps + 8)
    gen = torch.Generator().manual_seed(803)
    knew = W.randn((steps, B, w.g, w.d), w.torch_dtype, gen)
    vnew = W.randn((steps, B, w.g, w.d), w.torch_dtype, gen)
    qs = W.randn((steps, B, w.h, w.d), w.torch_dtype, gen)
    k_host, v_host = x["k_cache"].clone(), x["v_cache"].clone()
    lengths = torch.full((B,), prefix, dtype=torch.int32)
    table = None
    if paged:
        table, nb = W.make_block_table(torch.full((B,), prefix + steps, dtype=torch.int32), 16,
                                       perm_seed=804)
        k_host = W.scatter_to_pool(x["k_cache"], lengths, table, nb, 16)
        v_host = W.scatter_to_pool(x["v_cache"], lengths, table, nb, 16)
    kd, vd = dev(k_host), dev(v_host)
    bt = dev(table) if paged else None
    for t in range(steps):
        before = lengths.clone()
        after = before + 1
        out, lse = kvc.append_decode(dev(qs[t]), dev(knew[t]), dev(vnew[t]), kd, vd, dev(before),
                                     block_table=bt)
        ek, ev = oracle.append(knew[t], vnew[t], k_host, v_host, before, block_table=table)
        k_host, v_host = _to_torch(ek, k_host), _to_torch(ev, v_host)
        assert torch.equal(kd.cpu(), k_host) and torch.equal(vd.cpu(), v_host), f"step {t}"
        if paged:
            ro, rl = oracle.decode(qs[t], k_host, v_host, after, w.scale, block_table=table)
            vmax = attended_vmax_paged(v_host, table, after, 16)
        else:
            ro, rl = oracle.decode(qs[t], k_host, v_host, after, w.scale)
            vmax = attended_vmax_contig(v_host, after)
        check_parity(out, lse, ro, rl, vmax, f"{name}/step{t}")
        lengths = after


def test_fused_full_cache_appends_nothing():
    """A sequence whose cache is full attends to its t_cap positions and
    appends nothing, as kvc_append followed by a decode does."""
    _log("case fused_full_cache")
    w = W.Workload("fc", B=3, h=16, g=2, d=128, dtype="bf16", T=40, seed=805)
    x = W.make_contiguous(w, t_cap=48)
    before = torch.tensor([48, 47, 2000], dtype=torch.int32)
    kc, vc = dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.append_decode(dev(x["q"]), dev(x["k_new"]), dev(x["v_new"]), kc, vc, dev(before),
                                 scale=x["scale"])
    torch.cuda.synchronize()
    # only sequence 1 has a free slot: the oracle appends for it alone
    k_host, v_host = x["k_cache"].clone(), x["v_cache"].clone()
    ek, ev = oracle.append(x["k_new"][1:2], x["v_new"][1:2], x["k_cache"][1:2], x["v_cache"][1:2],
                           before[1:2])
    k_host[1:2], v_host[1:2] = _to_torch(ek, x["k_cache"]), _to_torch(ev, x["v_cache"])
    assert torch.equal(kc.cpu(), k_host) and torch.equal(vc.cpu(), v_host)
    after = torch.clamp(before + 1, max=48)
    ro, rl = oracle.decode(x["q"], k_host, v_host, after, x["scale"])
    check_parity(out, lse, ro, rl, attended_vmax_contig(v_host, after), "full_cache")
