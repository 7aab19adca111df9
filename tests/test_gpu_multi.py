"""GPU parity of several new tokens per sequence (kvc_*_multi): token t of a
sequence with P cached positions sits at position P + t and sees positions
0 .. P + t.  Checked against the oracle's composition of the single-token
definition (pinned to a full causal forward), for every kernel family, split
mode and layout, with NaN in every unwritten slot."""
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

# (id, shape, n): rows per KV head = (h / g) * n picks the kernel family
CASES = [
    ("valu_rows2", dict(h=4, g=4, d=128, dtype="bf16"), 2),
    ("valu_rows3", dict(h=3, g=1, d=128, dtype="bf16"), 1),
    ("valu_rows3_n3", dict(h=4, g=4, d=128, dtype="bf16"), 3),
    ("mfma_rows4", dict(h=4, g=4, d=128, dtype="bf16"), 4),
    ("mfma_rows16", dict(h=8, g=2, d=128, dtype="bf16"), 4),
    ("mfma_rows32", dict(h=16, g=2, d=128, dtype="bf16"), 4),
    ("mfma_rows30", dict(h=6, g=1, d=128, dtype="bf16"), 5),
    ("mfma_slices_64", dict(h=16, g=2, d=128, dtype="bf16"), 8),
    ("mfma_slices_33", dict(h=11, g=1, d=128, dtype="bf16"), 3),
    # one query head per KV head and more than 32 new tokens: the new
    # positions span two or more 32-position tiles
    ("mfma_mha_n33", dict(h=1, g=1, d=128, dtype="bf16"), 33),
    ("mfma_mha_n64", dict(h=2, g=2, d=128, dtype="bf16"), 64),
    ("generic_f32_d16", dict(h=4, g=2, d=16, dtype="f32"), 3),
    ("generic_f32_rows40", dict(h=8, g=1, d=16, dtype="f32"), 5),
]
BEFORE = [0, 1, 14, 15, 16, 29, 30, 31, 32, 127, 1000, 4093, 4096, 4200]
T_CAP = 4210


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


def _inputs(name, s, n, seed, paged=False, block_size=16):
    before = torch.tensor(BEFORE, dtype=torch.int32)
    B = len(BEFORE)
    w = W.Workload(name, B=B, seed=seed, block_size=block_size, paged=paged, **s)
    gen = torch.Generator().manual_seed(seed + 1)
    q = W.randn((B, w.h, n, w.d), w.torch_dtype, gen)
    k_new = W.randn((B, w.g, n, w.d), w.torch_dtype, gen)
    v_new = W.randn((B, w.g, n, w.d), w.torch_dtype, gen)
    x = W.make_contiguous(w, lengths=before, t_cap=max(T_CAP, max(BEFORE) + n), fill=float("nan"))
    if paged:
        table, nb = W.make_block_table(before + n, block_size, perm_seed=seed + 2, extra_blocks=3)
        kc = W.scatter_to_pool(x["k_cache"], before, table, nb, block_size, fill=float("nan"))
        vc = W.scatter_to_pool(x["v_cache"], before, table, nb, block_size, fill=float("nan"))
    else:
        table, kc, vc = None, x["k_cache"], x["v_cache"]
    return w, before, q, k_new, v_new, kc, vc, table, x["scale"]


def _expected(w, before, q, k_new, v_new, kc, vc, table, scale, block_size):
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before, block_table=table)
    k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, scale, block_table=table,
                                 block_size=block_size)
    n = q.shape[2]
    after = before + n
    if table is None:
        vmax = attended_vmax_contig(v_host, after)
    else:
        vmax = attended_vmax_paged(v_host, table, after, block_size)
    return ek, ev, k_host, v_host, ro, rl, vmax


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_splits", [0, 1, 3, -1])
@pytest.mark.parametrize("paged", [False, True])
def test_append_decode_multi(case, num_splits, paged):
    name, s, n = case
    _log(f"case multi {name} n={n} splits={num_splits} paged={paged}")
    bs = 16
    w, before, q, k_new, v_new, kc, vc, table, scale = _inputs(name, s, n, 900, paged, bs)
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       block_table=dev(table) if paged else None, scale=scale,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev, k_host, v_host, ro, rl, vmax = _expected(w, before, q, k_new, v_new, kc, vc, table,
                                                     scale, bs)
    assert np.array_equal(_raw(kd), _raw_np(ek)) and np.array_equal(_raw(vd), _raw_np(ev)), \
        f"{name}: cache after the multi-token step differs from the oracle's append"
    e = check_parity(out, lse, ro, rl, vmax, name)
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_multi_over_filled_cache(case, paged):
    """The tokens are already in the cache (seq_lens counts them)."""
    name, s, n = case
    _log(f"case decode_multi {name} n={n} paged={paged}")
    bs = 16
    w, before, q, k_new, v_new, kc, vc, table, scale = _inputs(name, s, n, 910, paged, bs)
    ek, ev, k_host, v_host, ro, rl, vmax = _expected(w, before, q, k_new, v_new, kc, vc, table,
                                                     scale, bs)
    out, lse = kvc.decode_multi(dev(q), dev(k_host), dev(v_host), dev(before + n),
                                block_table=dev(table) if paged else None, scale=scale,
                                num_splits=2)
    check_parity(out, lse, ro, rl, vmax, name)


def test_multi_capacity_clamp():
    """Tokens past the capacity are not written and every token sees at most
    the capacity, as kvc_append then single-token decodes would."""
    _log("case multi_clamp")
    w = W.Workload("mc", B=2, h=16, g=2, d=128, dtype="bf16", T=40, seed=920)
    n = 4
    x = W.make_contiguous(w, t_cap=48)
    gen = torch.Generator().manual_seed(921)
    q = W.randn((2, 16, n, 128), w.torch_dtype, gen)
    k_new = W.randn((2, 2, n, 128), w.torch_dtype, gen)
    v_new = W.randn((2, 2, n, 128), w.torch_dtype, gen)
    before = torch.tensor([46, 48], dtype=torch.int32)
    kd, vd = dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       scale=x["scale"])
    torch.cuda.synchronize()
    k_host, v_host = x["k_cache"].clone(), x["v_cache"].clone()
    k_host[0, :, 46:48] = k_new[0, :, :2]
    v_host[0, :, 46:48] = v_new[0, :, :2]
    assert torch.equal(kd.cpu(), k_host) and torch.equal(vd.cpu(), v_host)
    for t in range(n):
        vis = torch.clamp(before + t + 1, max=48)
        ro, rl = oracle.decode(q[:, :, t].contiguous(), k_host, v_host, vis, x["scale"])
        check_parity(out[:, :, t], lse[:, :, t], ro, rl, attended_vmax_contig(v_host, vis),
                     f"clamp t={t}")


@pytest.mark.parametrize("n", [2, 4, 8])
def test_multi_full_size_70b(n):
    """The 70B GQA shape (B=32, h=64, g=8, d=128, 4096 cached positions) with
    n draft tokens per sequence, in the launch the benchmark times."""
    _log(f"case multi_full_70b n={n}")
    w = W.WORKLOADS["gqa_70b_bf16"]
    x = W.make_contiguous(w)
    gen = torch.Generator().manual_seed(930 + n)
    q = W.randn((w.B, w.h, n, w.d), w.torch_dtype, gen)
    k_new = W.randn((w.B, w.g, n, w.d), w.torch_dtype, gen)
    v_new = W.randn((w.B, w.g, n, w.d), w.torch_dtype, gen)
    before = x["seq_lens_before"]
    kd, vd = dev(x["k_cache"]), dev(x["v_cache"])
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       scale=x["scale"])
    torch.cuda.synchronize()
    ek, ev = oracle.append_multi(k_new, v_new, x["k_cache"], x["v_cache"], before)
    assert np.array_equal(_raw(kd), _raw_np(ek)) and np.array_equal(_raw(vd), _raw_np(ev))
    k_host, v_host = _to_torch(ek, x["k_cache"]), _to_torch(ev, x["v_cache"])
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, x["scale"])
    e = check_parity(out, lse, ro, rl, attended_vmax_contig(v_host, before + n), "70b multi")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")
