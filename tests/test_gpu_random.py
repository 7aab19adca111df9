"""Seeded random sweep of the boundary against the oracle: every case draws
its own shape (batch, query and KV heads, head size, dtype), lengths (with
zeros and ones), layout (contiguous capacity or page size), split request
and, per mode, new tokens or window, then checks one call through the C ABI
(out, lse, and the cache bytes where the call appends).  The case list is
fixed by the seeds; a failure names its mode, seed and shape."""
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

MODES = ["decode", "append_decode", "multi", "window", "fp8"]
CASES_PER_MODE = 40


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.view(torch.int32).numpy().view(np.uint32)


def _bits(a: np.ndarray) -> np.ndarray:
    """The oracle's cache arrays as raw bits (bf16 arrays already are)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _to_torch(a: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    if like.dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def _vmax(v, table, lengths, bs) -> float:
    """max |V| over the attended entries (1 when nothing is attended)."""
    if int(lengths.max()) == 0:
        return 1.0
    if table is None:
        return attended_vmax_contig(v, lengths)
    return attended_vmax_paged(v, table, lengths, bs)


DIMS = [16, 32, 64, 96, 128, 256]
# the second sweep: head dims of every kernel family (80 and 96 on the
# multi-row kernel with bf16, 112 and the fp32 ones on the generic kernel)
DIMS_WIDE = [16, 32, 64, 80, 96, 112, 128, 256]
CASES_PER_MODE_WIDE = 20


def _draw(mode: str, seed: int, dims=DIMS) -> dict:
    r = np.random.default_rng(seed)
    fp8 = mode == "fp8"
    dtype = "bf16" if fp8 or r.random() < 0.75 else "f32"
    d = 128 if (dtype == "bf16" and r.random() < 0.7) else int(r.choice(dims))
    g = int(r.choice([1, 2, 4, 8]))
    m = int(r.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 40]))
    n = 1
    if mode in ("multi", "window"):
        n = int(r.choice([1, 2, 3, 5, 8, 17, 40]))
    B = int(r.integers(1, 7))
    lengths = r.integers(0, 2600, size=B)
    lengths[r.random(B) < 0.15] = 0
    lengths[r.random(B) < 0.15] = 1
    paged = bool(r.random() < 0.5)
    bs = int(r.choice([8, 16, 32, 64])) if paged else 16
    splits = int(r.choice([0, 0, -1, 1, 2, 5]))
    window = int(r.integers(1, 700)) if mode == "window" else 0
    return dict(dtype=dtype, d=d, g=g, h=g * m, n=n, B=B, lengths=lengths.astype(np.int32),
                paged=paged, bs=bs, splits=splits, window=window, pad=int(r.integers(0, 40)))


def _cases():
    out = []
    for mi, mode in enumerate(MODES):
        for k in range(CASES_PER_MODE):
            out.append((mode, 9000 + 100 * mi + k))
        for k in range(CASES_PER_MODE_WIDE):  # seeds 19000.. draw from DIMS_WIDE
            out.append((mode, 19000 + 100 * mi + k))
    return out


@pytest.mark.parametrize("mode,seed", _cases(), ids=[f"{m}-{s}" for m, s in _cases()])
def test_random_case(mode, seed):
    c = _draw(mode, seed, DIMS_WIDE if seed >= 19000 else DIMS)
    _log(f"case random {mode} seed={seed} {dict((k, v) for k, v in c.items() if k != 'lengths')} "
         f"lengths={c['lengths'].tolist()}")
    B, h, g, d, n, bs = c["B"], c["h"], c["g"], c["d"], c["n"], c["bs"]
    before = torch.from_numpy(c["lengths"])
    t_cap = int(before.max()) + n + c["pad"] + 1
    w = W.Workload(f"rand{seed}", B=B, h=h, g=g, d=d, dtype=c["dtype"], seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    scale = d ** -0.5
    if mode == "fp8":
        kc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
        vc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
        kc[(kc & 0x7F) == 0x7F] = 0x3C
        vc[(vc & 0x7F) == 0x7F] = 0x3C
        ks = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
        vs = (torch.rand(g, generator=gen) * 0.5 + 0.01).to(torch.float32)
        q = W.randn((B, h, d), torch.bfloat16, gen)
        table = None
        if c["paged"]:
            table, nb = W.make_block_table(before, bs, perm_seed=seed + 2, extra_blocks=2)
            kc = W.scatter_to_pool(kc, before, table, nb, bs, fill=0x7F)
            vc = W.scatter_to_pool(vc, before, table, nb, bs, fill=0x7F)
        out, lse = kvc.decode_fp8(dev(q), dev(kc), dev(vc), dev(ks), dev(vs), dev(before),
                                  block_table=dev(table) if table is not None else None,
                                  scale=scale, num_splits=c["splits"])
        ro, rl = oracle.decode_fp8(q, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), before, scale,
                                   block_table=table, block_size=bs)
        vals = torch.from_numpy(oracle.e4m3_values())
        deq = vals[vc.long()] * vs.double().view(1, -1, 1, 1)  # the pools' fill codes are NaN
        fin = deq[torch.isfinite(deq)]
        vmax = float(fin.abs().max()) if fin.numel() else 1.0
        check_parity(out, lse, ro, rl, vmax, f"{mode} seed {seed}")
        return

    x = W.make_contiguous(w, lengths=before, t_cap=t_cap, fill=0.0)
    kc, vc = x["k_cache"], x["v_cache"]
    table = None
    if c["paged"]:
        table, nb = W.make_block_table(before + n, bs, perm_seed=seed + 2, extra_blocks=2)
        kc = W.scatter_to_pool(kc, before, table, nb, bs, fill=0.0)
        vc = W.scatter_to_pool(vc, before, table, nb, bs, fill=0.0)
    kd, vd = dev(kc), dev(vc)
    bt = dev(table) if table is not None else None
    if mode == "decode":
        q = x["q"]
        if table is None:
            out, lse = kvc.decode(dev(q), kd, vd, dev(before), scale=scale, num_splits=c["splits"])
        else:
            out, lse = kvc.decode_paged(dev(q), kd, vd, bt, dev(before), scale=scale,
                                        num_splits=c["splits"])
        ro, rl = oracle.decode(q, kc, vc, before, scale, block_table=table, block_size=bs)
        check_parity(out, lse, ro, rl, _vmax(vc, table, before, bs), f"{mode} seed {seed}")
        return

    q = W.randn((B, h, n, d), w.torch_dtype, gen)
    k_new = W.randn((B, g, n, d), w.torch_dtype, gen)
    v_new = W.randn((B, g, n, d), w.torch_dtype, gen)
    if mode == "append_decode":
        out, lse = kvc.append_decode(dev(q[:, :, 0]), dev(k_new[:, :, 0]), dev(v_new[:, :, 0]), kd,
                                     vd, dev(before), block_table=bt, scale=scale,
                                     num_splits=c["splits"])
        ek, ev = oracle.append(k_new[:, :, 0], v_new[:, :, 0], kc, vc, before, block_table=table,
                               block_size=bs)
        out, lse = out.unsqueeze(2), lse.unsqueeze(2)
    elif mode == "multi":
        out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                           block_table=bt, scale=scale, num_splits=c["splits"])
        ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before, block_table=table)
    else:
        out, lse = kvc.decode_window(dev(q), kd, vd, dev(before), c["window"], block_table=bt,
                                     scale=scale, num_splits=c["splits"], k_new=dev(k_new),
                                     v_new=dev(v_new))
        ek, ev = oracle.append_window(k_new, v_new, kc, vc, before, block_table=table)
    torch.cuda.synchronize()
    assert np.array_equal(_raw(kd), _bits(ek)) and np.array_equal(_raw(vd), _bits(ev)), \
        f"{mode} seed {seed}: cache bytes differ from the oracle's append"
    k_host, v_host = _to_torch(ek, kc), _to_torch(ev, vc)
    if mode == "window":
        ro, rl = oracle.decode_window(q, k_host, v_host, before, scale, c["window"],
                                      block_table=table, block_size=bs)
    else:
        ro, rl = oracle.decode_multi(q, k_host, v_host, before, scale, block_table=table,
                                     block_size=bs)
    check_parity(out, lse, ro, rl, _vmax(v_host, table, before + n, bs), f"{mode} seed {seed}")
