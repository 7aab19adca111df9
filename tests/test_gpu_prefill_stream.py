"""GPU parity of the multi-row kernel's stream grid: paged pools whose unit
rows fit one 4-wavefront work-group (head dims 64 and 256 at any row count
up to 64, and more than 32 rows per KV head at d = 128 up to 128) lay every
(sequence, KV head) end to end and give each persistent work-group an equal
share of positions, so a work-group may hold several whole units (final
rows) and parts of two more (record slots combined by the stream merge).
The automatic plan takes this grid for bf16 at d = 256 with at most 16 rows
per KV head; the other shapes ask for it (KVC_SPLITS_STREAM).

Batches mix many short sequences (0 to 90 positions, so that work-groups
cover many segments) with a few long ones (units spread over many
work-groups); unwritten slots hold NaN.  Appends of one and several new
tokens, sliding windows under an explicit stream split, and FP8 caches
with per-KV-head scales; every output row against the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import attended_vmax_paged, check_parity, dev

pytestmark = pytest.mark.gpu

BS = 16
NAN_CODE = 0x7F


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _lengths(seed: int, B: int = 40, long=(2000, 5000)) -> torch.Tensor:
    gen = torch.Generator().manual_seed(seed)
    short = torch.randint(0, 91, (B - len(long),), generator=gen, dtype=torch.int64)
    lens = torch.cat([short, torch.tensor(long, dtype=torch.int64)])
    perm = torch.randperm(B, generator=gen)
    return lens[perm].to(torch.int32)


def _raw(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _to_torch(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)


# (id, h, g, n, d): rows per KV head (h / g) * n
SHAPES = [
    ("d64_rows4", 8, 2, 1, 64),
    ("d64_rows64_n16", 8, 2, 16, 64),
    ("d256_rows4", 8, 2, 1, 256),
    ("d256_rows48_n12", 8, 2, 12, 256),
    ("d128_rows40_n20", 4, 2, 20, 128),
    ("d128_rows96_n24", 8, 2, 24, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("num_splits", [0, kvc.SPLITS_STREAM])
def test_stream_multi_row_paged(shape, num_splits):
    name, h, g, n, d = shape
    auto = d == 256 and (h // g) * n <= 16
    if num_splits == 0 and not auto:
        pytest.skip("the automatic plan chunks this shape (covered by the other suites)")
    assert kvc.plan(8, h * n, g, d, 4096, num_splits, paged=True)[0] == "stream", name
    _log(f"case prefill_stream {name} splits={num_splits}")
    seed = 2100 + d + n
    before = _lengths(seed)
    B = len(before)
    w = W.Workload("ps", B=B, h=h, g=g, d=d, dtype="bf16", seed=seed)
    gen = torch.Generator().manual_seed(seed + 1)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    x = W.make_contiguous(w, lengths=before, t_cap=int(before.max()) + n + 3, fill=float("nan"))
    table, nb = W.make_block_table(before + n, BS, perm_seed=seed + 2, extra_blocks=2)
    kc = W.scatter_to_pool(x["k_cache"], before, table, nb, BS, fill=float("nan"))
    vc = W.scatter_to_pool(x["v_cache"], before, table, nb, BS, fill=float("nan"))
    kd, vd = dev(kc), dev(vc)
    out, lse = kvc.append_decode_multi(dev(q), dev(k_new), dev(v_new), kd, vd, dev(before),
                                       block_table=dev(table), scale=w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    ek, ev = oracle.append_multi(k_new, v_new, kc, vc, before, block_table=table)
    assert np.array_equal(_raw(kd), ek) and np.array_equal(_raw(vd), ev), f"{name}: pool"
    k_host, v_host = _to_torch(ek), _to_torch(ev)
    ro, rl = oracle.decode_multi(q, k_host, v_host, before, w.scale, block_table=table,
                                 block_size=BS)
    vmax = attended_vmax_paged(v_host, table, before + n, BS)
    e = check_parity(out, lse, ro, rl, vmax, f"stream {name}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("window,n", [(1, 1), (50, 3)])
def test_stream_multi_row_paged_window(d, window, n):
    """A sliding window under an explicit stream split: each unit's range
    starts at its window's first position."""
    h, g = 4, 2
    _log(f"case prefill_stream_window d={d} W={window} n={n}")
    seed = 2200 + d + window
    before = _lengths(seed, B=24, long=(900, 1700))
    B = len(before)
    gen = torch.Generator().manual_seed(seed)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    v_new = W.randn((B, g, n, d), torch.bfloat16, gen)
    t_cap = int(before.max()) + n + 3
    k = W.randn((B, g, t_cap, d), torch.bfloat16, gen)
    v = W.randn((B, g, t_cap, d), torch.bfloat16, gen)
    pos = torch.arange(t_cap).view(1, 1, t_cap, 1)
    unwritten = pos >= before.view(-1, 1, 1, 1).to(torch.int64)
    k.masked_fill_(unwritten, float("nan"))
    v.masked_fill_(unwritten, float("nan"))
    table, nb = W.make_block_table(before + n, BS, perm_seed=seed + 1, extra_blocks=2)
    kp = W.scatter_to_pool(k, before, table, nb, BS, fill=float("nan"))
    vp = W.scatter_to_pool(v, before, table, nb, BS, fill=float("nan"))
    kd, vd = dev(kp), dev(vp)
    out, lse = kvc.decode_window(dev(q), kd, vd, dev(before), window, block_table=dev(table),
                                 k_new=dev(k_new), v_new=dev(v_new), num_splits=kvc.SPLITS_STREAM)
    torch.cuda.synchronize()
    ek, ev = oracle.append_window(k_new, v_new, kp, vp, before, block_table=table)
    assert np.array_equal(_raw(kd), ek.view(np.uint16)) and np.array_equal(_raw(vd), ev.view(np.uint16))
    k_host, v_host = _to_torch(ek), _to_torch(ev)
    ro, rl = oracle.decode_window(q, k_host, v_host, before, d ** -0.5, window, block_table=table)
    vmax = attended_vmax_paged(v_host, table, before + n, BS)
    e = check_parity(out, lse, ro, rl, vmax, f"stream window d={d}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2], SHAPES[4], SHAPES[5]],
                         ids=[SHAPES[i][0] for i in (0, 2, 4, 5)])
def test_stream_multi_row_paged_fp8(shape):
    """FP8 codes with a scale per KV head on the stream grid: the appended
    tokens' codes bit-exact, attention against the dequantise-then-exact
    reference."""
    name, h, g, n, d = shape
    _log(f"case prefill_stream_fp8 {name}")
    seed = 2300 + d + n
    before = _lengths(seed)
    B = len(before)
    gen = torch.Generator().manual_seed(seed)
    ks = (torch.rand(g, generator=gen) * 0.4 + 0.02).to(torch.float32)
    vs = (torch.rand(g, generator=gen) * 0.4 + 0.02).to(torch.float32)
    q = W.randn((B, h, n, d), torch.bfloat16, gen)
    k_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    v_new = (W.randn((B, g, n, d), torch.float32, gen) * 3).to(torch.bfloat16)
    t_cap = int(before.max()) + n + 3
    kc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (B, g, t_cap, d), generator=gen, dtype=torch.int32).to(torch.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    pos = torch.arange(t_cap).view(1, 1, t_cap, 1)
    unwritten = pos.expand(B, g, t_cap, d) >= before.view(-1, 1, 1, 1)
    kc[unwritten] = NAN_CODE
    vc[unwritten] = NAN_CODE
    table, nb = W.make_block_table(before + n, BS, perm_seed=seed + 1, extra_blocks=2)
    kc = W.scatter_to_pool(kc, before, table, nb, BS, fill=NAN_CODE)
    vc = W.scatter_to_pool(vc, before, table, nb, BS, fill=NAN_CODE)
    kd, vd = dev(kc), dev(vc)
    assert kvc.plan(8, h * n, g, d, 4096, kvc.SPLITS_STREAM, dtype=kvc.FP8_E4M3,
                    paged=True)[0] == "stream", name
    out, lse = kvc.decode_fp8_window(dev(q), kd, vd, dev(ks), dev(vs), dev(before), window=0,
                                     block_table=dev(table), num_splits=kvc.SPLITS_STREAM,
                                     k_new=dev(k_new), v_new=dev(v_new))
    torch.cuda.synchronize()
    ek, ev = oracle.append_fp8(k_new, v_new, kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(), before,
                               block_table=table)
    assert np.array_equal(kd.cpu().numpy(), ek) and np.array_equal(vd.cpu().numpy(), ev), \
        f"{name}: codes after the step differ from the oracle's quantising append"
    ro, rl = oracle.decode_fp8_window(q, ek, ev, ks.numpy(), vs.numpy(), before, d ** -0.5, 0,
                                      block_table=table)
    vals = torch.from_numpy(oracle.e4m3_values())
    evt = torch.from_numpy(ev)
    vmax = 0.0
    for b in range(B):
        for p in range(int(before[b]) + n):
            row = evt[int(table[b, p // BS]), :, p % BS]
            vmax = max(vmax, float((vals[row.long()] * vs.double().view(-1, 1)).abs().max()))
    e = check_parity(out, lse, ro, rl, vmax, f"stream fp8 {name}")
    _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")
