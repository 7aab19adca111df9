"""GPU parity of the persistent, position-balanced split (automatic
num_splits) on shapes that stress its bookkeeping: ragged and zero lengths
between non-empty ones, segments longer than one block-table window, batches
smaller than the grid, and large batches of short sequences."""
from __future__ import annotations

import sys

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import attended_vmax_contig, attended_vmax_paged, check_parity, dev

pytestmark = pytest.mark.gpu

SHAPES = [("valu_m1", 4, 4), ("valu_m3", 6, 2), ("mfma_m8", 16, 2), ("mfma_m32", 32, 1)]
CASES = {
    "zeros_between": [0, 0, 700, 0, 1, 0, 2500, 0, 0, 33, 0],
    "all_zero": [0, 0, 0],
    "one_long": [20000],
    "tiny": [1, 2],
    "ragged": [129, 8193, 4000, 77, 1, 6000, 3333, 2048, 0, 515],
}


def _lengths(name):
    return torch.tensor(CASES[name], dtype=torch.int32)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("case", list(CASES))
def test_stream_contiguous(shape, case):
    name, h, g = shape
    print(f"case stream_contig {name} {case}", file=sys.stderr, flush=True)
    L = _lengths(case)
    w = W.Workload(name, B=len(L), h=h, g=g, d=128, dtype="bf16", T=0, seed=500)
    x = W.make_contiguous(w, lengths=L, fill=float("nan"))
    assert kvc.plan(w.B, h, g, 128, x["t_cap"], 0)[0] == "stream"
    out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L))
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], L), f"{name}/{case}")


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("case", ["zeros_between", "one_long", "ragged"])
def test_stream_paged(shape, case):
    name, h, g = shape
    print(f"case stream_paged {name} {case}", file=sys.stderr, flush=True)
    L = _lengths(case)
    w = W.Workload(name, B=len(L), h=h, g=g, d=128, dtype="bf16", T=0, paged=True, seed=501)
    x = W.make_paged(w, lengths=L, fill=float("nan"))
    out, lse = kvc.decode_paged(dev(x["q"]), dev(x["k_pool"]), dev(x["v_pool"]),
                                dev(x["block_table"]), dev(L))
    ro, rl = oracle.decode(x["q"], x["k_pool"], x["v_pool"], L, x["scale"],
                           block_table=x["block_table"], block_size=16)
    vmax = attended_vmax_paged(x["v_pool"], x["block_table"], L, 16)
    check_parity(out, lse, ro, rl, vmax, f"{name}/{case}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]], ids=["valu_m1", "mfma_m8"])
def test_stream_large_batch(shape):
    """1024 sequences (the stream-mode limit) of lengths 0..40."""
    name, h, g = shape
    print(f"case stream_large_batch {name}", file=sys.stderr, flush=True)
    gen = torch.Generator().manual_seed(502)
    L = torch.randint(0, 41, (1024,), generator=gen, dtype=torch.int32)
    w = W.Workload(name, B=1024, h=h, g=g, d=128, dtype="bf16", T=0, seed=503)
    x = W.make_contiguous(w, lengths=L, t_cap=48)
    assert kvc.plan(1024, h, g, 128, 48, 0)[0] == "stream"
    out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L))
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], L), f"{name}/large_batch")
