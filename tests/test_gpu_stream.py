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
    assert kvc.plan(w.B, h, g, 128, x["t_cap"], kvc.SPLITS_STREAM)[0] == "stream"
    out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L),
                          num_splits=kvc.SPLITS_STREAM)
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
    assert kvc.plan(1024, h, g, 128, 48, kvc.SPLITS_STREAM)[0] == "stream"
    out, lse = kvc.decode(dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L),
                          num_splits=kvc.SPLITS_STREAM)
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], L), f"{name}/large_batch")



LARGE_SHAPES = [("valu_m1_wide", 8, 8, 64), ("mfma_m8_wide", 16, 2, 64), ("mfma_m4_wide", 32, 8, 48)]


@pytest.mark.parametrize("shape", LARGE_SHAPES, ids=[s[0] for s in LARGE_SHAPES])
@pytest.mark.parametrize("paged", [False, True])
def test_stream_repeated_calls_one_workspace(shape, paged):
    """Batches where each (sequence, KV head) spans few work-groups; ragged
    lengths with zeros; five stream-mode calls on one workspace give the
    oracle's result and identical bits every time."""
    name, h, g, B = shape
    print(f"case stream_repeat {name} paged={paged}", file=sys.stderr, flush=True)
    gen = torch.Generator().manual_seed(504)
    L = torch.randint(1, 3000, (B,), generator=gen, dtype=torch.int32)
    L[::7] = 0
    w = W.Workload(name, B=B, h=h, g=g, d=128, dtype="bf16", T=0, paged=paged, seed=505)
    if paged:
        x = W.make_paged(w, lengths=L, fill=float("nan"))
        kc, vc, bt = dev(x["k_pool"]), dev(x["v_pool"]), dev(x["block_table"])
        max_len = x["block_table"].shape[1] * 16
        ro, rl = oracle.decode(x["q"], x["k_pool"], x["v_pool"], L, x["scale"],
                               block_table=x["block_table"], block_size=16)
        vmax = attended_vmax_paged(x["v_pool"], x["block_table"], L, 16)
    else:
        x = W.make_contiguous(w, lengths=L, fill=float("nan"))
        kc, vc, bt = dev(x["k_cache"]), dev(x["v_cache"]), None
        max_len = x["t_cap"]
        ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
        vmax = attended_vmax_contig(x["v_cache"], L)
    ns = kvc.SPLITS_STREAM
    assert kvc.plan(B, h, g, 128, max_len, ns, paged=paged)[0] == "stream"
    ws = torch.empty(kvc.workspace_bytes(B, h, g, 128, max_len, ns, paged=paged), dtype=torch.uint8,
                     device="cuda")
    q, sl = dev(x["q"]), dev(L)
    first = None
    for call in range(5):
        if paged:
            out, lse = kvc.decode_paged(q, kc, vc, bt, sl, num_splits=ns, workspace=ws)
        else:
            out, lse = kvc.decode(q, kc, vc, sl, num_splits=ns, workspace=ws)
        check_parity(out, lse, ro, rl, vmax, f"{name}/call{call}")
        if first is None:
            first = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1]), f"call {call}"


def test_launch_planning_from_many_threads():
    """The library caches occupancy queries per process; planning the same
    launches from eight host threads at once gives every thread the shapes a
    single thread gets (ctypes releases the GIL during the calls)."""
    import threading
    cases = [(32, 64, 8, 128, 4096, 0, "bf16", False), (64, 32, 8, 128, 8192, 0, "bf16", True),
             (4, 32, 1, 128, 131072, 64, "bf16", False), (8, 32, 32, 128, 2048, 0, "bf16", False),
             (32, 64, 8, 128, 4096, 0, "fp8", False), (64, 32, 8, 128, 8192, 0, "fp8", True),
             (32, 512, 8, 128, 4096, 0, "bf16", False), (8, 8, 2, 64, 1000, 0, "f32", False)]
    results, errors = {}, []

    def work(tid):
        try:
            for r in range(20):
                for k, c in enumerate(cases):
                    B, h, g, d, L, ns, dt, paged = c
                    results[(tid, r, k)] = kvc.launch_shape(B, h, g, d, L, ns, dtype=dt, paged=paged)
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k, c in enumerate(cases):
        B, h, g, d, L, ns, dt, paged = c
        want = kvc.launch_shape(B, h, g, d, L, ns, dtype=dt, paged=paged)
        assert want[1] > 1 or B * g == 1, (c, want)
        got = {results[(t, r, k)] for t in range(8) for r in range(20)}
        assert got == {want}, (c, got, want)


@pytest.mark.parametrize("handle", [False, True], ids=["stream_object", "raw_handle"])
def test_explicit_side_stream_owns_its_allocations(handle):
    """stream= names a side stream (a torch stream, or its raw HIP handle):
    the outputs and the split plan's workspace are allocated for that
    stream, so work the default stream queues meanwhile (allocations and
    writes) cannot reuse their memory while the call still runs."""
    print(f"case side_stream handle={handle}", file=sys.stderr, flush=True)
    gen = torch.Generator().manual_seed(506)
    L = torch.randint(1, 6000, (6,), generator=gen, dtype=torch.int32)
    w = W.Workload("side", B=6, h=16, g=2, d=128, dtype="bf16", T=0, seed=507)
    x = W.make_contiguous(w, lengths=L)
    q, kc, vc, sl = dev(x["q"]), dev(x["k_cache"]), dev(x["v_cache"]), dev(L)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    results = []
    for rep in range(3):
        out, lse = kvc.decode(q, kc, vc, sl, num_splits=5,
                              stream=s.cuda_stream if handle else s)
        # the default stream allocates and fills memory while the side stream runs
        junk = [torch.full((1 << 20,), float(rep + 1), device="cuda") for _ in range(8)]
        del junk
        s.synchronize()
        results.append((out.clone(), lse.clone()))
        assert out.device.index == torch.cuda.current_device()
    ro, rl = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    for out, lse in results:
        check_parity(out, lse, ro, rl, attended_vmax_contig(x["v_cache"], L), "side stream")
        assert torch.equal(out, results[0][0]) and torch.equal(lse, results[0][1])
