"""GPU parity of automatic chunking when it picks one wide work-group per
(sequence, KV head): batches with at least as many units as the device has
wide work-group slots.  Ragged lengths (0, 1, tile and window edges, lengths
that need several windows of a single chunk), NaN in unwritten slots, and
needles at window boundaries; each case is checked against the oracle."""
from __future__ import annotations

import sys

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import attended_vmax_contig, check_parity, dev, plant_needles_contig

pytestmark = pytest.mark.gpu

# (id, shape, batch): units = B * g fill a 256-CU device's wide slots once
# (256 units each).  The VALU kernels (m <= 3) have no wide kernel with equal
# residency and stay on 4-wavefront chunks: parity must hold either way.
CASES = [
    ("valu_m1", dict(h=32, g=32, d=128, dtype="bf16"), 8),
    ("valu_m2", dict(h=8, g=4, d=128, dtype="bf16"), 64),
    ("mfma_m8_w8", dict(h=64, g=8, d=128, dtype="bf16"), 32),
    ("mfma_m4_w8", dict(h=16, g=4, d=128, dtype="bf16"), 64),
    ("mfma_m32_w8", dict(h=64, g=2, d=128, dtype="bf16"), 128),
]
EDGES = [0, 1, 31, 32, 33, 4095, 4096, 4097, 8193, 9000, 2, 257]


def _lengths(B: int, seed: int) -> torch.Tensor:
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, 2048, (B,), generator=gen, dtype=torch.int32)
    lens[: min(B, len(EDGES))] = torch.tensor(EDGES[:B], dtype=torch.int32)
    return lens


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_wide_auto_chunks(case):
    name, s, B = case
    print(f"case wide {name} B={B}", file=sys.stderr, flush=True)
    w = W.Workload(name, B=B, seed=700, **s)
    lengths = _lengths(B, 701)
    x = W.make_contiguous(w, lengths=lengths, fill=float("nan"))
    t_cap = x["t_cap"]
    waves, wgs, cl, nc = kvc.launch_shape(B, w.h, w.g, w.d, t_cap, 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"  waves={waves} wgs={wgs} chunk_len={cl} chunks={nc} cus={cus}", file=sys.stderr, flush=True)
    if name.endswith(("_w8", "_w16")) and cus == 256:
        assert waves == int(name.rsplit("_w", 1)[1]) and nc == 1 and cl >= t_cap
    if waves > 4:
        assert nc == 1
    # Needles on window edges (and 0 / last) so that a dropped or repeated
    # window moves the output by about |V|.
    special = [0, 4095, 4096, 4097, 8191, 8192]
    pos = [[min(special[(b + j) % len(special)], max(int(lengths[b]) - 1, 0)) for j in range(w.g)]
           for b in range(B)]
    keep = lengths > 0
    xs = dict(x)
    plant_needles_contig(xs, pos)
    # planting writes position 0 of empty sequences too: restore their NaN slots
    xs["k_cache"][~keep] = float("nan")
    ws = torch.empty(max(1, kvc.workspace_bytes(B, w.h, w.g, w.d, t_cap, 0)), dtype=torch.uint8,
                     device="cuda")
    out, lse = kvc.decode(dev(xs["q"]), dev(xs["k_cache"]), dev(xs["v_cache"]), dev(lengths),
                          scale=xs["scale"], num_splits=0, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(xs["q"], xs["k_cache"], xs["v_cache"], lengths, xs["scale"])
    e = check_parity(out, lse, ro, rl, attended_vmax_contig(xs["v_cache"], lengths), name)
    print(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}", file=sys.stderr, flush=True)
    # the same inputs through explicit chunks agree to the same bar
    out2, lse2 = kvc.decode(dev(xs["q"]), dev(xs["k_cache"]), dev(xs["v_cache"]), dev(lengths),
                            scale=xs["scale"], num_splits=3)
    check_parity(out2, lse2, ro, rl, attended_vmax_contig(xs["v_cache"], lengths), name + "/3")


@pytest.mark.parametrize("kv8", [False, True], ids=["bf16", "fp8"])
def test_fixed_chunks_two_tiles_wide(kv8):
    """32 query rows per KV head (long-context MQA shape) with a fixed grid of
    64 chunks per sequence that the device holds at once: 8-wavefront
    work-groups (on 256 CUs), each chunk split over eight wavefronts; needles
    at chunk edges; parity with the oracle for bf16 and FP8 caches."""
    print(f"case fixed_chunks_wide kv8={kv8}", file=sys.stderr, flush=True)
    B, h, g, d, ns = 4, 32, 1, 128, 64
    w = W.Workload("mqa_wide", B=B, h=h, g=g, d=d, dtype="bf16", seed=710)
    lengths = torch.tensor([20000, 1, 12345, 19968], dtype=torch.int32)
    x = W.make_contiguous(w, lengths=lengths, t_cap=20016, fill=float("nan"))
    waves, wgs, cl, nc = kvc.launch_shape(B, h, g, d, 20016, ns)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"  waves={waves} wgs={wgs} chunk_len={cl} chunks={nc}", file=sys.stderr, flush=True)
    if cus == 256:  # about 64 chunks of a multiple of 32 positions, all resident at once
        assert waves == 8 and abs(nc - ns) <= 1
    pos = [[min(p, int(lengths[b]) - 1)] for b, p in enumerate([cl - 1, 0, 5 * cl, 63 * cl])]
    xs = dict(x)
    plant_needles_contig(xs, pos)
    if not kv8:
        out, lse = kvc.decode(dev(xs["q"]), dev(xs["k_cache"]), dev(xs["v_cache"]), dev(lengths),
                              scale=xs["scale"], num_splits=ns)
        ro, rl = oracle.decode(xs["q"], xs["k_cache"], xs["v_cache"], lengths, xs["scale"])
        vmax = attended_vmax_contig(xs["v_cache"], lengths)
    else:
        gen = torch.Generator().manual_seed(711)
        ks = (torch.rand(g, generator=gen) * 0.05 + 0.01).to(torch.float32)
        vs = (torch.rand(g, generator=gen) * 0.05 + 0.01).to(torch.float32)
        kc = torch.from_numpy(oracle.quantize_fp8(xs["k_cache"], ks.numpy(), 1))
        vc = torch.from_numpy(oracle.quantize_fp8(xs["v_cache"], vs.numpy(), 1))
        out, lse = kvc.decode_fp8(dev(xs["q"]), dev(kc), dev(vc), dev(ks), dev(vs), dev(lengths),
                                  scale=xs["scale"], num_splits=ns)
        ro, rl = oracle.decode_fp8(xs["q"], kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(),
                                   lengths, xs["scale"])
        vals = torch.from_numpy(oracle.e4m3_values())
        vmax = max(float((vals[vc[b, :, :int(lengths[b])].long()] * float(vs[0])).abs().max())
                   for b in range(B))
    e = check_parity(out, lse, ro, rl, vmax, f"fixed chunks kv8={kv8}")
    print(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}", file=sys.stderr, flush=True)
