"""A decode step captured in a HIP graph (as the benchmark replays it) gives,
on every replay, exactly the result of the same calls launched eagerly."""
from __future__ import annotations

import sys

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("h,g,paged,splits", [(16, 2, False, 5), (4, 4, False, 3), (32, 8, True, 4),
                                              (32, 1, False, 64), (64, 8, False, 0),
                                              (32, 8, True, 0)])
def test_graph_replay_matches_eager(h, g, paged, splits, fused):
    print(f"case graph h={h} g={g} paged={paged} splits={splits} fused={fused}", file=sys.stderr,
          flush=True)
    w = W.Workload("gr", B=3, h=h, g=g, d=128, dtype="bf16", T_range=(100, 900), paged=paged,
                   seed=400)
    dev = torch.device("cuda:0")
    if paged:
        x = W.make_paged(w)
        kc, vc = x["k_pool"].to(dev), x["v_pool"].to(dev)
        bt = x["block_table"].to(dev)
    else:
        x = W.make_contiguous(w)
        kc, vc = x["k_cache"].to(dev), x["v_cache"].to(dev)
        bt = None
    q, kn, vn = x["q"].to(dev), x["k_new"].to(dev), x["v_new"].to(dev)
    before, after = x["seq_lens_before"].to(dev), x["seq_lens_after"].to(dev)
    max_len = bt.shape[1] * 16 if paged else kc.shape[2]
    ws = torch.empty(max(1, kvc.workspace_bytes(w.B, h, g, 128, max_len, splits, paged=paged)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(w.B, h, 128, device=dev)
    lse = torch.empty(w.B, h, device=dev)

    def step():
        if fused:
            kvc.append_decode(q, kn, vn, kc, vc, before, block_table=bt, num_splits=splits,
                              workspace=ws, out=out, lse=lse)
            return
        kvc.append(kn, vn, kc, vc, before, block_table=bt)
        if paged:
            kvc.decode_paged(q, kc, vc, bt, after, num_splits=splits, workspace=ws, out=out, lse=lse)
        else:
            kvc.decode(q, kc, vc, after, num_splits=splits, workspace=ws, out=out, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    ref_k = kc.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {rep}"
        assert torch.equal(kc, ref_k), f"replay {rep}: cache"
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"eager after replay {rep}"
