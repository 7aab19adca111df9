"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte accounting against closed forms written out here, the HBM-traffic
summary of rocprofv3 counter CSVs, and the source-hash gate on stored
traffic figures."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import torch

import bench
import kvc_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _closed_form(B, h, g, d, lengths_after, n=1, kv_bytes=2, in_bytes=2, window=0, paged_blocks=0):
    """Bytes of one one-call step, written out term by term."""
    attended = [min(L, window + n - 1) if window else L for L in lengths_after]
    kv = 2 * sum(attended) * g * d * kv_bytes              # K and V over the attended positions
    q = B * h * n * d * in_bytes                            # queries
    out = B * h * n * d * 4 + B * h * n * 4                 # out and lse, float32
    lens = B * 4                                            # seq_lens
    table = paged_blocks * 4                                # block-table entries
    scales = 2 * g * 4 if kv_bytes == 1 else 0              # FP8 head scales
    new_read = 2 * B * g * n * d * (in_bytes - kv_bytes)    # new rows come in bf16
    written = 2 * B * g * n * d * kv_bytes                  # new rows stored
    return kv + q + out + lens + table + scales + new_read + written


def test_algorithmic_bytes_match_the_closed_forms():
    w = W.WORKLOADS["gqa_70b_bf16"]
    L = torch.full((w.B,), w.T + 1, dtype=torch.int64)
    nb = bench.algorithmic_bytes(w, L)
    assert nb["fused"] == _closed_form(w.B, w.h, w.g, w.d, L.tolist()) == 538_714_240
    assert nb["decode"] == 538_714_240 - 2 * w.B * w.g * w.d * 2
    fp8 = bench.algorithmic_bytes(w, L, kv_bytes=1)
    assert fp8["fused"] == _closed_form(w.B, w.h, w.g, w.d, L.tolist(), kv_bytes=1) == 270_213_312
    L4 = torch.full((w.B,), w.T + 4, dtype=torch.int64)
    assert bench.algorithmic_bytes(w, L4, n=4)["fused"] == \
        _closed_form(w.B, w.h, w.g, w.d, L4.tolist(), n=4) == 544_243_840
    Lw = torch.full((w.B,), 1024, dtype=torch.int64)  # a window of 1024 keeps 1024 positions
    assert bench.algorithmic_bytes(w, Lw)["fused"] == \
        _closed_form(w.B, w.h, w.g, w.d, [w.T + 1] * w.B, window=1024) == 135_929_984


def test_algorithmic_bytes_paged_counts_the_table():
    w = W.WORKLOADS["paged_gqa_bf16"]
    lens = W.seq_lengths(w) + 1
    blocks = W.block_counts(lens, w.block_size)
    nb = bench.algorithmic_bytes(w, lens.to(torch.int64), blocks)
    assert nb["fused"] == _closed_form(w.B, w.h, w.g, w.d, lens.tolist(),
                                       paged_blocks=int(blocks.sum()))


def test_paged_inputs_hold_every_new_token():
    """A paged multi-token step (bench.py --queries n on a paged workload):
    each sequence owns blocks for its n new tokens, the slots they land in
    are blank, and the byte accounting counts their blocks and the n
    tokens' reads and writes."""
    w = W.Workload("p", B=5, h=8, g=2, d=16, dtype="bf16", T_range=(0, 70), paged=True, seed=7)
    n = 21
    one = W.make_paged(w)
    x = W.make_paged(w, new_tokens=n, fill=float("nan"))
    lens = x["seq_lens_before"]
    assert torch.equal(lens, one["seq_lens_before"])
    bs = x["block_size"]
    table = x["block_table"]
    owned = (table >= 0).sum(dim=1)
    assert torch.equal(owned, W.block_counts(lens + n, bs))
    assert x["num_blocks"] == int(W.block_counts(lens + n, bs).sum())
    for b in range(w.B):
        L = int(lens[b])
        for p in range(L, L + n):
            slot = x["k_pool"][int(table[b, p // bs]), :, p % bs]
            assert torch.isnan(slot.float()).all(), (b, p)
        if L > 0:
            assert not torch.isnan(x["k_pool"][int(table[b, (L - 1) // bs]), :, (L - 1) % bs].float()).any()
    blocks = W.block_counts(lens + n, bs)
    after = (lens + n).to(torch.int64)
    nb = bench.algorithmic_bytes(w, after, blocks, n=n)
    eb = 2
    expect = (2 * int(after.sum()) * w.g * w.d * eb          # K/V read (new rows from k_new)
              + w.B * w.h * n * w.d * eb                      # queries
              + w.B * w.h * n * (w.d * 4 + 4)                 # out and lse
              + int(blocks.sum()) * 4 + w.B * 4               # block table, lengths
              + 2 * w.B * w.g * n * w.d * eb)                 # the new rows written
    assert nb["fused"] == expect


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        for did, name, kib in rows:
            wr.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": kib})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    mib = 64
    calib_kib = mib * 1024
    decode = "void kvc::decode_mfma_chunked<1, false, 8, false, false>(kvc::DecodeArgs)"
    # the counters read half the copy's bytes for FETCH_SIZE and all of them for WRITE_SIZE
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", calib_kib / 2),
                                                        (2, decode, 1000.0), (3, decode, 1002.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", calib_kib),
                                                        (2, decode, 10.0), (3, decode, 12.0)])
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "unit_test", mib, ["cmd"])
    kv = {}
    for line in open(bench.traffic_file("unit_test")):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert float(kv["fetch_factor"]) == 2.0 and float(kv["write_factor"]) == 1.0
    assert int(kv["fetch_bytes_per_call"]) == round(1001.0 * 1024 * 2)
    assert int(kv["write_bytes_per_call"]) == round(11.0 * 1024)
    assert bench.stored_traffic("unit_test") == int(kv["traffic_bytes_per_call"])
    # a figure taken on other kernel sources is not reported
    text = open(bench.traffic_file("unit_test")).read()
    open(bench.traffic_file("unit_test"), "w").write(
        text.replace(kv["source_sha256"], "0" * 64))
    assert bench.stored_traffic("unit_test") is None


def test_traffic_summary_counts_the_merge_kernels(tmp_path, monkeypatch):
    """A split call's traffic is its decode kernel plus its merge, whether the
    merge is a plain kernel (kvc::merge_stream_kernel) or a template one
    (void kvc::merge128_kernel<G>); other kernels are left out."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    mib = 64
    calib_kib = mib * 1024
    decode = "void kvc::decode_valu_chunked<1, false, 4, false, 0>(kvc::DecodeArgs)"
    merge_t = "void kvc::merge128_kernel<8>(kvc::DecodeArgs)"
    merge_p = "kvc::merge_stream_kernel(kvc::DecodeArgs)"
    other = "void at::native::vectorized_elementwise_kernel<4>(int)"
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                    [(1, "__amd_rocclr_copyBuffer", calib_kib / 2), (2, decode, 1000.0),
                     (3, merge_t, 20.0), (4, merge_p, 6.0), (5, other, 500.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE",
                    [(1, "__amd_rocclr_copyBuffer", calib_kib), (2, decode, 10.0),
                     (3, merge_t, 2.0), (4, merge_p, 1.0), (5, other, 500.0)])
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "unit_merge", mib, ["cmd"])
    kv = {}
    for line in open(bench.traffic_file("unit_merge")):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert int(kv["fetch_bytes_per_call"]) == round((1000.0 + 20.0 + 6.0) * 1024 * 2)
    assert int(kv["write_bytes_per_call"]) == round((10.0 + 2.0 + 1.0) * 1024)
