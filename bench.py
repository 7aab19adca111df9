#!/usr/bin/env python3
"""Benchmark of one decode step on one MI355X.

A step is the whole hot path over one batch of synthetic, seeded input that
is already resident in HBM: one kvc_append_decode_attention[_paged] call
(the new token's K/V into the cache, GQA head map, scores, online softmax,
PV, and the log-sum-exp merge of split partials when the plan splits).
--separate times kvc_append followed by kvc_decode_attention[_paged]
instead.  --kv-fp8 keeps the cache as FP8 E4M3 codes with per-KV-head
scales (kvc_append_decode_attention_fp8[_paged]).

Metric: decode tokens/s = B / step time (one new token per sequence), with
the achieved HBM bandwidth of the decode kernel against the 8 TB/s peak.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload gqa_70b_bf16]

Prints one JSON line.  The KV caches rotate over enough copies (>= 3 and
>= 800 MB in total, at most 64) that the 256 MB Infinity Cache cannot serve
a repeat; the tiny workload's caches stay partly cache-resident.
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """sha256 over the library's kernel and ABI sources: a stored traffic
    figure is valid only for the sources it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_gqa_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    files.append(os.path.join(ROOT, "include", "kvc.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload: str) -> str:
    """Stored counter figure of a workload; an FP8-cache run of workload X is
    stored under the key X + "_kvfp8"."""
    return os.path.join(PROFILES, f"decode_{workload}_hbm_traffic.txt")


def _is_decode_call_kernel(name: str) -> bool:
    """The kernels of one decode call: the decode kernel (or the multi-row
    kernel) and its merge (a plain or a template kernel name)."""
    return name.startswith(("void kvc::decode_", "void kvc::prefill_", "kvc::merge",
                            "void kvc::merge"))


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, calib_mib: int, commands):
    """Turn two rocprofv3 --pmc runs of `bench.py --eager --calibration-copy-mib N`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into the stored HBM
    traffic of one decode call.  The counters are scaled by what they read
    for the calibration copy (a plain device-to-device copy of N MiB: N MiB
    read and N MiB written)."""
    def load(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        return {int(r["Dispatch_Id"]): (r["Kernel_Name"], float(r["Counter_Value"])) for r in rows}
    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    calib = calib_mib * 2**20
    copies = [d for d, (n, v) in write.items()
              if "copyBuffer" in n and abs(v * 1024 - calib) <= 0.02 * calib]
    if len(copies) != 1 or copies[0] not in fetch or "copyBuffer" not in fetch[copies[0]][0]:
        raise SystemExit(f"calibration copy of {calib} bytes not found exactly once in both runs")
    c = copies[0]
    fetch_factor = calib / (fetch[c][1] * 1024)
    write_factor = calib / (write[c][1] * 1024)
    per = {}
    for tab, key in ((fetch, "fetch"), (write, "write")):
        for d, (n, v) in tab.items():
            if _is_decode_call_kernel(n):
                e = per.setdefault(n, {"fetch": [], "write": []})
                e[key].append(v)
    decode_names = [n for n in per if n.startswith(("void kvc::decode_", "void kvc::prefill_"))]
    if len(decode_names) != 1:
        raise SystemExit(f"expected one decode kernel, found {decode_names}")
    calls = len(per[decode_names[0]]["fetch"])
    fetch_b = sum(sum(e["fetch"]) for e in per.values()) * 1024 * fetch_factor / calls
    write_b = sum(sum(e["write"]) for e in per.values()) * 1024 * write_factor / calls
    lines = [f"# HBM traffic of one decode call, workload {workload}",
             "# rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by the same",
             "# counters over a plain device-to-device copy of known size.",
             "# commands (from the repository root):"]
    lines += [f"#   {cmd}" for cmd in commands]
    for n, e in sorted(per.items()):
        lines.append(f"# kernel {n}: {len(e['fetch'])} dispatches, FETCH_SIZE avg "
                     f"{sum(e['fetch']) / max(len(e['fetch']), 1):.1f} KiB, WRITE_SIZE avg "
                     f"{sum(e['write']) / max(len(e['write']), 1):.1f} KiB")
    lines += [f"calibration_copy_bytes: {calib}",
              f"calibration_fetch_kib: {fetch[c][1]:.1f}",
              f"calibration_write_kib: {write[c][1]:.1f}",
              f"fetch_factor: {fetch_factor:.4f}",
              f"write_factor: {write_factor:.4f}",
              f"decode_call_kernels: {'; '.join(sorted(per))}",
              f"fetch_bytes_per_call: {fetch_b:.0f}",
              f"write_bytes_per_call: {write_b:.0f}",
              f"traffic_bytes_per_call: {fetch_b + write_b:.0f}",
              f"source_sha256: {kernel_source_hash()}"]
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stored_traffic(workload: str):
    """HBM bytes per decode call from the stored counter runs, or None when
    there are none or the kernel sources changed since they were taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    return int(kv["traffic_bytes_per_call"])


def algorithmic_bytes(w, attended, nblocks=None, n=1, kv_bytes=None, block_scales=False):
    """Bytes one step must move: KV read (``attended`` positions per
    sequence: all of them, or those a sliding window keeps), q read, out and
    lse written (float32), the appended K/V written, and the block table read
    (paged).  n new tokens (queries) per sequence.  kv_bytes: bytes per
    cached element when the cache is stored narrower than the inputs (1 for
    FP8 codes, whose per-KV-head scales are read too; with block_scales one
    K and one V scale per block and KV head read instead)."""
    B, h, g, d, eb = w.B, w.h, w.g, w.d, w.elem_bytes
    cb = eb if kv_bytes is None else kv_bytes
    kv_read = 2 * int(attended.sum()) * g * d * cb
    q_read = B * h * n * d * eb
    out_write = B * h * n * d * 4 + B * h * n * 4
    append_write = 2 * B * g * n * d * cb
    append_read = 2 * B * g * n * d * eb
    table = 0 if nblocks is None else int(nblocks.sum()) * 4
    scales = 0 if kv_bytes is None else 2 * g * 4
    if block_scales and nblocks is not None:
        scales = 2 * int(nblocks.sum()) * g * 4
    decode = kv_read + q_read + out_write + table + B * 4 + scales
    # One-call step: the new token's K/V are read once, from k_new / v_new
    # (counted in kv_read at the cache's width, so the difference to the
    # inputs' width is added), and written once into the cache.
    new_read = 2 * B * g * n * d * (eb - cb)
    return dict(decode=decode, step=decode + append_write + append_read + B * 4 + scales,
                fused=decode + new_read + append_write, kv_read=kv_read)


def attention_flops(w, before, n=1, window=0):
    """Floating-point operations of the attention of one step, counted per
    visible position of every query row (not the dense rectangle): 2*d for
    the score q.k and 2*d for adding p*V, so 4*d per (row, position).  Token
    t of a sequence with ``before`` cached positions sees before + t + 1
    positions, at most ``window`` with a sliding window."""
    total = 0
    for b0 in before.tolist():
        for t in range(n):
            vis = b0 + t + 1
            total += min(vis, window) if window > 0 else vis
    return 4 * w.d * w.h * total


def cpu_model_name() -> str:
    """The host CPU's model name (/proc/cpuinfo, or lscpu when that is terse)."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                alt = line.split(":", 1)[1].strip()
                if len(alt) > len(model):
                    model = alt
    except (OSError, subprocess.SubprocessError):
        pass
    return model


def cpu_baseline(w, x, paged: bool, budget_s: float = 12.0, fp8=None, decode_bytes=None):
    """The oracle (plain C, fp64, OpenMP over (sequence, head) rows) timed on
    this host on the same inputs.  Runs whole batches until about budget_s
    seconds have passed (at least one), reports decode tokens/s.  fp8:
    (k codes, v codes, k scales, v scales) of an FP8 cache on the host."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    runs, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        if fp8 is not None:
            oracle.decode_fp8(x["q"], *fp8, x["seq_lens_after"], x["scale"],
                              block_table=x["block_table"] if paged else None,
                              block_size=x.get("block_size", 16), nthreads=threads)
        elif paged:
            oracle.decode(x["q"], x["k_pool"], x["v_pool"], x["seq_lens_after"], x["scale"],
                          block_table=x["block_table"], block_size=x["block_size"], nthreads=threads)
        else:
            oracle.decode(x["q"], x["k_cache"], x["v_cache"], x["seq_lens_after"], x["scale"],
                          nthreads=threads)
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total >= budget_s or t_total / runs > budget_s / 2:
            break
    per_step = t_total / runs
    # one single-threaded run of the same batch
    t0 = time.perf_counter()
    if fp8 is not None:
        oracle.decode_fp8(x["q"], *fp8, x["seq_lens_after"], x["scale"],
                          block_table=x["block_table"] if paged else None,
                          block_size=x.get("block_size", 16), nthreads=1)
    elif paged:
        oracle.decode(x["q"], x["k_pool"], x["v_pool"], x["seq_lens_after"], x["scale"],
                      block_table=x["block_table"], block_size=x["block_size"], nthreads=1)
    else:
        oracle.decode(x["q"], x["k_cache"], x["v_cache"], x["seq_lens_after"], x["scale"],
                      nthreads=1)
    single = time.perf_counter() - t0
    res = {"value": w.B / per_step, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"full batch of the workload (B={w.B}), decode only, {runs} run(s), "
                     f"{per_step:.3f} s per run",
           "single_thread_value": w.B / single, "host_cpu": cpu_model_name()}
    if decode_bytes:  # the same algorithmic bytes as the GPU's decode call
        res["effective_gbs"] = round(decode_bytes / per_step / 1e9, 3)
        res["single_thread_effective_gbs"] = round(decode_bytes / single / 1e9, 3)
    return res


def bench_block_op(args, torch, kvc, W):
    """Bandwidth of the block operations: bytes read + written per call over
    the average call time (K calls captured in one HIP graph)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(77)
    if args.op == "copy_blocks":
        w = W.WORKLOADS["paged_gqa_bf16"] if args.workload == "gqa_70b_bf16" else W.WORKLOADS[args.workload]
        nb, n_pairs = 16384, 4096
        kp = torch.empty((nb, w.g, w.block_size, w.d), dtype=w.torch_dtype, device=dev).normal_()
        vp = torch.empty_like(kp).normal_()
        perm = torch.randperm(nb, generator=gen)
        pairs = torch.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], 1).to(torch.int32).to(dev)
        moved = 2 * 2 * n_pairs * w.g * w.block_size * w.d * w.elem_bytes
        call = lambda: kvc.copy_blocks(kp, vp, pairs)  # noqa: E731
        cfg = {"workload": f"copy_blocks {n_pairs} of {nb} blocks [g={w.g}, bs={w.block_size}, "
                           f"d={w.d}] bf16", "pairs": n_pairs}
    else:
        w = W.WORKLOADS[args.workload]
        x = W.make_contiguous(w)
        ks, vs = x["k_cache"].to(dev), x["v_cache"].to(dev)
        kd, vd = torch.empty_like(ks), torch.empty_like(vs)
        lens = x["seq_lens_after"].to(dev)
        parent = torch.randint(0, w.B, (w.B,), generator=gen, dtype=torch.int32)
        moved = 2 * 2 * int(x["seq_lens_after"][parent.long()].sum()) * w.g * w.d * w.elem_bytes
        parent = parent.to(dev)
        call = lambda: kvc.gather_cache(ks, vs, lens, parent, kd, vd)  # noqa: E731
        cfg = {"workload": f"gather_cache {w.name} (B={w.B}, g={w.g}, T={w.T}, d={w.d})"}
    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            call()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = moved / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"{args.op} bandwidth (bytes read + written per call / call time)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (bit-exact copies)",
        "data": "synthetic, seeded", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": moved, "traffic": None},
        "cpu_baseline": None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_70b_bf16")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="override the workload's head dimension (bf16 caches: 64, 80, 96, 128 and 256 run "
                         "on the matrix-core kernels, other values on the generic kernel)")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="override the workload's split count (0 = library's choice)")
    ap.add_argument("--copies", type=int, default=0, help="KV cache copies to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="a step is kvc_append then the decode call (two calls) instead of one "
                         "kvc_append_decode_attention call")
    ap.add_argument("--queries", type=int, default=1,
                    help="new tokens per sequence in one step (draft tokens checked at once, or a "
                         "prefill chunk after the cached prefix): kvc_append_decode_attention_multi")
    ap.add_argument("--slice-baseline", action="store_true",
                    help="with --queries n: also time the attention of the same rows in groups "
                         "of at most 32 rows per KV head, one kvc_decode_attention_multi call "
                         "each (every call reads the unit's K/V), beside the one-call step")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window W: each token sees the last W positions up to itself "
                         "(kvc_append_decode_attention_window)")
    ap.add_argument("--ring", action="store_true",
                    help="with --window: the contiguous cache is a ring of W + n + 14 slots")
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "gather_cache"],
                    help="decode: the decode step (default); copy_blocks: copy-on-write copies of "
                         "4096 pool blocks of the paged workload; gather_cache: beam re-ranking of "
                         "the contiguous workload's caches")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="the cache holds FP8 E4M3 codes with per-KV-head scales "
                         "(kvc_append_decode_attention_fp8); one token per sequence, no window")
    ap.add_argument("--fp8-block-scales", action="store_true",
                    help="with --kv-fp8 on a paged workload: one scale per (physical block, KV "
                         "head) instead of per KV head (kvc_decode_attention_fp8_paged_block_scaled)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying HIP graphs")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="steps per HIP graph in the timed region (0 = automatic: whole cycles "
                         "of the cache copies, enough of them that one replay keeps the GPU busy "
                         "for about 200 us, so that host replays do not pace small steps)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before warm-up, copy this many MiB device-to-device once (a plain copy "
                         "of known size for scaling hardware byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of "
                         "an --eager --calibration-copy-mib run into the stored traffic figure")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-pmc: a command line to record in the summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                      args.workload + ("_kvfp8" if args.kv_fp8 else ""),
                      args.calibration_copy_mib or 1024, args.command)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_gqa_amd as kvc
    import kvc_workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    kvc.load_library()
    if args.op != "decode":
        bench_block_op(args, torch, kvc, W)
        return
    w = W.WORKLOADS[args.workload]
    if args.head_dim is not None and args.head_dim != w.d:
        # the same shapes, seeds and lengths with another head dimension;
        # the workload name says so (and no stored counter figure matches)
        w = dataclasses.replace(w, d=args.head_dim, name=f"{w.name}_d{args.head_dim}")
    ns = w.num_splits if args.num_splits is None else args.num_splits
    dev = torch.device("cuda:0")

    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    if w.paged:
        # blocks for the n new tokens of a multi-token step
        x = W.make_paged(w, new_tokens=max(args.queries, 1))
        k_src, v_src = x["k_pool"], x["v_pool"]
        nblocks = W.block_counts(x["seq_lens_before"] + max(args.queries, 1), x["block_size"])
    else:
        # a ring cache holds W + n - 1 positions plus spare slots, every slot
        # written; a linear cache holds the n new tokens past the spare slots
        if args.ring:
            t_cap = args.window + args.queries + 14
        elif args.queries > w.cap_pad and w.T is not None:
            t_cap = w.T + args.queries + w.cap_pad
        else:
            t_cap = None
        x = W.make_contiguous(w, t_cap=t_cap)
        k_src, v_src = x["k_cache"], x["v_cache"]
        nblocks = None
    fp8 = args.kv_fp8
    if fp8 and w.dtype != "bf16":
        print("--kv-fp8 takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    blk_sc = args.fp8_block_scales
    if blk_sc and not (fp8 and w.paged and not args.separate):
        print("--fp8-block-scales needs --kv-fp8, a paged workload and the one-call step",
              file=sys.stderr)
        sys.exit(2)
    if fp8:
        # per-KV-head scales amax / 448 over the cache (or per block and KV
        # head with --fp8-block-scales); codes by torch's
        # float8_e4m3fn conversion (round to nearest even), from the same
        # seeded N(0, 1) cache as the bf16 run
        def quantise(t):
            if blk_sc:  # per (block, KV head): amax over the block's rows
                sc = (t.float().abs().amax(dim=(2, 3)) / 448.0).clamp(min=1e-12)
                codes = (t.float() / sc.view(sc.shape[0], -1, 1, 1)).to(torch.float8_e4m3fn)
                return codes.view(torch.uint8), sc
            amax = t.float().abs().amax(dim=(0, 2, 3))
            sc = (amax / 448.0).clamp(min=1e-12)
            codes = (t.float() / sc.view(1, -1, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
            return codes, sc
        k_src, k_sc = quantise(k_src)
        v_src, v_sc = quantise(v_src)
        k_sc_d, v_sc_d = k_sc.to(dev), v_sc.to(dev)
    cache_bytes = 2 * k_src.numel() * k_src.element_size()
    # At least 3 copies and 800 MB in all, so that the 256 MB Infinity Cache
    # cannot serve a repeat; at most 64 (one graph node per copy and step):
    # caches under 12.5 MB (the tiny workload) are then partly cache-resident.
    copies = args.copies or min(64, max(3, -(-800 * 2**20 // cache_bytes)))
    k0, v0 = k_src.to(dev), v_src.to(dev)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    nq = args.queries
    win, ring = args.window, args.ring
    if nq < 1 or (nq > 1 and (args.separate or (w.T is None and not w.paged))):
        print("--queries takes n >= 1; n > 1 only with the one-call step", file=sys.stderr)
        sys.exit(2)
    if args.slice_baseline and (nq < 2 or args.window or w.paged):
        print("--slice-baseline needs --queries n > 1, no window and a contiguous workload",
              file=sys.stderr)
        sys.exit(2)
    if win < 0 or (win > 0 and args.separate) or (ring and (win <= 0 or w.paged)):
        print("--window takes W >= 0 with the one-call step; --ring needs --window and a "
              "contiguous workload", file=sys.stderr)
        sys.exit(2)
    windowed = win > 0
    if nq > 1:
        gen = torch.Generator().manual_seed(w.seed + 77)
        q = W.randn((w.B, w.h, nq, w.d), w.torch_dtype, gen).to(dev)
        k_new = W.randn((w.B, w.g, nq, w.d), w.torch_dtype, gen).to(dev)
        v_new = W.randn((w.B, w.g, nq, w.d), w.torch_dtype, gen).to(dev)
    else:
        q = x["q"].to(dev)
        k_new, v_new = x["k_new"].to(dev), x["v_new"].to(dev)
    sl_before, sl_after = x["seq_lens_before"].to(dev), x["seq_lens_after"].to(dev)
    bt = x["block_table"].to(dev) if w.paged else None
    if windowed:  # the window calls take [B, h, n, d] queries for every n
        q = q.view(w.B, w.h, nq, w.d)
        k_new, v_new = k_new.view(w.B, w.g, nq, w.d), v_new.view(w.B, w.g, nq, w.d)
    if nq > 1 or windowed:
        out = torch.empty((w.B, w.h, nq, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.h, nq), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((w.B, w.h, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.h), dtype=torch.float32, device=dev)
    hq = w.h * nq  # query rows per sequence (the workspace query takes h * n)
    if w.paged:
        capacity = bt.shape[1] * x["block_size"]
    else:
        capacity = k0.shape[2]
    max_len = capacity
    if windowed:  # plans and workspaces cover the positions a window reads
        max_len = min(win + nq - 1, max_len)
    ws_bytes = kvc.workspace_bytes(w.B, hq, w.g, w.d, max_len, ns, dtype=w.torch_dtype,
                                   paged=w.paged)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # the plan and launch of this call (n tokens, window): the _multi queries
    plan_dtype = "fp8" if fp8 else w.torch_dtype
    split_mode, chunk_len, num_chunks = kvc.plan_multi(w.B, w.h, w.g, w.d, nq, capacity, window=win,
                                                       num_splits=ns, dtype=plan_dtype,
                                                       paged=w.paged)
    waves, n_wgs, launch_chunk, launch_chunks = kvc.launch_shape_multi(
        w.B, w.h, w.g, w.d, nq, capacity, window=win, num_splits=ns, dtype=plan_dtype,
        paged=w.paged)
    merged = split_mode == "stream" or launch_chunks > 1

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * 2**20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst

    def append_call(i):
        kc, vc = ks[i % copies], vs[i % copies]
        if fp8:
            kvc.append_fp8(k_new, v_new, kc, vc, k_sc_d, v_sc_d, sl_before, block_table=bt)
        else:
            kvc.append(k_new, v_new, kc, vc, sl_before, block_table=bt)

    def decode_call(i):
        kc, vc = ks[i % copies], vs[i % copies]
        if fp8:
            kvc.decode_fp8(q, kc, vc, k_sc_d, v_sc_d, sl_after, block_table=bt, scale=x["scale"],
                           num_splits=ns, workspace=ws, out=out, lse=lse)
        elif w.paged:
            kvc.decode_paged(q, kc, vc, bt, sl_after, scale=x["scale"], num_splits=ns,
                             workspace=ws, out=out, lse=lse)
        else:
            kvc.decode(q, kc, vc, sl_after, scale=x["scale"], num_splits=ns, workspace=ws,
                       out=out, lse=lse)

    def fused_call(i):
        kc, vc = ks[i % copies], vs[i % copies]
        if blk_sc:
            kvc.decode_fp8_block_scaled(q.view(w.B, w.h, nq, w.d), kc, vc, k_sc_d, v_sc_d,
                                        sl_before, bt, window=win, scale=x["scale"],
                                        num_splits=ns, workspace=ws,
                                        out=out.view(w.B, w.h, nq, w.d),
                                        lse=lse.view(w.B, w.h, nq),
                                        k_new=k_new.view(w.B, w.g, nq, w.d),
                                        v_new=v_new.view(w.B, w.g, nq, w.d))
        elif fp8 and (nq > 1 or windowed):
            kvc.decode_fp8_window(q, kc, vc, k_sc_d, v_sc_d, sl_before, window=win, ring=ring,
                                  block_table=bt, scale=x["scale"], num_splits=ns, workspace=ws,
                                  out=out, lse=lse, k_new=k_new, v_new=v_new)
        elif fp8:
            kvc.decode_fp8(q, kc, vc, k_sc_d, v_sc_d, sl_before, block_table=bt, scale=x["scale"],
                           num_splits=ns, workspace=ws, out=out, lse=lse, k_new=k_new,
                           v_new=v_new)
        elif windowed:
            kvc.decode_window(q, kc, vc, sl_before, win, ring=ring, block_table=bt,
                              scale=x["scale"], num_splits=ns, workspace=ws, out=out, lse=lse,
                              k_new=k_new, v_new=v_new)
        elif nq > 1:
            kvc.append_decode_multi(q, k_new, v_new, kc, vc, sl_before, block_table=bt,
                                    scale=x["scale"], num_splits=ns, workspace=ws, out=out,
                                    lse=lse)
        else:
            kvc.append_decode(q, k_new, v_new, kc, vc, sl_before, block_table=bt, scale=x["scale"],
                              num_splits=ns, workspace=ws, out=out, lse=lse)

    def step(i):
        if args.separate:
            append_call(i)
            decode_call(i)
        else:
            fused_call(i)

    # The call whose bandwidth the roofline reports.
    timed_call = decode_call if args.separate else fused_call

    print(f"[bench] {copies} cache copies ({cache_bytes * copies / 2**30:.2f} GiB), split "
          f"{split_mode} chunk_len={chunk_len} num_chunks={num_chunks}; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(args.warmup, copies)):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # HIP graphs hold whole steps (every kernel of a step), so that host
    # launch latency does not sit between the kernels.  --eager launches from
    # Python instead.
    graphs = []
    cycle = None
    if not args.eager:
        for r in range(copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(r)
            graphs.append(gr)
        for r in range(copies):
            graphs[r].replay()
        torch.cuda.synchronize()
        # Graphs of G steps back to back, step i on cache copy i mod copies,
        # as a model's decode graph holds one attention step per layer: G is
        # a whole number of cycles over the copies, enough that one replay
        # keeps the GPU busy for about 200 us (a step of a few µs would
        # otherwise wait for the host's next replay), and at most K.
        gsteps = args.graph_steps
        if gsteps <= 0:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(copies):
                graphs[r].replay()
            e1.record()
            torch.cuda.synchronize()
            cycle_us = max(e0.elapsed_time(e1) * 1e3, 1e-3)
            gsteps = copies * max(1, math.ceil(200.0 / cycle_us))
        gsteps = max(1, min(gsteps, args.steps))
        full_graphs, rest_steps = divmod(args.steps, gsteps)

        def capture(n):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(n):
                    step(i)
            return gr
        cycle = capture(gsteps)
        rest = capture(rest_steps) if rest_steps else None
        cycle.replay()
        if rest is not None:
            rest.replay()
        torch.cuda.synchronize()

    # Timed region: exactly K steps between two synchronisations.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    if graphs:
        for _ in range(full_graphs):
            cycle.replay()
        if rest is not None:
            rest.replay()
    else:
        for i in range(args.steps):
            step(i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # Secondary figures, outside the timed region: each of K steps timed on
    # its own (median and spread), and the hot repeat (one cache copy over
    # and over, so that caches may serve part of it).
    def replay_one(i):
        if graphs:
            graphs[i % copies].replay()
        else:
            step(i)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(marks):
        e0.record()
        replay_one(i)
        e1.record()
    torch.cuda.synchronize()
    each = sorted(e0.elapsed_time(e1) for e0, e1 in marks)
    pct = lambda q: each[min(len(each) - 1, int(q * (len(each) - 1) + 0.5))]  # noqa: E731
    h_start = torch.cuda.Event(enable_timing=True)
    h_end = torch.cuda.Event(enable_timing=True)
    h_start.record()
    for _ in range(args.steps):
        replay_one(0)
    h_end.record()
    torch.cuda.synchronize()
    hot_ms = h_start.elapsed_time(h_end) / args.steps

    # The dominant kernel: decode calls alone, back to back on the launch
    # stream (a HIP graph holding one call per cache copy, replayed until at
    # least K calls ran), between two HIP events on that stream.
    reps = -(-args.steps // copies)
    if graphs:
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for r in range(copies):
                timed_call(r)
        dgraph.replay()
        torch.cuda.synchronize()
    d_start = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    d_start.record()
    for i in range(reps):
        if graphs:
            dgraph.replay()
        else:
            for r in range(copies):
                timed_call(r)
    d_end.record()
    torch.cuda.synchronize()
    dec_avg_ms = d_start.elapsed_time(d_end) / (reps * copies)

    # The same attention as groups of at most 32 rows per KV head, one
    # kvc_decode_attention_multi call each over the cache that already holds
    # the n tokens: every call reads its units' K/V again.
    slice_res = None
    if args.slice_baseline:
        per = max(1, 32 // w.m)  # tokens per call
        groups = [(t0, min(nq, t0 + per)) for t0 in range(0, nq, per)]
        qs = [q[:, :, t0:t1].contiguous() for t0, t1 in groups]
        outs = [torch.empty((w.B, w.h, t1 - t0, w.d), dtype=torch.float32, device=dev)
                for t0, t1 in groups]
        lses = [torch.empty((w.B, w.h, t1 - t0), dtype=torch.float32, device=dev)
                for t0, t1 in groups]
        sls = [(sl_before + t1).to(torch.int32) for t0, t1 in groups]
        ws_s = torch.empty(max(1, kvc.workspace_bytes(w.B, w.h * per, w.g, w.d, k0.shape[2], ns)),
                           dtype=torch.uint8, device=dev)

        def slices_call(i):
            kc, vc = ks[i % copies], vs[i % copies]
            for qq, oo, ll, sl in zip(qs, outs, lses, sls):
                kvc.decode_multi(qq, kc, vc, sl, scale=x["scale"], num_splits=ns, workspace=ws_s,
                                 out=oo, lse=ll)
        for r in range(copies):
            slices_call(r)
        torch.cuda.synchronize()
        sgraph = None
        if graphs:
            sgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(sgraph):
                for r in range(copies):
                    slices_call(r)
            sgraph.replay()
            torch.cuda.synchronize()
        s_start = torch.cuda.Event(enable_timing=True)
        s_end = torch.cuda.Event(enable_timing=True)
        s_start.record()
        for _ in range(reps):
            if sgraph is not None:
                sgraph.replay()
            else:
                for r in range(copies):
                    slices_call(r)
        s_end.record()
        torch.cuda.synchronize()
        slice_ms = s_start.elapsed_time(s_end) / (reps * copies)
        slice_res = {"calls_per_step": len(groups), "tokens_per_call": per,
                     "ms_per_step": round(slice_ms, 5),
                     "note": "attention only (the cache already holds the tokens), "
                             "kvc_decode_attention_multi per group of <= 32 rows per KV head"}

    hi = x["seq_lens_before"].to(torch.int64) + nq
    lo = torch.clamp(x["seq_lens_before"].to(torch.int64) + 1 - win, min=0) if windowed \
        else torch.zeros_like(hi)
    nbytes = algorithmic_bytes(w, hi - lo, nblocks, n=nq, kv_bytes=1 if fp8 else None,
                               block_scales=blk_sc)
    # stored counter runs are of the default (one-call) step
    traffic = None if (args.separate or nq > 1 or windowed) else \
        stored_traffic(w.name + ("_kvfp8" if fp8 else ""))
    call_bytes = nbytes["decode"] if args.separate else nbytes["fused"]
    achieved_gbs = call_bytes / (dec_avg_ms * 1e-3) / 1e9
    tokens_per_s = w.B * nq / (ms_per_step * 1e-3)
    # Which roof bounds the call: its bytes at 8 TB/s or its flops at the
    # bf16 matrix-core peak, whichever takes longer (FP8 caches too: their
    # codes are widened to bf16 for the same matrix-core products).
    flops = attention_flops(w, x["seq_lens_before"], n=nq, window=win)
    mfma_bound = w.dtype == "bf16" and \
        flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > call_bytes / (HBM_PEAK_GBS * 1e9)
    achieved_tflops = flops / (dec_avg_ms * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline and nq == 1 and not windowed and not blk_sc:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x, w.paged,
                           fp8=(k_src.numpy(), v_src.numpy(), k_sc.numpy(), v_sc.numpy())
                           if fp8 else None, decode_bytes=nbytes["decode"])

    res = {
        "metric": "decode tokens/s (GQA KV-cache attention, one layer)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3 KV cache (per-block, per-KV-head scales), bf16 q, fp32 accumulate"
                  if blk_sc else
                  "fp8 e4m3 KV cache (per-KV-head scales), bf16 q, fp32 accumulate" if fp8
                  else "bf16 in, fp32 accumulate" if w.dtype == "bf16" else "f32"),
        "data": "synthetic, seeded N(0,1)",
        "config": {
            "workload": w.name, "B": w.B, "h": w.h, "g": w.g, "d": w.d,
            "kv_len_before_step": w.T if w.T is not None else list(w.T_range),
            "paged": w.paged, "block_size": w.block_size if w.paged else None,
            "num_splits": ns, "split": split_mode, "chunk_len": chunk_len,
            "num_chunks": num_chunks, "queries_per_sequence": nq, "window": win,
            "ring_cache": ring, "kv_cache": "fp8_e4m3" if fp8 else w.dtype,
            # the launch-shape query describes calls without a sliding window
            "launch": None if windowed else {"waves_per_workgroup": waves, "workgroups": n_wgs,
                                             "chunk_len": launch_chunk, "chunks": launch_chunks},
            "cache_copies_rotated": copies,
            "rotation_exceeds_infinity_cache": copies * cache_bytes >= 800 * 2**20,
            "parallelism": "single GPU",
        },
        "step": (("kvc_append_fp8 + decode call" if args.separate
                  else f"one kvc_append_decode_attention_fp8_{'window' if windowed else 'multi'} "
                       f"call (W={win}, ring={ring}, {nq} tokens per sequence)"
                  if (nq > 1 or windowed) else "one kvc_append_decode_attention_fp8 call") if fp8
                 else "kvc_append + decode call" if args.separate
                 else f"one kvc_append_decode_attention_window call (W={win}, ring={ring}, "
                      f"{nq} tokens per sequence)" if windowed
                 else f"one kvc_append_decode_attention_multi call ({nq} tokens per sequence)"
                 if nq > 1 else "one kvc_append_decode_attention call"),
        "step_hbm_gbs": round((nbytes["step"] if args.separate else nbytes["fused"])
                              / (ms_per_step * 1e-3) / 1e9, 1),
        "step_ms_each": {"p10": round(pct(0.1), 5), "p50": round(pct(0.5), 5),
                         "p90": round(pct(0.9), 5), "samples": len(each),
                         "note": "each step timed alone (includes its launch)"},
        "hot_ms_per_step": round(hot_ms, 5),
        "timing": "eager" if args.eager else f"HIP graphs of {gsteps} whole steps (step i on cache copy i mod copies)",
        "roofline": ({
            "bound": "mfma",
            "kernel": "append+decode call: " + ("partials + log-sum-exp merge" if merged
                                                else "one kernel, no merge"),
            "achieved": round(achieved_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": flops,
            "flops_counted": "4*d per visible position per query row",
            "hbm_achieved_gbs": round(achieved_gbs, 1),
            "algorithmic_bytes_per_launch": call_bytes,
            "decode_call_ms_avg": round(dec_avg_ms, 5),
            "traffic": traffic,
        } if mfma_bound else {
            "bound": "hbm",
            "kernel": ("decode call" if args.separate else "append+decode call") + ": "
                      + ("partials + log-sum-exp merge" if merged else "one kernel, no merge"),
            "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": call_bytes,
            "decode_call_ms_avg": round(dec_avg_ms, 5),
            "traffic": traffic,
            "mfma_achieved_tflops": round(achieved_tflops, 2),
        }),
        "cpu_baseline": cpu,
    }
    if slice_res is not None:
        slice_res["speedup_of_one_call"] = round(slice_res["ms_per_step"] / dec_avg_ms, 3)
        res["slice_baseline"] = slice_res
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
