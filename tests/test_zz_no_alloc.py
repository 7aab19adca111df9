"""GPU check of kvc_append_decode_attention_noalloc (the one-call decode
step whose split partials live in the library's static scratch instead of
a caller's workspace), called through the C ABI: two calls in a row, the
second with a smaller input, each against kvc_append_decode_attention on
the same inputs (identical caches afterwards, outputs within the parity
bar and in fact bit-identical: same kernels, same plan) and against the
oracle."""
from __future__ import annotations

import ctypes
import sys

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W
import oracle
from gpu_util import attended_vmax_contig, check_parity, dev

pytestmark = pytest.mark.gpu

SCRATCH_STATUS = 5


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _run(lib, noalloc: bool, x, w, num_splits):
    """One call of either entry point on fresh copies of the caches."""
    kc, vc = dev(x["k_cache"]), dev(x["v_cache"])
    q, kn, vn, sl = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"]), dev(x["seq_lens_before"])
    out = torch.full((w.B, w.h, w.d), float("nan"), device="cuda")
    lse = torch.full((w.B, w.h), float("nan"), device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    t_cap = x["k_cache"].shape[2]
    if noalloc:
        st = lib.kvc_append_decode_attention_noalloc(
            _ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), _ptr(sl), w.B, w.h, w.g, w.d, t_cap,
            x["scale"], kvc.BF16, num_splits, _ptr(out), _ptr(lse), stream)
    else:
        need = lib.kvc_decode_workspace_bytes(w.B, w.h, w.g, w.d, kvc.BF16, t_cap, num_splits, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        st = lib.kvc_append_decode_attention(
            _ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), _ptr(sl), w.B, w.h, w.g, w.d, t_cap,
            x["scale"], kvc.BF16, num_splits, _ptr(ws), need, _ptr(out), _ptr(lse), stream)
    assert st == 0, kvc.KvcError("append_decode", st)
    torch.cuda.synchronize()
    return out, lse, kc, vc


# (name, B, h, g, T, num_splits): both split their positions, so the
# partials go through the scratch; the second is smaller than the first
CALLS = [("long_mqa_like", 2, 32, 1, 40000, 0), ("gqa_small", 3, 16, 2, 3000, 3)]


def test_noalloc_matches_the_workspace_entry_point():
    lib = kvc.load_library()
    scratch = lib.kvc_noalloc_scratch_bytes()
    assert scratch == 16 << 20
    for k, (name, B, h, g, T, ns) in enumerate(CALLS):
        _log(f"case noalloc {name} B={B} h={h} g={g} T={T} splits={ns}")
        w = W.Workload(name, B=B, h=h, g=g, d=128, dtype="bf16", T=T, seed=1200 + k)
        x = W.make_contiguous(w)
        need = lib.kvc_decode_workspace_bytes(B, h, g, 128, kvc.BF16, x["k_cache"].shape[2], ns, 0)
        assert 0 < need <= scratch, (name, need)
        o0, l0, k0, v0 = _run(lib, False, x, w, ns)
        o1, l1, k1, v1 = _run(lib, True, x, w, ns)
        assert torch.equal(k0, k1) and torch.equal(v0, v1), f"{name}: caches differ"
        assert torch.equal(o0, o1) and torch.equal(l0, l1), f"{name}: results differ"
        after = x["seq_lens_after"]
        ro, rl = oracle.decode(x["q"], k1.cpu(), v1.cpu(), after, x["scale"])
        e = check_parity(o1, l1, ro, rl, attended_vmax_contig(v1.cpu(), after), name)
        _log(f"  err/vmax {e[0]:.2e} lse {e[1]:.2e}")


def test_noalloc_rejects_a_split_beyond_the_scratch():
    """A plan that needs more than the scratch (200 chunks of 8 x 32 rows over
    131088 positions): KVC_ERR_SCRATCH, nothing
    launched (out keeps its contents)."""
    lib = kvc.load_library()
    w = W.Workload("too_big", B=8, h=32, g=1, d=128, dtype="bf16", T=131072, seed=1210)
    need = lib.kvc_decode_workspace_bytes(8, 32, 1, 128, kvc.BF16, 131088, 200, 0)
    assert need > lib.kvc_noalloc_scratch_bytes()
    q = torch.zeros((8, 32, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((8, 1, 64, 128), dtype=torch.bfloat16, device="cuda")  # never read
    kn = torch.zeros((8, 1, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.zeros((8,), dtype=torch.int32, device="cuda")
    out = torch.full((8, 32, 128), 3.0, device="cuda")
    lse = torch.full((8, 32), 3.0, device="cuda")
    st = lib.kvc_append_decode_attention_noalloc(
        _ptr(q), _ptr(kn), _ptr(kn), _ptr(kc), _ptr(kc), _ptr(sl), 8, 32, 1, 128, 131088,
        w.scale, kvc.BF16, 200, _ptr(out), _ptr(lse), None)
    assert st == SCRATCH_STATUS
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 3.0).all())
