"""Host-only checks of libkvc: the library loads, exports every function
include/kvc.h declares, plans work splits as documented, and rejects bad
arguments with the documented status before touching the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import kv_cache_gqa_amd as kvc
import kvc_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH),
                                reason="libkvc.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kvc_append", "kvc_decode_attention", "kvc_decode_attention_paged",
              "kvc_append_decode_attention", "kvc_append_decode_attention_paged",
              "kvc_decode_workspace_bytes", "kvc_decode_plan", "kvc_decode_launch_shape",
              "kvc_decode_plan_multi", "kvc_decode_launch_shape_multi",
              "kvc_status_string", "kvc_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = kvc.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = kvc.load_library()
    assert lib.kvc_status_string(0) == b"ok"
    assert lib.kvc_status_string(3).startswith(b"workspace")
    assert lib.kvc_version() > 0


def test_plan_modes():
    # explicit 64 splits over 131073 positions: chunks of 2080 (a multiple of 32)
    assert kvc.plan(4, 32, 1, 128, 131073 + 15, 64) == ("chunks", 2080, 64)
    # automatic: contiguous -> chunk count fixed at launch; paged -> stream
    for (B, h, g, T) in [(8, 32, 32, 2064), (32, 64, 8, 4112), (64, 32, 8, 8208), (4, 32, 1, 131088)]:
        assert kvc.plan(B, h, g, 128, T, 0) == ("auto_chunks", 0, 0)
        assert kvc.plan(B, h, g, 128, T, 0, paged=True) == ("stream", 0, 0)
        assert kvc.plan(B, h, g, 128, T, kvc.SPLITS_STREAM) == ("stream", 0, 0)
    # the generic kernel (fp32; bf16 or FP8 head dims other than 64, 80, 96,
    # 128, 256) always chunks
    assert kvc.plan(1, 4, 2, 16, 48, 0, dtype=torch.float32)[0] == "chunks"
    assert kvc.plan(2, 8, 2, 112, 4096, 0, paged=True)[0] == "chunks"
    assert kvc.plan(2, 8, 2, 112, 4096, 0, dtype=kvc.FP8_E4M3, paged=True)[0] == "chunks"
    for d in (80, 96):
        assert kvc.plan(2, 8, 2, d, 4096, 0, dtype=kvc.FP8_E4M3, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 8, 2, 128, 4096, kvc.SPLITS_STREAM, dtype=torch.float32)[0] == "chunks"
    # bf16 head dims 64, 80, 96 and 256: the multi-row kernel.  Paged pools stream
    # automatically at d = 256 with at most 16 rows per KV head (FP8 not),
    # and whenever asked while a unit's rows fit one 4-wavefront work-group
    # (64 rows, or 128 below d = 256); contiguous caches take chunks fixed
    # at launch.
    assert kvc.plan(2, 8, 2, 256, 4096, 0, paged=True)[0] == "stream"
    assert kvc.plan(2, 32, 2, 256, 4096, 0, paged=True)[0] == "stream"
    assert kvc.plan(2, 8, 2, 256, 4096, 0, dtype=kvc.FP8_E4M3, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 34, 2, 256, 4096, 0, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 8, 2, 64, 4096, 0, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 8, 2, 80, 4096, 0, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 8, 2, 96, 4096, 0, paged=True)[0] == "auto_chunks"
    for d in (64, 80, 96, 256):
        assert kvc.plan(2, 8, 2, d, 4096, kvc.SPLITS_STREAM, paged=True)[0] == "stream"
        assert kvc.plan(2, 8, 2, d, 4096, 0)[0] == "auto_chunks"
        assert kvc.plan(2, 8, 8, d, 4096, kvc.SPLITS_STREAM)[0] == "auto_chunks"
    # more than 32 query rows per KV head at d = 128: the multi-row kernel,
    # chunks unless a paged pool asks for the stream grid
    assert kvc.plan(2, 64, 1, 128, 4096, 0, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 64, 1, 128, 4096, kvc.SPLITS_STREAM, paged=True)[0] == "stream"
    assert kvc.plan(2, 128, 1, 128, 4096, kvc.SPLITS_STREAM, paged=True)[0] == "stream"
    assert kvc.plan(2, 256, 1, 128, 4096, kvc.SPLITS_STREAM, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 128, 1, 256, 4096, kvc.SPLITS_STREAM, paged=True)[0] == "auto_chunks"
    assert kvc.plan(2, 64, 1, 128, 4096, kvc.SPLITS_STREAM)[0] == "auto_chunks"
    # FP8 caches with 17-32 rows per KV head on the decode kernel (two query
    # tiles) chunk on paged pools; up to 16 rows and bf16 stream
    for kv in (kvc.FP8_E4M3, torch.bfloat16):
        want = "auto_chunks" if kv == kvc.FP8_E4M3 else "stream"
        assert kvc.plan(64, 32, 1, 128, 8208, 0, dtype=kv, paged=True)[0] == want
        assert kvc.plan(64, 24, 1, 128, 8208, 0, dtype=kv, paged=True)[0] == want
        assert kvc.plan(64, 16, 1, 128, 8208, 0, dtype=kv, paged=True)[0] == "stream"
    # the queries of calls with several tokens or a window (h query heads,
    # capacity): FP8 paged pools with n > 1 take chunks, bf16 ones stream;
    # windows chunk; n = 1 and no window match the single-token query
    fp8 = kvc.FP8_E4M3
    assert kvc.plan_multi(64, 32, 8, 128, 2, 8208, dtype=fp8, paged=True)[0] == "auto_chunks"
    assert kvc.plan_multi(64, 32, 8, 128, 2, 8208, paged=True)[0] == "stream"
    assert kvc.plan_multi(64, 32, 8, 128, 1, 8208, dtype=fp8, paged=True)[0] == "stream"
    assert kvc.plan_multi(64, 32, 8, 128, 2, 8208, window=1024, paged=True)[0] == "auto_chunks"
    for (B, h, g, d, L, ns, dt, pg) in [(32, 64, 8, 128, 4112, 0, torch.bfloat16, False),
                                         (64, 32, 8, 128, 8208, 0, fp8, True),
                                         (8, 8, 2, 96, 1000, 3, torch.float32, False)]:
        assert kvc.plan_multi(B, h, g, d, 1, L, num_splits=ns, dtype=dt, paged=pg) == \
            kvc.plan(B, h, g, d, L, ns, dtype=dt, paged=pg)
    # rows h * n; a window caps the planned length at W + n - 1
    assert kvc.plan_multi(2, 8, 2, 128, 4, 4096, num_splits=2) == kvc.plan(2, 32, 2, 128, 4096, 2)
    assert kvc.plan_multi(2, 8, 2, 128, 4, 4096, window=100, num_splits=2) == \
        kvc.plan(2, 32, 2, 128, 103, 2)
    lib = kvc.load_library()
    assert lib.kvc_decode_plan_multi(2, 8, 2, 128, 0, 0, 1, 64, 0, 0, None, None, None) == INVALID
    assert lib.kvc_decode_plan_multi(2, 8, 2, 128, 1, -1, 1, 64, 0, 0, None, None, None) == INVALID
    assert lib.kvc_decode_plan_multi(2, 4096, 2, 128, 32, 0, 1, 64, 0, 0, None, None, None) == \
        UNSUPPORTED
    # the head map is checked on the query heads, not on the h * n rows: 3 heads over 2 KV heads
    # is invalid however many tokens make the row count even
    for n in (1, 2, 4):
        assert lib.kvc_decode_plan_multi(2, 3, 2, 128, n, 0, 1, 64, 0, 0, None, None, None) == INVALID
        assert lib.kvc_decode_launch_shape_multi(2, 3, 2, 128, n, 0, 1, 64, 0, 0,
                                                 None, None, None, None) == INVALID
    assert lib.kvc_decode_plan_multi(2, 8, 0, 128, 2, 0, 1, 64, 0, 0, None, None, None) == INVALID
    assert lib.kvc_decode_launch_shape_multi(2, 8, 0, 128, 2, 0, 1, 64, 0, 0,
                                             None, None, None, None) == INVALID
    # stream mode needs B <= 1024
    assert kvc.plan(2048, 8, 8, 128, 512, 0, paged=True)[0] == "auto_chunks"
    # chunks: a multiple of 32, covering max_seq_len, at most 4096
    for (B, h, g, T) in [(8, 32, 32, 2064), (32, 64, 8, 4112), (64, 32, 8, 8208), (4, 32, 1, 131088),
                         (1, 4, 2, 48)]:
        for ns in (1, 3, 8, 64):
            _, cl, nc = kvc.plan(B, h, g, 128, T, ns)
            assert cl % 32 == 0 and cl * nc >= T and cl * (nc - 1) < T and cl <= 4096


def _ws(rows, d=128):
    return -(-rows * d * 4 // 256) * 256 + -(-rows * 4 // 256) * 256


def test_workspace_bytes():
    assert kvc.workspace_bytes(1, 4, 2, 16, 48, 1, dtype=torch.float32) == 0
    _, cl, nc = kvc.plan(4, 32, 1, 128, 131088, 64)
    assert kvc.workspace_bytes(4, 32, 1, 128, 131088, 64) == _ws(4 * 32 * nc)
    # stream mode: two records of m rows for each of at most 1024 work-groups
    assert kvc.workspace_bytes(32, 64, 8, 128, 4112, 0, paged=True) == _ws(1024 * 2 * 8)
    # automatic chunks: sized for 1024 work-groups -> 4 chunks per (b, j) at B*g = 256
    assert kvc.workspace_bytes(32, 64, 8, 128, 4112, 0) == _ws(32 * 64 * 4)
    # B*g = 4: 256 chunks asked, rounded to 544-position chunks -> 241 chunks
    chunk = -(-(-(-131088 // 256)) // 32) * 32
    assert chunk == 544
    assert kvc.workspace_bytes(4, 32, 1, 128, 131088, 0) == _ws(4 * 32 * -(-131088 // chunk))


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sl=FAKE, B=2, h=8, g=2, d=128, t_cap=64, scale=0.1, dtype=1,
             splits=1, ws=None, wsb=0, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.kvc_decode_attention(a["q"], a["k"], a["v"], a["sl"], a["B"], a["h"], a["g"], a["d"],
                                    a["t_cap"], a["scale"], a["dtype"], a["splits"], a["ws"],
                                    a["wsb"], a["out"], a["lse"], None)


def test_decode_validation_codes():
    lib = kvc.load_library()
    assert _decode(lib, h=8, g=3) == INVALID             # h % g != 0
    assert _decode(lib, g=0) == INVALID
    assert _decode(lib, d=0) == INVALID
    assert _decode(lib, q=None) == INVALID                # null pointer
    assert _decode(lib, out=None) == INVALID
    assert _decode(lib, t_cap=0) == INVALID
    assert _decode(lib, scale=float("inf")) == INVALID
    assert _decode(lib, splits=-2) == INVALID
    assert _decode(lib, d=300) == UNSUPPORTED
    assert _decode(lib, dtype=7) == UNSUPPORTED
    assert _decode(lib, splits=2, ws=None, wsb=0) == WORKSPACE   # plan needs a workspace
    need = lib.kvc_decode_workspace_bytes(2, 8, 2, 128, 1, 64, 2, 0)
    assert need > 0
    assert _decode(lib, splits=2, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert _decode(lib, B=0) == OK                        # nothing to do, nothing launched


def test_paged_validation_codes():
    lib = kvc.load_library()

    def call(**kw):
        a = dict(bt=FAKE, mb=8, bs=16, nb=10, B=2, h=8, g=2, d=128, splits=1)
        a.update(kw)
        return lib.kvc_decode_attention_paged(FAKE, FAKE, FAKE, a["bt"], a["mb"], a["bs"], a["nb"],
                                              FAKE, a["B"], a["h"], a["g"], a["d"], 0.1, 1,
                                              a["splits"], None, 0, FAKE, FAKE, None)
    assert call(bt=None) == INVALID
    assert call(bs=12) == INVALID      # not a power of two
    assert call(bs=4) == INVALID       # below 8
    assert call(bs=512) == INVALID     # above 256
    assert call(mb=0) == INVALID
    assert call(nb=0) == INVALID
    assert call(h=6, g=4) == INVALID
    assert call(splits=2) == WORKSPACE
    # pool rows (num_blocks * g * block_size) are indexed in 32 bits
    assert call(nb=(1 << 31) - 1, g=2, h=8, bs=16) == UNSUPPORTED
    assert call(nb=(1 << 27) - 1, g=2, h=8, bs=16, splits=2) == WORKSPACE  # 2^32 - 32 rows: accepted


def test_append_validation_codes():
    lib = kvc.load_library()
    f = lib.kvc_append
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 0, 128, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 2, 128, 0, 1, None) == INVALID
    assert f(None, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 2, 128, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, FAKE, 2, 2, 128, 64, 1, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 2, 128, 64, 9, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 0, 2, 128, 64, 1, None) == OK


def test_python_binding_refuses_cpu_tensors():
    w = W.WORKLOADS["tiny_gqa_f32"]
    x = W.make_contiguous(w)
    with pytest.raises(ValueError):
        kvc.decode(x["q"], x["k_cache"], x["v_cache"], x["seq_lens_after"])


def test_fused_validation_codes():
    lib = kvc.load_library()
    f = lib.kvc_append_decode_attention
    # every call below fails validation (or has B = 0) before any HIP call
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 1, None, 0, FAKE, FAKE, None]
    bad = list(args); bad[1] = None                  # k_new missing
    assert f(*bad) == INVALID
    bad = list(args); bad[2] = None                  # v_new missing
    assert f(*bad) == INVALID
    bad = list(args); bad[8] = 3                     # h % g != 0
    assert f(*bad) == INVALID
    bad = list(args); bad[13] = 2                    # a split plan needs a workspace
    assert f(*bad) == WORKSPACE
    bad = list(args); bad[6] = 0                     # nothing to do
    assert f(*bad) == OK
    fp = lib.kvc_append_decode_attention_paged
    pargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 0.1, 1, 1, None, 0,
             FAKE, FAKE, None]
    bad = list(pargs); bad[1] = None
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[7] = 12                   # block size not a power of two
    assert fp(*bad) == INVALID


def test_multi_validation_codes():
    lib = kvc.load_library()
    f = lib.kvc_decode_attention_multi
    # every call below fails validation before any HIP call
    args = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 4, 64, 0.1, 1, 1, None, 0, FAKE, FAKE, None]
    bad = list(args); bad[8] = 0                     # n = 0
    assert f(*bad) == INVALID
    bad = list(args); bad[8] = 10000                 # h * n > 65535
    assert f(*bad) == UNSUPPORTED
    bad = list(args); bad[12] = 2                    # split plan needs a workspace
    assert f(*bad) == WORKSPACE
    fa = lib.kvc_append_decode_attention_multi
    aargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 4, 64, 0.1, 1, 1, None, 0, FAKE,
             FAKE, None]
    bad = list(aargs); bad[1] = None                 # k_new missing
    assert fa(*bad) == INVALID
    bad = list(aargs); bad[10] = -1                  # n < 1
    assert fa(*bad) == INVALID
    fp = lib.kvc_decode_attention_multi_paged
    pargs = [FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 4, 0.1, 1, 1, None, 0, FAKE,
             FAKE, None]
    bad = list(pargs); bad[12] = 0                   # n = 0
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[3] = None                 # no block table
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[5] = 12                   # block size not a power of two
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[15] = 2                   # split plan needs a workspace
    assert fp(*bad) == WORKSPACE
    fap = lib.kvc_append_decode_attention_multi_paged
    apargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 4, 0.1, 1, 1,
              None, 0, FAKE, FAKE, None]
    bad = list(apargs); bad[2] = None                # v_new missing
    assert fap(*bad) == INVALID
    bad = list(apargs); bad[14] = 0                  # n = 0
    assert fap(*bad) == INVALID
    # the workspace of a multi call is that of h * n query rows
    need = lib.kvc_decode_workspace_bytes(2, 8 * 4, 2, 128, 1, 64, 2, 0)
    assert need > lib.kvc_decode_workspace_bytes(2, 8, 2, 128, 1, 64, 2, 0) > 0


def test_window_validation_codes():
    lib = kvc.load_library()
    f = lib.kvc_decode_attention_window
    # every call below fails validation before any HIP call
    args = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 2, 64, 10, 1, 0.1, 1, 1, None, 0, FAKE, FAKE,
            None]
    bad = list(args); bad[10] = 0                    # ring without a window
    assert f(*bad) == INVALID
    bad = list(args); bad[10] = 64                   # window + n - 1 > t_cap
    assert f(*bad) == INVALID
    bad = list(args); bad[10] = -3                   # negative window
    assert f(*bad) == INVALID
    # split plan without a workspace (window 60 + n - 1 = 61 positions: two chunks)
    assert lib.kvc_decode_workspace_bytes(2, 16, 2, 128, 1, 61, 2, 0) > 0
    bad = list(args); bad[10] = 60; bad[11] = 0; bad[14] = 2
    assert f(*bad) == WORKSPACE
    fp = lib.kvc_append_decode_attention_window_paged
    pargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 2, 5, 0.1, 1, 1,
             None, 0, FAKE, FAKE, None]
    bad = list(pargs); bad[15] = -1                  # negative window
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[1] = None                 # k_new missing
    assert fp(*bad) == INVALID
    fwp = lib.kvc_decode_attention_window_paged
    wargs = [FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 2, 5, 0.1, 1, 1, None, 0,
             FAKE, FAKE, None]
    bad = list(wargs); bad[13] = -1                  # negative window
    assert fwp(*bad) == INVALID
    bad = list(wargs); bad[6] = 0                    # empty pool
    assert fwp(*bad) == INVALID
    fwa = lib.kvc_append_decode_attention_window
    waargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 2, 64, 10, 1, 0.1, 1, 1, None, 0,
              FAKE, FAKE, None]
    bad = list(waargs); bad[12] = 0                  # ring without a window
    assert fwa(*bad) == INVALID
    bad = list(waargs); bad[12] = 64                 # window + n - 1 > t_cap
    assert fwa(*bad) == INVALID
    bad = list(waargs); bad[1] = None                # k_new missing
    assert fwa(*bad) == INVALID


def test_block_op_validation_codes():
    lib = kvc.load_library()
    # every call below fails validation (or has nothing to do) before any HIP call
    assert lib.kvc_copy_blocks(FAKE, FAKE, FAKE, 2, 0, 2, 16, 128, 1, None) == INVALID   # no blocks
    assert lib.kvc_copy_blocks(FAKE, FAKE, FAKE, -1, 8, 2, 16, 128, 1, None) == INVALID
    assert lib.kvc_copy_blocks(FAKE, FAKE, FAKE, 2, 8, 2, 16, 128, 5, None) == UNSUPPORTED
    assert lib.kvc_copy_blocks(None, FAKE, FAKE, 2, 8, 2, 16, 128, 1, None) == INVALID
    assert lib.kvc_copy_blocks(FAKE, FAKE, None, 0, 8, 2, 16, 128, 1, None) == OK     # no pairs
    f = lib.kvc_fork_block_tables
    assert f(FAKE, FAKE, 0, 4, FAKE, 2, FAKE, FAKE, None) == INVALID                  # B_src = 0
    assert f(FAKE, FAKE, 2, 4, FAKE, 2, FAKE, FAKE, None) == INVALID                  # aliasing
    assert f(FAKE, FAKE, 2, 4, FAKE, 0, None, None, None) == OK
    gc = lib.kvc_gather_cache
    other = ctypes.c_void_p(0x2000)
    assert gc(FAKE, FAKE, FAKE, 2, FAKE, 2, other, other, 2, 64, 128, 1, None) == INVALID  # aliasing
    assert gc(FAKE, other, FAKE, 2, FAKE, 2, FAKE, other, 2, 64, 128, 1, None) == INVALID
    assert gc(FAKE, FAKE, FAKE, 2, FAKE, 2, other, other, 2, 0, 128, 1, None) == INVALID   # t_cap = 0


def test_fp8_validation_codes():
    lib = kvc.load_library()
    # every call below fails validation (or has nothing to do) before any HIP call
    ap = lib.kvc_append_fp8
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 2, 128, 64, None]
    bad = list(args); bad[4] = None                  # k_scale missing
    assert ap(*bad) == INVALID
    bad = list(args); bad[5] = None                  # v_scale missing
    assert ap(*bad) == INVALID
    bad = list(args); bad[13] = 0                    # no capacity
    assert ap(*bad) == INVALID
    bad = list(args); bad[6] = FAKE                  # table without max_blocks / block_size
    assert ap(*bad) == INVALID
    ok = list(args); ok[10] = 0                      # B = 0: nothing to do
    assert ap(*ok) == OK
    dc = lib.kvc_decode_attention_fp8
    dargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, None, 0, FAKE, FAKE,
             None]
    bad = list(dargs); bad[3] = None
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[7] = 7                    # h not a multiple of g
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[12] = 2                   # a split plan needs a workspace
    bad[10] = 4096
    assert dc(*bad) == WORKSPACE
    dp = lib.kvc_decode_attention_fp8_paged
    pargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 0.1, 1, None, 0,
             FAKE, FAKE, None]
    bad = list(pargs); bad[4] = None
    assert dp(*bad) == INVALID
    bad = list(pargs); bad[7] = 0                    # block size 0
    assert dp(*bad) == INVALID
    fc = lib.kvc_append_decode_attention_fp8
    fargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, None, 0,
             FAKE, FAKE, None]
    for i in (1, 2, 5, 6):                           # k_new, v_new, k_scale, v_scale
        bad = list(fargs); bad[i] = None
        assert fc(*bad) == INVALID
    fpp = lib.kvc_append_decode_attention_fp8_paged
    fpargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 0.1,
              1, None, 0, FAKE, FAKE, None]
    for i in (1, 2, 5, 6):
        bad = list(fpargs); bad[i] = None
        assert fpp(*bad) == INVALID


def test_fp8_planning_dtype_plans_like_bf16():
    """KVC_FP8_E4M3 in the planning queries (FP8 caches with a scale per KV
    head): the workspaces of bf16, and its plans, the same kernel families,
    except that a paged bf16 pool at d = 256 with at most 16 rows per KV head
    streams the multi-row kernel automatically and an FP8 one does not (it
    was not faster there)."""
    lib = kvc.load_library()
    for shape in [(32, 64, 8, 128, 4112, 0, 0), (64, 32, 8, 128, 8208, 0, 1), (4, 32, 1, 128, 131088, 64, 0),
                  (3, 8, 2, 128, 5000, 3, 1), (2, 8, 2, 64, 100, -1, 0), (8, 64, 8, 256, 4096, 0, 0),
                  (8, 256, 8, 256, 4096, 0, 1), (8, 64, 8, 256, 4096, -1, 1)]:
        B, h, g, d, L, ns, paged = shape
        assert kvc.plan(B, h, g, d, L, ns, dtype="fp8", paged=bool(paged)) == \
            kvc.plan(B, h, g, d, L, ns, dtype=torch.bfloat16, paged=bool(paged))
        assert kvc.workspace_bytes(B, h, g, d, L, ns, dtype="fp8", paged=bool(paged)) == \
            kvc.workspace_bytes(B, h, g, d, L, ns, dtype=torch.bfloat16, paged=bool(paged))
    assert kvc.plan(8, 64, 8, 256, 4096, 0, dtype=torch.bfloat16, paged=True)[0] == "stream"
    assert kvc.plan(8, 64, 8, 256, 4096, 0, dtype="fp8", paged=True)[0] == "auto_chunks"
    assert kvc.workspace_bytes(8, 64, 8, 256, 4096, 0, dtype="fp8", paged=True) == \
        kvc.workspace_bytes(8, 64, 8, 256, 4096, 0, dtype=torch.bfloat16, paged=True)
    assert lib.kvc_decode_plan(2, 8, 2, 128, 3, 64, 0, 0, None, None, None) == UNSUPPORTED


def test_public_calls_carry_the_device_guard():
    """Every binding call that takes tensors runs with the device of its
    first GPU tensor made current (and rejects tensors of another device)."""
    for name in ["append", "decode", "decode_paged", "append_decode", "decode_multi",
                 "append_decode_multi", "decode_window", "copy_blocks", "fork_block_tables",
                 "gather_cache", "append_fp8", "decode_fp8", "decode_fp8_window",
                 "append_decode_noalloc", "append_fp8_block_scaled", "decode_fp8_block_scaled"]:
        fn = getattr(kvc, name)
        assert hasattr(fn, "__wrapped__"), name
        assert name in kvc.__all__, name


def test_misaligned_pointers_are_rejected_before_any_hip_call():
    """Element tensors must be 16-byte aligned, int32/float32 arrays 4-byte
    aligned; anything else is KVC_ERR_INVALID (the pointers are never
    dereferenced: validation fails first)."""
    lib = kvc.load_library()
    off8 = ctypes.c_void_p(0x1008)   # 8-byte aligned, not 16
    off2 = ctypes.c_void_p(0x1002)   # 2-byte aligned, not 4
    for i in (0, 1, 2, 14):          # q, k_cache, v_cache, out
        bad = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 1, None, 0, FAKE, FAKE, None]
        bad[i] = off8
        assert lib.kvc_decode_attention(*bad) == INVALID, i
    for i in (3, 15):                # seq_lens, lse
        bad = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 1, None, 0, FAKE, FAKE, None]
        bad[i] = off2
        assert lib.kvc_decode_attention(*bad) == INVALID, i
    # the workspace of a split plan
    need = lib.kvc_decode_workspace_bytes(2, 8, 2, 128, 1, 64, 2, 0)
    args = [FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 2, off8, need, FAKE, FAKE, None]
    assert lib.kvc_decode_attention(*args) == INVALID
    # k_new / v_new of the one-call step
    fargs = [FAKE, off8, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 1, None, 0, FAKE, FAKE,
             None]
    assert lib.kvc_append_decode_attention(*fargs) == INVALID
    # the block table of a paged call
    assert lib.kvc_decode_attention_paged(FAKE, FAKE, FAKE, off2, 8, 16, 10, FAKE, 2, 8, 2, 128,
                                          0.1, 1, 1, None, 0, FAKE, FAKE, None) == INVALID
    # FP8 scales
    assert lib.kvc_decode_attention_fp8(FAKE, FAKE, FAKE, off2, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1,
                                        1, None, 0, FAKE, FAKE, None) == INVALID
    # append, block copies, forks, gathers
    assert lib.kvc_append(FAKE, FAKE, off8, FAKE, None, 0, 0, FAKE, 2, 2, 128, 64, 1,
                          None) == INVALID
    assert lib.kvc_append(FAKE, FAKE, FAKE, FAKE, None, 0, 0, off2, 2, 2, 128, 64, 1,
                          None) == INVALID
    assert lib.kvc_append_fp8(off8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0, FAKE, 2, 2, 128, 64,
                              None) == INVALID
    assert lib.kvc_copy_blocks(off8, FAKE, FAKE, 2, 8, 2, 16, 128, 1, None) == INVALID
    assert lib.kvc_copy_blocks(FAKE, FAKE, off2, 2, 8, 2, 16, 128, 1, None) == INVALID
    other = ctypes.c_void_p(0x2000)
    assert lib.kvc_fork_block_tables(FAKE, FAKE, 2, 4, off2, 2, other, ctypes.c_void_p(0x3000),
                                     None) == INVALID
    assert lib.kvc_gather_cache(FAKE, FAKE, FAKE, 2, FAKE, 2, other, off8, 2, 64, 128, 1,
                                None) == INVALID


def test_noalloc_validation_codes():
    """kvc_append_decode_attention_noalloc validates like the workspace entry
    point and rejects a split beyond its static scratch (KVC_ERR_SCRATCH)
    before any HIP call."""
    lib = kvc.load_library()
    f = lib.kvc_append_decode_attention_noalloc
    assert lib.kvc_noalloc_scratch_bytes() == 16 << 20
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 64, 0.1, 1, 1, FAKE, FAKE, None]
    bad = list(args); bad[1] = None                  # k_new missing
    assert f(*bad) == INVALID
    bad = list(args); bad[8] = 3                     # h % g != 0
    assert f(*bad) == INVALID
    bad = list(args); bad[0] = ctypes.c_void_p(0x1008)  # misaligned q
    assert f(*bad) == INVALID
    ok = list(args); ok[6] = 0                       # nothing to do
    assert f(*ok) == OK
    # 8 x 32 query rows over 131088 positions in 200 chunks: more than 16 MiB
    # of partials
    assert lib.kvc_decode_workspace_bytes(8, 32, 1, 128, 1, 131088, 200, 0) > 16 << 20
    big = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 1, 128, 131088, 0.1, 1, 200, FAKE, FAKE, None]
    assert f(*big) == 5
    assert lib.kvc_status_string(5).startswith(b"the call needs more split scratch")


def test_fp8_multi_window_validation_codes():
    """The FP8 multi-token and window calls validate like the bf16 ones,
    plus the scales, before any HIP call."""
    lib = kvc.load_library()
    f = lib.kvc_decode_attention_fp8_window
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 2, 64, 10, 1, 0.1, 1, None, 0, FAKE,
            FAKE, None]
    bad = list(args); bad[3] = None                  # k_scale missing
    assert f(*bad) == INVALID
    bad = list(args); bad[12] = 0                    # ring without a window
    assert f(*bad) == INVALID
    bad = list(args); bad[12] = 64                   # window + n - 1 > t_cap
    assert f(*bad) == INVALID
    bad = list(args); bad[10] = 0                    # n = 0
    assert f(*bad) == INVALID
    fm = lib.kvc_append_decode_attention_fp8_multi
    margs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 128, 4, 64, 0.1, 1, None, 0,
             FAKE, FAKE, None]
    for i in (1, 2, 5, 6):                           # k_new, v_new, k_scale, v_scale
        bad = list(margs); bad[i] = None
        assert fm(*bad) == INVALID
    bad = list(margs); bad[15] = 2                   # split plan without a workspace
    assert fm(*bad) == WORKSPACE
    fp = lib.kvc_append_decode_attention_fp8_window_paged
    pargs = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 2, 5,
             0.1, 1, None, 0, FAKE, FAKE, None]
    bad = list(pargs); bad[17] = -1                  # negative window
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[9] = 12                   # block size not a power of two
    assert fp(*bad) == INVALID
    bad = list(pargs); bad[6] = ctypes.c_void_p(0x1002)  # misaligned k_scale
    assert fp(*bad) == INVALID


def test_fp8_block_scaled_validation_codes():
    lib = kvc.load_library()
    ap = lib.kvc_append_fp8_paged_block_scaled
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 2, 128, 1, None]
    for i in (0, 1, 4, 5, 6, 10):                    # null data, scales, table, lengths
        bad = list(args); bad[i] = None
        assert ap(*bad) == INVALID, i
    bad = list(args); bad[14] = 0                    # n = 0
    assert ap(*bad) == INVALID
    bad = list(args); bad[9] = 0                     # empty pool
    assert ap(*bad) == INVALID
    ok = list(args); ok[11] = 0                      # B = 0: nothing to do
    assert ap(*ok) == OK
    dc = lib.kvc_decode_attention_fp8_paged_block_scaled
    dargs = [FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 10, FAKE, 2, 8, 2, 128, 1, 0,
             0.1, 1, None, 0, FAKE, FAKE, None]
    bad = list(dargs); bad[5] = None                 # k_scale missing
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[1] = FAKE                 # k_new without v_new
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[9] = 12                   # block size not a power of two
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[17] = -1                  # negative window
    assert dc(*bad) == INVALID
    bad = list(dargs); bad[19] = 2                   # a split plan needs a workspace
    assert dc(*bad) == WORKSPACE


def test_workspace_query_covers_fp8_plans():
    """One workspace query serves bf16 and FP8 caches (the FP8 calls size
    with KVC_BF16 or KVC_FP8_E4M3), per-block FP8 scales included.  At head
    dims 64 and 256 those take the generic kernel while bf16 takes the
    multi-row one, and the generic plan has more chunks: the query must cover
    its partial rows (the generic plan is the one an fp32 query reports)."""
    for (B, h, g, d, T) in [(64, 32, 8, 64, 4096), (32, 64, 8, 256, 8192), (256, 8, 8, 64, 2048),
                            (6, 6, 2, 64, 4100)]:
        for paged in (False, True):
            mode, _, chunks = kvc.plan(B, h, g, d, T, 0, dtype=torch.float32, paged=paged)
            assert mode == "chunks", (B, h, g, d, mode)
            assert kvc.plan(B, h, g, d, T, 0, dtype=torch.bfloat16, paged=paged)[0] == (
                "stream" if paged and d == 256 and h // g <= 16 else "auto_chunks")
            rows = B * h * chunks if chunks > 1 else 0
            need = rows * d * 4 + rows * 4
            for dt in (torch.bfloat16, kvc.FP8_E4M3):
                ws = kvc.workspace_bytes(B, h, g, d, T, 0, dtype=dt, paged=paged)
                assert ws >= need, (B, h, g, d, paged, dt, ws, need)
