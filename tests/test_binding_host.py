"""Host-only checks of the Python binding: every public call compares the
shapes of its tensors with each other and raises ValueError on a mismatch
before any pointer reaches the library (CPU tensors are enough: the shape
checks come before the device checks)."""
from __future__ import annotations

import os

import pytest
import torch

import kv_cache_gqa_amd as kvc

pytestmark = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH),
                                reason="libkvc.so not built (run __graft_entry__.build())")

B, H, G, D, T = 2, 8, 2, 128, 64
bf = torch.bfloat16


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def contig():
    return dict(q=z(B, H, D), k=z(B, G, T, D), v=z(B, G, T, D), sl=i32(B))


def bad_shape(fn, *a, **kw):
    with pytest.raises(ValueError, match="shape"):
        fn(*a, **kw)


def test_decode_shape_mismatches():
    c = contig()
    bad_shape(kvc.decode, c["q"], z(B + 1, G, T, D), c["v"], c["sl"])        # cache batch
    bad_shape(kvc.decode, c["q"], z(B, G, T, 64), c["v"], c["sl"])           # cache head dim
    bad_shape(kvc.decode, c["q"], c["k"], z(B, G, T + 1, D), c["sl"])        # v differs from k
    bad_shape(kvc.decode, c["q"], c["k"], c["v"], i32(B + 1))                # seq_lens
    bad_shape(kvc.decode, c["q"], c["k"], c["v"], c["sl"], out=z(B, H, D + 1, dtype=torch.float32))
    bad_shape(kvc.decode, c["q"], c["k"], c["v"], c["sl"], lse=z(B, H + 1, dtype=torch.float32))
    bad_shape(kvc.decode, z(B, H, D, 1), c["k"], c["v"], c["sl"])            # q rank


def test_paged_shape_mismatches():
    q, kp, vp, bt, sl = z(B, H, D), z(10, G, 16, D), z(10, G, 16, D), i32(B, 4), i32(B)
    bad_shape(kvc.decode_paged, q, kp, z(10, G, 16, D + 8), bt, sl)
    bad_shape(kvc.decode_paged, q, kp, vp, i32(B + 1, 4), sl)                 # table rows
    bad_shape(kvc.decode_paged, q, z(10, G, 16, 64), z(10, G, 16, 64), bt, sl)
    bad_shape(kvc.decode_paged, q, kp, vp, bt, i32(3))


def test_append_shape_mismatches():
    c = contig()
    kn, vn = z(B, G, D), z(B, G, D)
    bad_shape(kvc.append, kn, z(B, G, D + 1), c["k"], c["v"], c["sl"])
    bad_shape(kvc.append, kn, vn, z(B + 1, G, T, D), z(B + 1, G, T, D), c["sl"])
    bad_shape(kvc.append, kn, vn, c["k"], c["v"], i32(B + 2))
    with pytest.raises(ValueError, match="KV heads"):
        kvc.append(kn, vn, z(B, G + 1, T, D), z(B, G + 1, T, D), c["sl"])
    bad_shape(kvc.append_decode, c["q"], z(B, G + 1, D), vn, c["k"], c["v"], c["sl"])
    bad_shape(kvc.append_decode, c["q"], kn, vn, c["k"], c["v"], c["sl"],
              block_table=i32(B + 1, 4))


def test_multi_and_window_shape_mismatches():
    c = contig()
    n = 3
    q = z(B, H, n, D)
    kn, vn = z(B, G, n, D), z(B, G, n, D)
    bad_shape(kvc.append_decode_multi, q, z(B, G, n + 1, D), vn, c["k"], c["v"], c["sl"])
    bad_shape(kvc.decode_multi, q, c["k"], c["v"], c["sl"], out=z(B, H, D, dtype=torch.float32))
    bad_shape(kvc.decode_multi, q, c["k"], c["v"], c["sl"], lse=z(B, H, dtype=torch.float32))
    bad_shape(kvc.decode_window, q, c["k"], c["v"], c["sl"], 16, k_new=kn, v_new=z(B, G, n, 64))
    bad_shape(kvc.decode_window, q, c["k"], c["v"], i32(1), 16)
    with pytest.raises(ValueError, match="ring"):
        kvc.decode_window(q, c["k"], c["v"], c["sl"], 16, ring=True, block_table=i32(B, 4))


def test_fp8_and_block_op_shape_mismatches():
    q, sl = z(B, H, D), i32(B)
    kc = torch.zeros((B, G, T, D), dtype=torch.uint8)
    sc = torch.ones(G, dtype=torch.float32)
    bad_shape(kvc.decode_fp8, q, kc, kc, torch.ones(G + 1), sc, sl)
    bad_shape(kvc.decode_fp8, q, kc, kc, sc, sc, sl, k_new=z(B, G, D), v_new=z(B, G + 1, D))
    bad_shape(kvc.append_fp8, z(B, G, D), z(B, G, D), kc, kc, sc, torch.ones(1), sl)
    kp = z(10, G, 16, D)
    bad_shape(kvc.copy_blocks, kp, z(11, G, 16, D), i32(3, 2))
    bad_shape(kvc.copy_blocks, kp, kp, i32(3, 3))
    bad_shape(kvc.fork_block_tables, i32(4, 8), i32(5), i32(2))
    src = z(B, G, T, D)
    bad_shape(kvc.gather_cache, src, src, i32(B), i32(3), z(3, G, T + 1, D), z(3, G, T + 1, D))
    bad_shape(kvc.gather_cache, src, src, i32(B + 1), i32(3), z(3, G, T, D), z(3, G, T, D))
