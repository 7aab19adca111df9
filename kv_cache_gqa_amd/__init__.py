"""kv_cache_gqa_amd -- single-token decode attention over a KV cache on AMD
MI355X (gfx950).

A thin ctypes binding over ``libkvc.so`` (the C ABI in ``include/kvc.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor properties and passes device pointers, sizes and the
current HIP stream.  PyTorch provides device memory and streams.

    append(k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None)
    out, lse = decode(q, k_cache, v_cache, seq_lens, scale=None, num_splits=0)
    out, lse = decode_paged(q, k_pool, v_pool, block_table, seq_lens, ...)

There is no CPU fallback: without the built library (``python -m
kv_cache_gqa_amd.build``) or without a GPU every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["append", "decode", "decode_paged", "append_decode", "decode_multi",
           "append_decode_multi", "decode_window", "append_fp8", "decode_fp8", "decode_fp8_window",
           "append_decode_noalloc", "append_fp8_block_scaled", "decode_fp8_block_scaled",
           "copy_blocks",
           "fork_block_tables", "gather_cache", "plan", "workspace_bytes", "launch_shape",
           "plan_multi", "launch_shape_multi",
           "KvcError", "load_library", "LIB_PATH", "F32", "BF16", "FP8_E4M3", "SPLITS_STREAM"]

# KVC_LIB names another build of the library (the sanitizer test loads one
# whose host code is built with AddressSanitizer and UBSan).
LIB_PATH = os.environ.get("KVC_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libkvc.so")
F32, BF16 = 0, 1
SPLITS_STREAM = -1  # num_splits value that asks for the stream split
_MODES = {0: "chunks", 1: "stream", 2: "auto_chunks"}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype or shape",
           3: "workspace missing or too small", 4: "HIP launch error",
           5: "split needs more than the library's static scratch"}

_lib = None


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


def load_library():
    """Load libkvc.so and declare its C signatures.  Raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m kv_cache_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ip, fp, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kvc_version.argtypes = []
    lib.kvc_version.restype = ip
    lib.kvc_status_string.argtypes = [ip]
    lib.kvc_status_string.restype = ctypes.c_char_p
    lib.kvc_append.argtypes = [vp, vp, vp, vp, vp, ip, ip, vp, ip, ip, ip, ip, ip, vp]
    lib.kvc_append.restype = ip
    lib.kvc_decode_plan.argtypes = [ip, ip, ip, ip, ip, ip, ip, ip, ctypes.POINTER(ip),
                                    ctypes.POINTER(ip), ctypes.POINTER(ip)]
    lib.kvc_decode_plan.restype = ip
    lib.kvc_decode_workspace_bytes.argtypes = [ip, ip, ip, ip, ip, ip, ip, ip]
    lib.kvc_decode_workspace_bytes.restype = sz
    lib.kvc_decode_launch_shape.argtypes = [ip] * 8 + [ctypes.POINTER(ip)] * 4
    lib.kvc_decode_launch_shape.restype = ip
    lib.kvc_decode_plan_multi.argtypes = [ip] * 10 + [ctypes.POINTER(ip)] * 3
    lib.kvc_decode_plan_multi.restype = ip
    lib.kvc_decode_launch_shape_multi.argtypes = [ip] * 10 + [ctypes.POINTER(ip)] * 4
    lib.kvc_decode_launch_shape_multi.restype = ip
    lib.kvc_append_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, fp, ip,
                                                ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention.restype = ip
    lib.kvc_append_decode_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip,
                                                        fp, ip, ip, vp, vp, vp]
    lib.kvc_append_decode_attention_noalloc.restype = ip
    lib.kvc_noalloc_scratch_bytes.argtypes = []
    lib.kvc_noalloc_scratch_bytes.restype = sz
    lib.kvc_append_decode_attention_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, vp, ip,
                                                      ip, ip, ip, fp, ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_paged.restype = ip
    lib.kvc_decode_attention_multi.argtypes = [vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, fp, ip, ip,
                                               vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_multi.restype = ip
    lib.kvc_decode_attention_multi_paged.argtypes = [vp, vp, vp, vp, ip, ip, ip, vp, ip, ip, ip,
                                                     ip, ip, fp, ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_multi_paged.restype = ip
    lib.kvc_append_decode_attention_multi.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip,
                                                      ip, fp, ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_multi.restype = ip
    lib.kvc_append_decode_attention_multi_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip,
                                                            vp, ip, ip, ip, ip, ip, fp, ip, ip,
                                                            vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_multi_paged.restype = ip
    lib.kvc_decode_attention_window.argtypes = [vp, vp, vp, vp, ip, ip, ip, ip, ip, ip, ip, ip, fp,
                                                ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_window.restype = ip
    lib.kvc_decode_attention_window_paged.argtypes = [vp, vp, vp, vp, ip, ip, ip, vp, ip, ip, ip,
                                                      ip, ip, ip, fp, ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_window_paged.restype = ip
    lib.kvc_append_decode_attention_window.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip,
                                                       ip, ip, ip, fp, ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_window.restype = ip
    lib.kvc_append_decode_attention_window_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip,
                                                             vp, ip, ip, ip, ip, ip, ip, fp, ip,
                                                             ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_window_paged.restype = ip
    lib.kvc_append_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, ip, ip, vp, ip, ip, ip, ip, vp]
    lib.kvc_append_fp8.restype = ip
    lib.kvc_decode_attention_fp8.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, fp, ip, vp,
                                             sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8.restype = ip
    lib.kvc_decode_attention_fp8_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, vp, ip, ip,
                                                   ip, ip, fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8_paged.restype = ip
    lib.kvc_append_decode_attention_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, ip, ip,
                                                    ip, fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_fp8.restype = ip
    lib.kvc_append_decode_attention_fp8_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, ip,
                                                          ip, vp, ip, ip, ip, ip, fp, ip, vp, sz,
                                                          vp, vp, vp]
    lib.kvc_append_decode_attention_fp8_paged.restype = ip
    # FP8 multi-token / window calls
    lib.kvc_decode_attention_fp8_multi.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, ip,
                                                   fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8_multi_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, vp, ip,
                                                         ip, ip, ip, ip, fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_fp8_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, ip,
                                                          ip, ip, ip, fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_append_decode_attention_fp8_multi_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip,
                                                                ip, ip, vp, ip, ip, ip, ip, ip, fp,
                                                                ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8_window.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip, ip,
                                                    ip, ip, fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8_window_paged.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, vp,
                                                          ip, ip, ip, ip, ip, ip, fp, ip, vp, sz,
                                                          vp, vp, vp]
    lib.kvc_append_decode_attention_fp8_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, ip,
                                                           ip, ip, ip, ip, ip, ip, fp, ip, vp, sz,
                                                           vp, vp, vp]
    lib.kvc_append_decode_attention_fp8_window_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                                                 ip, ip, ip, vp, ip, ip, ip, ip,
                                                                 ip, ip, fp, ip, vp, sz, vp, vp,
                                                                 vp]
    for name in ("kvc_decode_attention_fp8_multi", "kvc_decode_attention_fp8_multi_paged",
                 "kvc_append_decode_attention_fp8_multi",
                 "kvc_append_decode_attention_fp8_multi_paged", "kvc_decode_attention_fp8_window",
                 "kvc_decode_attention_fp8_window_paged", "kvc_append_decode_attention_fp8_window",
                 "kvc_append_decode_attention_fp8_window_paged"):
        getattr(lib, name).restype = ip
    lib.kvc_append_fp8_paged_block_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, ip, ip, ip, vp,
                                                      ip, ip, ip, ip, vp]
    lib.kvc_append_fp8_paged_block_scaled.restype = ip
    lib.kvc_decode_attention_fp8_paged_block_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip,
                                                                ip, ip, vp, ip, ip, ip, ip, ip, ip,
                                                                fp, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_fp8_paged_block_scaled.restype = ip
    lib.kvc_copy_blocks.argtypes = [vp, vp, vp, ip, ip, ip, ip, ip, ip, vp]
    lib.kvc_copy_blocks.restype = ip
    lib.kvc_fork_block_tables.argtypes = [vp, vp, ip, ip, vp, ip, vp, vp, vp]
    lib.kvc_fork_block_tables.restype = ip
    lib.kvc_gather_cache.argtypes = [vp, vp, vp, ip, vp, ip, vp, vp, ip, ip, ip, ip, vp]
    lib.kvc_gather_cache.restype = ip
    lib.kvc_decode_attention.argtypes = [vp, vp, vp, vp, ip, ip, ip, ip, ip, fp, ip, ip, vp, sz,
                                         vp, vp, vp]
    lib.kvc_decode_attention.restype = ip
    lib.kvc_decode_attention_paged.argtypes = [vp, vp, vp, vp, ip, ip, ip, vp, ip, ip, ip, ip, fp,
                                               ip, ip, vp, sz, vp, vp, vp]
    lib.kvc_decode_attention_paged.restype = ip
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _on_device(fn):
    """Run fn with the device of its first GPU tensor argument current, so
    that the library's launches and device queries and the default stream
    (torch's current stream) belong to the device that holds the data.  When
    the caller names a stream, fn also runs with that stream current, so
    that the tensors it allocates (out, lse, the workspace) belong to the
    stream the kernels use: the caching allocator then reuses them only
    after that stream's work."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def run(*args, **kw):
        for a in list(args) + list(kw.values()):
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    stream = sig.bind_partial(*args, **kw).arguments.get("stream")
                    if stream is None:
                        return fn(*args, **kw)
                    if not isinstance(stream, torch.cuda.Stream):
                        stream = torch.cuda.ExternalStream(int(stream), device=a.device)
                    with torch.cuda.stream(stream):
                        return fn(*args, **kw)
        return fn(*args, **kw)
    return run


def _shape(t, shape, name: str):
    """Raise ValueError unless tensor t has the given shape (None: any size)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dim() != len(shape) or any(e is not None and int(x) != int(e)
                                    for x, e in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    return tuple(int(x) for x in t.shape)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the call runs on cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int):
    if status != 0:
        raise KvcError(fn, status)


FP8_E4M3 = 2  # planning queries only: bf16 queries over an FP8 E4M3 cache


def _code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if dtype in ("fp8", "fp8_e4m3", torch.float8_e4m3fn):
        return FP8_E4M3
    return BF16 if dtype in (torch.bfloat16, "bf16") else F32


def plan(B: int, h: int, g: int, d: int, max_seq_len: int, num_splits: int = 0,
         dtype=torch.bfloat16, paged: bool = False) -> Tuple[str, int, int]:
    """(mode, chunk_len, num_chunks) of the split: mode "chunks" (chunk fields
    set), "auto_chunks" (count chosen at launch) or "stream"."""
    lib = load_library()
    mode, cl, nc = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check("kvc_decode_plan", lib.kvc_decode_plan(B, h, g, d, _code(dtype), max_seq_len, num_splits,
                                                  int(paged), ctypes.byref(mode), ctypes.byref(cl),
                                                  ctypes.byref(nc)))
    return _MODES[mode.value], cl.value, nc.value


def workspace_bytes(B: int, h: int, g: int, d: int, max_seq_len: int, num_splits: int = 0,
                    dtype=torch.bfloat16, paged: bool = False) -> int:
    return int(load_library().kvc_decode_workspace_bytes(B, h, g, d, _code(dtype), max_seq_len,
                                                         num_splits, int(paged)))


def launch_shape(B: int, h: int, g: int, d: int, max_seq_len: int, num_splits: int = 0,
                 dtype=torch.bfloat16, paged: bool = False) -> Tuple[int, int, int, int]:
    """(waves per work-group, work-groups, chunk_len, num_chunks) of the decode
    launch on the current device (chunk fields 0 in stream mode)."""
    lib = load_library()
    out = [ctypes.c_int(0) for _ in range(4)]
    _check("kvc_decode_launch_shape",
           lib.kvc_decode_launch_shape(B, h, g, d, _code(dtype), max_seq_len, num_splits, int(paged),
                                       *(ctypes.byref(x) for x in out)))
    return tuple(x.value for x in out)


def plan_multi(B: int, h: int, g: int, d: int, n: int, capacity: int, window: int = 0,
               num_splits: int = 0, dtype=torch.bfloat16, paged: bool = False) -> Tuple[str, int, int]:
    """plan() of a call with n query tokens per sequence and a sliding window
    (0 = none): h is query heads, capacity t_cap or max_blocks * block_size."""
    lib = load_library()
    mode, cl, nc = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check("kvc_decode_plan_multi",
           lib.kvc_decode_plan_multi(B, h, g, d, n, window, _code(dtype), capacity, num_splits,
                                     int(paged), ctypes.byref(mode), ctypes.byref(cl),
                                     ctypes.byref(nc)))
    return _MODES[mode.value], cl.value, nc.value


def launch_shape_multi(B: int, h: int, g: int, d: int, n: int, capacity: int, window: int = 0,
                       num_splits: int = 0, dtype=torch.bfloat16,
                       paged: bool = False) -> Tuple[int, int, int, int]:
    """launch_shape() of a call with n query tokens per sequence and a sliding
    window (0 = none): h is query heads, capacity t_cap or max_blocks *
    block_size."""
    lib = load_library()
    out = [ctypes.c_int(0) for _ in range(4)]
    _check("kvc_decode_launch_shape_multi",
           lib.kvc_decode_launch_shape_multi(B, h, g, d, n, window, _code(dtype), capacity,
                                             num_splits, int(paged),
                                             *(ctypes.byref(x) for x in out)))
    return tuple(x.value for x in out)


def _cache_shapes(k_cache, v_cache, B: int, d: int, block_table, names=("k_cache", "v_cache")):
    """Check the cache tensors against the batch and head dim.  Contiguous:
    [B, g, t_cap, d]; paged: pools [NB, g, bs, d] and block_table [B,
    max_blocks].  Returns (g, capacity, block_size, max_blocks, num_blocks);
    capacity is t_cap, or NB for pools."""
    if block_table is None:
        _, g, t_cap, _ = _shape(k_cache, (B, None, None, d), names[0])
        _shape(v_cache, tuple(k_cache.shape), names[1])
        return g, t_cap, 0, 0, 0
    nb, g, bs, _ = _shape(k_cache, (None, None, None, d), names[0].replace("cache", "pool"))
    _shape(v_cache, tuple(k_cache.shape), names[1].replace("cache", "pool"))
    _, mb = _shape(block_table, (B, None), "block_table")
    return g, nb, bs, mb, nb


@_on_device
def append(k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None, stream=None):
    """Write k_new/v_new [B,g,d] at position seq_lens_before[b] of each
    sequence's cache: contiguous [B,g,T,d], or pools [NB,g,bs,d] through
    block_table [B,max_blocks].  In place; seq_lens_before is not changed."""
    lib = load_library()
    dt = _dtype_code(k_cache)
    B, g, d = _shape(k_new, (None, None, None), "k_new")
    _shape(v_new, (B, g, d), "v_new")
    _shape(seq_lens_before, (B,), "seq_lens_before")
    gc, capacity, bs, mb, _ = _cache_shapes(k_cache, v_cache, B, d, block_table)
    if gc != g:
        raise ValueError(f"k_new has {g} KV heads, the cache {gc}")
    bt = _dev(block_table, "block_table", torch.int32) if block_table is not None else None
    st = lib.kvc_append(_dev(k_new, "k_new", k_cache.dtype), _dev(v_new, "v_new", k_cache.dtype),
                        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache", k_cache.dtype),
                        bt, mb, bs, _dev(seq_lens_before, "seq_lens_before", torch.int32),
                        B, g, d, capacity, dt, _stream(stream))
    _check("kvc_append", st)


def _outputs(q, out, lse):
    """out and lse for q [B, h, (n,) d]: out like q in float32, lse without
    the last dim.  Caller-supplied tensors are checked against that."""
    oshape, lshape = tuple(q.shape), tuple(q.shape[:-1])
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=q.device)
    else:
        _shape(out, oshape, "out")
    if lse is None:
        lse = torch.empty(lshape, dtype=torch.float32, device=q.device)
    else:
        _shape(lse, lshape, "lse")
    return out, lse


_outputs_multi = _outputs


def _workspace(nbytes: int, q: torch.Tensor, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def _new_tokens(k_new, v_new, B: int, g: int, n, d: int):
    """k_new, v_new [B, g, d] (n is None) or [B, g, n, d]."""
    shape = (B, g, d) if n is None else (B, g, n, d)
    _shape(k_new, shape, "k_new")
    _shape(v_new, shape, "v_new")


@_on_device
def decode(q, k_cache, v_cache, seq_lens, scale: Optional[float] = None, num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None, out=None, lse=None, stream=None):
    """Decode attention over a contiguous cache.

    q [B,h,d]; k_cache, v_cache [B,g,t_cap,d]; seq_lens int32 [B] (attended
    lengths).  Returns (out [B,h,d] float32, lse [B,h] float32)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, d = _shape(q, (None, None, None), "q")
    g, t_cap, _, _, _ = _cache_shapes(k_cache, v_cache, B, d, None)
    _shape(seq_lens, (B,), "seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, dt, t_cap, num_splits, 0), q,
                         workspace)
    st = lib.kvc_decode_attention(
        _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(seq_lens, "seq_lens", torch.int32), B, h, g, d, t_cap, float(scale), dt, num_splits,
        ws.data_ptr() if ws is not None else None, wsb,
        _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
    _check("kvc_decode_attention", st)
    return out, lse


@_on_device
def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: Optional[float] = None,
                 num_splits: int = 0, workspace: Optional[torch.Tensor] = None, out=None, lse=None,
                 stream=None):
    """Decode attention over a paged cache: pools [NB,g,bs,d], block_table
    int32 [B,max_blocks], seq_lens int32 [B].  Returns (out, lse)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, d = _shape(q, (None, None, None), "q")
    g, _, bs, mb, nb = _cache_shapes(k_pool, v_pool, B, d, block_table)
    _shape(seq_lens, (B,), "seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, dt, mb * bs, num_splits, 1), q,
                         workspace)
    st = lib.kvc_decode_attention_paged(
        _dev(q, "q"), _dev(k_pool, "k_pool", q.dtype), _dev(v_pool, "v_pool", q.dtype),
        _dev(block_table, "block_table", torch.int32), mb, bs, nb,
        _dev(seq_lens, "seq_lens", torch.int32), B, h, g, d, float(scale), dt, num_splits,
        ws.data_ptr() if ws is not None else None, wsb,
        _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
    _check("kvc_decode_attention_paged", st)
    return out, lse


@_on_device
def append_decode(q, k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None,
                  scale: Optional[float] = None, num_splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, out=None, lse=None, stream=None):
    """One decode step in one call: append k_new/v_new [B,g,d] at position
    seq_lens_before[b] of each sequence's cache (contiguous [B,g,t_cap,d], or
    pools [NB,g,bs,d] through block_table [B,max_blocks]) and attend over the
    seq_lens_before[b] + 1 positions.  seq_lens_before is not modified.
    Returns (out [B,h,d] float32, lse [B,h] float32)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, d = _shape(q, (None, None, None), "q")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _new_tokens(k_new, v_new, B, g, None, d)
    _shape(seq_lens_before, (B,), "seq_lens_before")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    kn, vn = _dev(k_new, "k_new", q.dtype), _dev(v_new, "v_new", q.dtype)
    sl = _dev(seq_lens_before, "seq_lens_before", torch.int32)
    if block_table is None:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, dt, cap, num_splits, 0),
                             q, workspace)
        st = lib.kvc_append_decode_attention(
            _dev(q, "q"), kn, vn, _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
            sl, B, h, g, d, cap, float(scale), dt, num_splits,
            ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_append_decode_attention", st)
    else:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, dt, mb * bs, num_splits, 1),
                             q, workspace)
        st = lib.kvc_append_decode_attention_paged(
            _dev(q, "q"), kn, vn, _dev(k_cache, "k_pool", q.dtype), _dev(v_cache, "v_pool", q.dtype),
            _dev(block_table, "block_table", torch.int32), mb, bs, nb, sl, B, h, g, d,
            float(scale), dt, num_splits, ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_append_decode_attention_paged", st)
    return out, lse


@_on_device
def decode_multi(q, k_cache, v_cache, seq_lens, block_table=None, scale: Optional[float] = None,
                 num_splits: int = 0, workspace: Optional[torch.Tensor] = None, out=None, lse=None,
                 stream=None):
    """n query tokens per sequence over a cache that already holds them.

    q [B,h,n,d]; seq_lens int32 [B] = cached length including the n tokens;
    token t sees positions 0 .. seq_lens[b] - n + t.  Contiguous caches
    [B,g,t_cap,d], or pools [NB,g,bs,d] with block_table.  Returns (out
    [B,h,n,d] float32, lse [B,h,n] float32)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, n, d = _shape(q, (None, None, None, None), "q")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _shape(seq_lens, (B,), "seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    sl = _dev(seq_lens, "seq_lens", torch.int32)
    if block_table is None:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt, cap, num_splits, 0),
                             q, workspace)
        st = lib.kvc_decode_attention_multi(
            _dev(q, "q"), _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype), sl,
            B, h, g, d, n, cap, float(scale), dt, num_splits,
            ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_decode_attention_multi", st)
    else:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt, mb * bs, num_splits,
                                                            1), q, workspace)
        st = lib.kvc_decode_attention_multi_paged(
            _dev(q, "q"), _dev(k_cache, "k_pool", q.dtype), _dev(v_cache, "v_pool", q.dtype),
            _dev(block_table, "block_table", torch.int32), mb, bs, nb, sl, B, h, g, d, n,
            float(scale), dt, num_splits, ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_decode_attention_multi_paged", st)
    return out, lse


@_on_device
def append_decode_multi(q, k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None,
                        scale: Optional[float] = None, num_splits: int = 0,
                        workspace: Optional[torch.Tensor] = None, out=None, lse=None, stream=None):
    """Append n new tokens per sequence (k_new, v_new [B,g,n,d]; token t at
    position seq_lens_before[b] + t) and attend with q [B,h,n,d], token t
    seeing positions 0 .. seq_lens_before[b] + t, in one call.  Returns
    (out [B,h,n,d] float32, lse [B,h,n] float32)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, n, d = _shape(q, (None, None, None, None), "q")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _new_tokens(k_new, v_new, B, g, n, d)
    _shape(seq_lens_before, (B,), "seq_lens_before")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    kn, vn = _dev(k_new, "k_new", q.dtype), _dev(v_new, "v_new", q.dtype)
    sl = _dev(seq_lens_before, "seq_lens_before", torch.int32)
    if block_table is None:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt, cap, num_splits, 0),
                             q, workspace)
        st = lib.kvc_append_decode_attention_multi(
            _dev(q, "q"), kn, vn, _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
            sl, B, h, g, d, n, cap, float(scale), dt, num_splits,
            ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_append_decode_attention_multi", st)
    else:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt, mb * bs, num_splits,
                                                            1), q, workspace)
        st = lib.kvc_append_decode_attention_multi_paged(
            _dev(q, "q"), kn, vn, _dev(k_cache, "k_pool", q.dtype), _dev(v_cache, "v_pool", q.dtype),
            _dev(block_table, "block_table", torch.int32), mb, bs, nb, sl, B, h, g, d, n,
            float(scale), dt, num_splits, ws.data_ptr() if ws is not None else None, wsb,
            _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_append_decode_attention_multi_paged", st)
    return out, lse


def _plan_len(capacity: int, window: int, n: int) -> int:
    return min(window + n - 1, capacity) if window > 0 else capacity


@_on_device
def decode_window(q, k_cache, v_cache, seq_lens, window: int, ring: bool = False,
                  block_table=None, scale: Optional[float] = None, num_splits: int = 0,
                  workspace: Optional[torch.Tensor] = None, out=None, lse=None, stream=None,
                  k_new=None, v_new=None):
    """Sliding-window attention for q [B,h,n,d] (n tokens per sequence): the
    token at position x sees positions max(0, x + 1 - window) .. x.

    Without k_new: the tokens are in the cache and seq_lens counts them.  With
    k_new, v_new [B,g,n,d]: seq_lens holds the lengths before the step and
    the call appends them (one launch).  ring: the contiguous cache is a ring
    of t_cap slots (position p in slot p mod t_cap).  Returns (out
    [B,h,n,d] float32, lse [B,h,n] float32)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, n, d = _shape(q, (None, None, None, None), "q")
    if ring and block_table is not None:
        raise ValueError("a ring cache is contiguous")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _shape(seq_lens, (B,), "seq_lens")
    fused = k_new is not None
    if fused:
        _new_tokens(k_new, v_new, B, g, n, d)
    elif v_new is not None:
        raise ValueError("v_new without k_new")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    sl = _dev(seq_lens, "seq_lens", torch.int32)
    kn = _dev(k_new, "k_new", q.dtype) if fused else None
    vn = _dev(v_new, "v_new", q.dtype) if fused else None
    wsp = lambda nbytes: _workspace(nbytes, q, workspace)  # noqa: E731
    if block_table is None:
        ws, wsb = wsp(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt, _plan_len(cap, window, n),
                                                     num_splits, 0))
        wsptr = ws.data_ptr() if ws is not None else None
        kc, vc = _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype)
        if fused:
            st = lib.kvc_append_decode_attention_window(
                _dev(q, "q"), kn, vn, kc, vc, sl, B, h, g, d, n, cap, window, int(ring),
                float(scale), dt, num_splits, wsptr, wsb, _dev(out, "out", torch.float32),
                _dev(lse, "lse", torch.float32), _stream(stream))
        else:
            st = lib.kvc_decode_attention_window(
                _dev(q, "q"), kc, vc, sl, B, h, g, d, n, cap, window, int(ring), float(scale), dt,
                num_splits, wsptr, wsb, _dev(out, "out", torch.float32),
                _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_*decode_attention_window", st)
    else:
        ws, wsb = wsp(lib.kvc_decode_workspace_bytes(B, h * n, g, d, dt,
                                                     _plan_len(mb * bs, window, n), num_splits, 1))
        wsptr = ws.data_ptr() if ws is not None else None
        kp, vp = _dev(k_cache, "k_pool", q.dtype), _dev(v_cache, "v_pool", q.dtype)
        bt = _dev(block_table, "block_table", torch.int32)
        if fused:
            st = lib.kvc_append_decode_attention_window_paged(
                _dev(q, "q"), kn, vn, kp, vp, bt, mb, bs, nb, sl, B, h, g, d, n, window,
                float(scale), dt, num_splits, wsptr, wsb, _dev(out, "out", torch.float32),
                _dev(lse, "lse", torch.float32), _stream(stream))
        else:
            st = lib.kvc_decode_attention_window_paged(
                _dev(q, "q"), kp, vp, bt, mb, bs, nb, sl, B, h, g, d, n, window, float(scale), dt,
                num_splits, wsptr, wsb, _dev(out, "out", torch.float32),
                _dev(lse, "lse", torch.float32), _stream(stream))
        _check("kvc_*decode_attention_window_paged", st)
    return out, lse


@_on_device
def copy_blocks(k_pool, v_pool, pairs, stream=None):
    """Copy physical block src -> dst of both pools [NB,g,bs,d] for every row
    (src, dst) of the device int32 tensor ``pairs`` [n, 2] (copy-on-write)."""
    lib = load_library()
    nb, g, bs, d = _shape(k_pool, (None, None, None, None), "k_pool")
    _shape(v_pool, (nb, g, bs, d), "v_pool")
    n = pairs.shape[0] if pairs.numel() else 0
    if n:
        _shape(pairs, (n, 2), "pairs")
    _check("kvc_copy_blocks", lib.kvc_copy_blocks(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
        _dev(pairs, "pairs", torch.int32) if n else None, n, nb, g, bs, d,
        _dtype_code(k_pool), _stream(stream)))


@_on_device
def fork_block_tables(block_table, seq_lens, parent, stream=None):
    """Forked tables: row b is row parent[b] (and its length).  Returns
    (tables [B,max_blocks], seq_lens [B]) on the device."""
    lib = load_library()
    B_src, mb = _shape(block_table, (None, None), "block_table")
    _shape(seq_lens, (B_src,), "seq_lens")
    (B,) = _shape(parent, (None,), "parent")
    out_t = torch.empty((B, mb), dtype=torch.int32, device=block_table.device)
    out_l = torch.empty((B,), dtype=torch.int32, device=block_table.device)
    _check("kvc_fork_block_tables", lib.kvc_fork_block_tables(
        _dev(block_table, "block_table", torch.int32), _dev(seq_lens, "seq_lens", torch.int32),
        B_src, mb, _dev(parent, "parent", torch.int32), B, _dev(out_t, "out"), _dev(out_l, "out"),
        _stream(stream)))
    return out_t, out_l


@_on_device
def gather_cache(k_src, v_src, seq_lens, parent, k_dst, v_dst, stream=None):
    """Contiguous caches re-ranked by parent into k_dst, v_dst [B,g,t_cap,d]:
    positions below seq_lens[parent[b]] of sequence b come from parent[b]."""
    lib = load_library()
    B_src, g, t_cap, d = _shape(k_src, (None, None, None, None), "k_src")
    _shape(v_src, (B_src, g, t_cap, d), "v_src")
    _shape(seq_lens, (B_src,), "seq_lens")
    (B,) = _shape(parent, (None,), "parent")
    _shape(k_dst, (B, g, t_cap, d), "k_dst")
    _shape(v_dst, (B, g, t_cap, d), "v_dst")
    _check("kvc_gather_cache", lib.kvc_gather_cache(
        _dev(k_src, "k_src"), _dev(v_src, "v_src", k_src.dtype),
        _dev(seq_lens, "seq_lens", torch.int32), B_src, _dev(parent, "parent", torch.int32), B,
        _dev(k_dst, "k_dst", k_src.dtype), _dev(v_dst, "v_dst", k_src.dtype), g, t_cap, d,
        _dtype_code(k_src), _stream(stream)))


@_on_device
def append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, seq_lens_before, block_table=None,
               stream=None):
    """Quantise the new token's K/V (bf16 [B,g,d]) into uint8 FP8 E4M3 caches
    (contiguous [B,g,t_cap,d] or pools [NB,g,bs,d]) with per-KV-head float32
    scales k_scale, v_scale [g]."""
    lib = load_library()
    B, g, d = _shape(k_new, (None, None, None), "k_new")
    _shape(v_new, (B, g, d), "v_new")
    _shape(seq_lens_before, (B,), "seq_lens_before")
    gc, capacity, bs, mb, _ = _cache_shapes(k_cache, v_cache, B, d, block_table)
    if gc != g:
        raise ValueError(f"k_new has {g} KV heads, the cache {gc}")
    _shape(k_scale, (g,), "k_scale")
    _shape(v_scale, (g,), "v_scale")
    bt = _dev(block_table, "block_table", torch.int32) if block_table is not None else None
    _check("kvc_append_fp8", lib.kvc_append_fp8(
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16),
        _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32), bt, mb,
        bs, _dev(seq_lens_before, "seq_lens_before", torch.int32), B, g, d, capacity,
        _stream(stream)))


@_on_device
def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table=None,
               scale: Optional[float] = None, num_splits: int = 0,
               workspace: Optional[torch.Tensor] = None, out=None, lse=None, stream=None,
               k_new=None, v_new=None):
    """Decode attention (q bf16 [B,h,d]) over uint8 FP8 E4M3 caches with
    per-KV-head scales.  Without k_new: seq_lens are attended lengths.  With
    k_new, v_new (bf16 [B,g,d]): seq_lens holds the lengths before the step;
    the call quantises and appends the new token and attends (one launch).
    Returns (out [B,h,d] float32, lse [B,h] float32)."""
    lib = load_library()
    B, h, d = _shape(q, (None, None, None), "q")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _shape(k_scale, (g,), "k_scale")
    _shape(v_scale, (g,), "v_scale")
    _shape(seq_lens, (B,), "seq_lens")
    fused = k_new is not None
    if fused:
        _new_tokens(k_new, v_new, B, g, None, d)
    elif v_new is not None:
        raise ValueError("v_new without k_new")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    qp = _dev(q, "q", torch.bfloat16)
    ks, vs = _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32)
    sl = _dev(seq_lens, "seq_lens", torch.int32)
    kn = _dev(k_new, "k_new", torch.bfloat16) if fused else None
    vn = _dev(v_new, "v_new", torch.bfloat16) if fused else None
    if block_table is None:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, BF16, cap, num_splits, 0),
                             q, workspace)
        wsp = ws.data_ptr() if ws is not None else None
        kc, vc = _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8)
        if fused:
            st = lib.kvc_append_decode_attention_fp8(qp, kn, vn, kc, vc, ks, vs, sl, B, h, g, d,
                                                     cap, float(scale), num_splits, wsp, wsb,
                                                     _dev(out, "out"), _dev(lse, "lse"),
                                                     _stream(stream))
        else:
            st = lib.kvc_decode_attention_fp8(qp, kc, vc, ks, vs, sl, B, h, g, d, cap,
                                              float(scale), num_splits, wsp, wsb,
                                              _dev(out, "out"), _dev(lse, "lse"), _stream(stream))
    else:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h, g, d, BF16, mb * bs, num_splits, 1),
                             q, workspace)
        wsp = ws.data_ptr() if ws is not None else None
        kp, vp = _dev(k_cache, "k_pool", torch.uint8), _dev(v_cache, "v_pool", torch.uint8)
        bt = _dev(block_table, "block_table", torch.int32)
        if fused:
            st = lib.kvc_append_decode_attention_fp8_paged(qp, kn, vn, kp, vp, ks, vs, bt, mb, bs,
                                                           nb, sl, B, h, g, d, float(scale),
                                                           num_splits, wsp, wsb, _dev(out, "out"),
                                                           _dev(lse, "lse"), _stream(stream))
        else:
            st = lib.kvc_decode_attention_fp8_paged(qp, kp, vp, ks, vs, bt, mb, bs, nb, sl, B, h, g,
                                                    d, float(scale), num_splits, wsp, wsb,
                                                    _dev(out, "out"), _dev(lse, "lse"),
                                                    _stream(stream))
    _check("kvc_*decode_attention_fp8", st)
    return out, lse


@_on_device
def decode_fp8_window(q, k_cache, v_cache, k_scale, v_scale, seq_lens, window: int = 0,
                      ring: bool = False, block_table=None, scale: Optional[float] = None,
                      num_splits: int = 0, workspace: Optional[torch.Tensor] = None, out=None,
                      lse=None, stream=None, k_new=None, v_new=None):
    """Several query tokens per sequence (q bf16 [B,h,n,d]) over uint8 FP8
    E4M3 caches with per-KV-head scales [g]; token t at position
    seq_lens[b] - n + t (or seq_lens_before[b] + t with k_new) sees the
    positions up to itself, the last ``window`` of them when window > 0
    (window 0: the _multi calls).  With k_new, v_new (bf16 [B,g,n,d]) the
    call quantises and appends the n tokens (seq_lens = lengths before the
    step).  ring: contiguous ring cache of t_cap slots.  Returns (out
    [B,h,n,d] float32, lse [B,h,n] float32)."""
    lib = load_library()
    B, h, n, d = _shape(q, (None, None, None, None), "q")
    if ring and block_table is not None:
        raise ValueError("a ring cache is contiguous")
    if ring and window <= 0:
        raise ValueError("a ring cache needs a window")
    g, cap, bs, mb, nb = _cache_shapes(k_cache, v_cache, B, d, block_table)
    _shape(k_scale, (g,), "k_scale")
    _shape(v_scale, (g,), "v_scale")
    _shape(seq_lens, (B,), "seq_lens")
    fused = k_new is not None
    if fused:
        _new_tokens(k_new, v_new, B, g, n, d)
    elif v_new is not None:
        raise ValueError("v_new without k_new")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    qp = _dev(q, "q", torch.bfloat16)
    ks, vs = _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32)
    sl = _dev(seq_lens, "seq_lens", torch.int32)
    kn = _dev(k_new, "k_new", torch.bfloat16) if fused else None
    vn = _dev(v_new, "v_new", torch.bfloat16) if fused else None
    o, l_ = _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32)
    sc, st = float(scale), _stream(stream)
    if block_table is None:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, BF16,
                                                            _plan_len(cap, window, n), num_splits,
                                                            0), q, workspace)
        wsp = ws.data_ptr() if ws is not None else None
        kc, vc = _dev(k_cache, "k_cache", torch.uint8), _dev(v_cache, "v_cache", torch.uint8)
        if fused and window > 0:
            r = lib.kvc_append_decode_attention_fp8_window(qp, kn, vn, kc, vc, ks, vs, sl, B, h, g,
                                                           d, n, cap, window, int(ring), sc,
                                                           num_splits, wsp, wsb, o, l_, st)
        elif fused:
            r = lib.kvc_append_decode_attention_fp8_multi(qp, kn, vn, kc, vc, ks, vs, sl, B, h, g, d,
                                                          n, cap, sc, num_splits, wsp, wsb, o, l_,
                                                          st)
        elif window > 0:
            r = lib.kvc_decode_attention_fp8_window(qp, kc, vc, ks, vs, sl, B, h, g, d, n, cap,
                                                    window, int(ring), sc, num_splits, wsp, wsb, o,
                                                    l_, st)
        else:
            r = lib.kvc_decode_attention_fp8_multi(qp, kc, vc, ks, vs, sl, B, h, g, d, n, cap, sc,
                                                   num_splits, wsp, wsb, o, l_, st)
    else:
        ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, BF16,
                                                            _plan_len(mb * bs, window, n),
                                                            num_splits, 1), q, workspace)
        wsp = ws.data_ptr() if ws is not None else None
        kp, vp = _dev(k_cache, "k_pool", torch.uint8), _dev(v_cache, "v_pool", torch.uint8)
        bt = _dev(block_table, "block_table", torch.int32)
        if fused and window > 0:
            r = lib.kvc_append_decode_attention_fp8_window_paged(qp, kn, vn, kp, vp, ks, vs, bt, mb,
                                                                 bs, nb, sl, B, h, g, d, n, window,
                                                                 sc, num_splits, wsp, wsb, o, l_,
                                                                 st)
        elif fused:
            r = lib.kvc_append_decode_attention_fp8_multi_paged(qp, kn, vn, kp, vp, ks, vs, bt, mb,
                                                                bs, nb, sl, B, h, g, d, n, sc,
                                                                num_splits, wsp, wsb, o, l_, st)
        elif window > 0:
            r = lib.kvc_decode_attention_fp8_window_paged(qp, kp, vp, ks, vs, bt, mb, bs, nb, sl, B,
                                                          h, g, d, n, window, sc, num_splits, wsp,
                                                          wsb, o, l_, st)
        else:
            r = lib.kvc_decode_attention_fp8_multi_paged(qp, kp, vp, ks, vs, bt, mb, bs, nb, sl, B,
                                                         h, g, d, n, sc, num_splits, wsp, wsb, o,
                                                         l_, st)
    _check("kvc_*decode_attention_fp8_(multi|window)", r)
    return out, lse


@_on_device
def append_decode_noalloc(q, k_new, v_new, k_cache, v_cache, seq_lens_before,
                          scale: Optional[float] = None, num_splits: int = 0, out=None, lse=None,
                          stream=None):
    """append_decode on a contiguous cache without a workspace: split
    partials go to the library's static scratch
    (kvc_append_decode_attention_noalloc; KvcError status 5 when the split
    needs more than it holds)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, h, d = _shape(q, (None, None, None), "q")
    g, cap, _, _, _ = _cache_shapes(k_cache, v_cache, B, d, None)
    _new_tokens(k_new, v_new, B, g, None, d)
    _shape(seq_lens_before, (B,), "seq_lens_before")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    st = lib.kvc_append_decode_attention_noalloc(
        _dev(q, "q"), _dev(k_new, "k_new", q.dtype), _dev(v_new, "v_new", q.dtype),
        _dev(k_cache, "k_cache", q.dtype), _dev(v_cache, "v_cache", q.dtype),
        _dev(seq_lens_before, "seq_lens_before", torch.int32), B, h, g, d, cap, float(scale), dt,
        num_splits, _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32),
        _stream(stream))
    _check("kvc_append_decode_attention_noalloc", st)
    return out, lse


@_on_device
def append_fp8_block_scaled(k_new, v_new, k_pool, v_pool, k_scale, v_scale, seq_lens_before,
                            block_table, stream=None):
    """Quantise n new tokens per sequence (bf16 [B,g,n,d]) into uint8 FP8
    pools [NB,g,bs,d] whose scales are per (physical block, KV head):
    k_scale, v_scale float32 [NB, g]."""
    lib = load_library()
    B, g, n, d = _shape(k_new, (None, None, None, None), "k_new")
    _shape(v_new, (B, g, n, d), "v_new")
    _shape(seq_lens_before, (B,), "seq_lens_before")
    gp, _, bs, mb, nb = _cache_shapes(k_pool, v_pool, B, d, block_table)
    if gp != g:
        raise ValueError(f"k_new has {g} KV heads, the pool {gp}")
    _shape(k_scale, (nb, g), "k_scale")
    _shape(v_scale, (nb, g), "v_scale")
    _check("kvc_append_fp8_paged_block_scaled", lib.kvc_append_fp8_paged_block_scaled(
        _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16),
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_table, "block_table", torch.int32), mb, bs, nb,
        _dev(seq_lens_before, "seq_lens_before", torch.int32), B, g, d, n, _stream(stream)))


@_on_device
def decode_fp8_block_scaled(q, k_pool, v_pool, k_scale, v_scale, seq_lens, block_table,
                            window: int = 0, scale: Optional[float] = None, num_splits: int = 0,
                            workspace: Optional[torch.Tensor] = None, out=None, lse=None,
                            stream=None, k_new=None, v_new=None):
    """Attention for q (bf16 [B,h,n,d]) over uint8 FP8 pools [NB,g,bs,d]
    with per-(block, KV head) scales [NB, g]; token t sees the positions up
    to its own (the last ``window`` of them when window > 0).  With k_new,
    v_new (bf16 [B,g,n,d]) the call also quantises and appends the tokens
    (seq_lens = lengths before the step).  Returns (out [B,h,n,d] float32,
    lse [B,h,n] float32)."""
    lib = load_library()
    B, h, n, d = _shape(q, (None, None, None, None), "q")
    g, _, bs, mb, nb = _cache_shapes(k_pool, v_pool, B, d, block_table)
    _shape(k_scale, (nb, g), "k_scale")
    _shape(v_scale, (nb, g), "v_scale")
    _shape(seq_lens, (B,), "seq_lens")
    fused = k_new is not None
    if fused:
        _new_tokens(k_new, v_new, B, g, n, d)
    elif v_new is not None:
        raise ValueError("v_new without k_new")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    ws, wsb = _workspace(lib.kvc_decode_workspace_bytes(B, h * n, g, d, BF16,
                                                        _plan_len(mb * bs, window, n), num_splits,
                                                        1), q, workspace)
    st = lib.kvc_decode_attention_fp8_paged_block_scaled(
        _dev(q, "q", torch.bfloat16), _dev(k_new, "k_new", torch.bfloat16) if fused else None,
        _dev(v_new, "v_new", torch.bfloat16) if fused else None,
        _dev(k_pool, "k_pool", torch.uint8), _dev(v_pool, "v_pool", torch.uint8),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_table, "block_table", torch.int32), mb, bs, nb,
        _dev(seq_lens, "seq_lens", torch.int32), B, h, g, d, n, window, float(scale), num_splits,
        ws.data_ptr() if ws is not None else None, wsb, _dev(out, "out", torch.float32),
        _dev(lse, "lse", torch.float32), _stream(stream))
    _check("kvc_decode_attention_fp8_paged_block_scaled", st)
    return out, lse
