"""CPU fp64 oracle for single-token decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``kv_cache_gqa_amd``) and never imports it.

The arithmetic lives in ``kvc_oracle.c`` (plain loops, double precision); this
module only marshals arrays into it.  Pages followed:

* "大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com), section 三 3.3:
  query head i uses KV head floor(i*g/h); section 二: KV cache size formula.
* "每生成一个词为何又重算全文？KV Cache 的增量解码" (zwjcode.cn), sections 02,
  04, 08, 10: per-step shapes, worked example, append position, invisible
  unwritten slots; section 02 also the element count 2*L*N*H*T*d.
* "KV Cache 优化与注意力机制加速：FlashAttention / PagedAttention"
  (plumephp.com), sections 2.2-2.5 (m, l, lse = m + log l, sequence split),
  3.2 (size formula), 4.2-4.3 (block table lookup), 5.3 (speculative
  decoding: several draft tokens checked in one pass).
* Sliding window (plumephp.com section 5.2: a token attends within a local
  window to its left; zwjcode.cn section 10: a window cache keeps only the
  last W positions, so its memory is bounded): the token at position x sees
  positions max(0, x + 1 - W) .. x, the last W including itself.  A ring
  cache of t_cap slots keeps position p in slot p mod t_cap.
* Block operations on a paged pool (plumephp.com section 4.3: requests fork
  a block table and share physical blocks; a block is copied before a
  sharing request writes into it; zwjcode.cn section 11: after beams are
  re-ranked, each beam's cache must follow its chosen parent): copy whole
  blocks, gather block-table rows by parent, gather contiguous caches by
  parent.  Plain index copies.
* Low-precision cache (plumephp.com section 2.5: FP8 attention;
  zwjcode.cn section 14: low-bit K/V cut memory and bandwidth at a cost in
  error): K and V stored as OCP FP8 E4M3 codes (1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite
  value 448) with one float32 scale per KV head.  Stored code of x:
  nearest E4M3 value to the float32 quotient x / scale, ties to the even
  code, values beyond 448 saturating to 448.  Attention runs over the
  dequantised values code * scale, exactly as over any other cache.
* Several new tokens at once (a prefill after a cached prefix, limoncc.com
  section 5.2; draft tokens, plumephp.com section 5.3): token t of a sequence
  with P cached positions sits at position P + t and sees positions 0..P + t
  (the causal mask of the full sequence, aligned to its bottom-right corner,
  which zwjcode.cn section 13 warns a non-square is_causal mask gets wrong).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_ORACLE_LIB names another build of kvc_oracle.c (the sanitizer test
# loads one built with AddressSanitizer and UndefinedBehaviorSanitizer).
LIB_PATH = os.environ.get("KVC_ORACLE_LIB") or os.path.join(HERE, "libkvc_oracle.so")

F32 = 0
BF16 = 1
F64 = 2  # values already in float64 (dequantised FP8 codes, widened queries)

_lib = None


def configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    vp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.kvo_decode.argtypes = [vp, vp, vp, ip, vp, ip, ip, vp, ip, ip, ip, ip, ip, dp,
                               vp, vp, ip]
    lib.kvo_decode.restype = None
    lib.kvo_decode_split.argtypes = [vp, vp, vp, ip, vp, ip, ip, vp, ip, ip, ip, ip, ip,
                                     dp, ip, vp, vp, ip]
    lib.kvo_decode_split.restype = None
    lib.kvo_append.argtypes = [vp, vp, vp, vp, ip, vp, ip, ip, vp, ip, ip, ip, ip]
    lib.kvo_append.restype = None
    lib.kvo_decode_range.argtypes = [vp, vp, vp, ip, vp, ip, ip, vp, vp, ip, ip, ip, ip, ip, dp,
                                     vp, vp, ip]
    lib.kvo_decode_range.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = configure(ctypes.CDLL(LIB_PATH))
    return _lib


def _raw(x, dtype_code=None):
    """Return (contiguous numpy view of the raw storage, dtype code).

    Accepts numpy arrays or CPU torch tensors (float32, bfloat16, int32).
    bfloat16 storage is passed as its uint16 bit pattern, unchanged."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        t = x.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be host (CPU) tensors")
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float32:
            return t.numpy(), F32
        if t.dtype == torch.float64:
            return t.numpy(), F64
        if t.dtype == torch.int32:
            return t.numpy(), None
        raise TypeError(f"unsupported oracle input dtype {t.dtype}")
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:  # raw bf16 bits
        return a, BF16
    if a.dtype == np.int32:
        return a, None
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _i32(x):
    """Contiguous int32 numpy copy of a list, numpy array or CPU torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _same_dtype(*codes):
    codes = [c for c in codes if c is not None]
    if len(set(codes)) != 1:
        raise TypeError("q, K and V must share one dtype")
    return codes[0]


def decode(q, k, v, seq_lens, scale, block_table=None, block_size=16, nthreads=0):
    """out [B,h,d] float64, lse [B,h] float64 of single-token decode attention.

    q [B,h,d]; k, v contiguous [B,g,t_cap,d] or (with block_table [B,max_blocks])
    paged pools [num_blocks,g,block_size,d]; seq_lens [B] attended lengths.
    ``scale`` is used as the float32 value the GPU receives, widened exactly."""
    qa, qd = _raw(q)
    ka, kd = _raw(k)
    va, vd = _raw(v)
    dt = _same_dtype(qd, kd, vd)
    sl = _i32(seq_lens)
    B, h, d = qa.shape
    if block_table is None:
        _, g, t_cap, _ = ka.shape
        bt, max_blocks, bsz = None, 0, 0
    else:
        bt = _i32(block_table)
        _, g, bsz, _ = ka.shape
        assert bsz == block_size
        max_blocks = bt.shape[1]
        t_cap = 0
    out = np.zeros((B, h, d), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    sc = float(np.float32(scale))
    _load().kvo_decode(_ptr(qa), _ptr(ka), _ptr(va), dt,
                       _ptr(bt) if bt is not None else None, max_blocks, bsz,
                       _ptr(sl), B, h, g, d, t_cap, sc, _ptr(out), _ptr(lse), int(nthreads))
    return out, lse


def decode_split(q, k, v, seq_lens, scale, chunk_len, block_table=None, block_size=16,
                 nthreads=0):
    """Split-and-merge reference: chunks of ``chunk_len`` positions, each turned
    into (O_c, lse_c), then merged by log-sum-exp.  Same arguments as decode."""
    qa, qd = _raw(q)
    ka, kd = _raw(k)
    va, vd = _raw(v)
    dt = _same_dtype(qd, kd, vd)
    sl = _i32(seq_lens)
    B, h, d = qa.shape
    if block_table is None:
        _, g, t_cap, _ = ka.shape
        bt, max_blocks, bsz = None, 0, 0
    else:
        bt = _i32(block_table)
        _, g, bsz, _ = ka.shape
        max_blocks = bt.shape[1]
        t_cap = 0
    out = np.zeros((B, h, d), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    sc = float(np.float32(scale))
    _load().kvo_decode_split(_ptr(qa), _ptr(ka), _ptr(va), dt,
                             _ptr(bt) if bt is not None else None, max_blocks, bsz,
                             _ptr(sl), B, h, g, d, t_cap, sc, int(chunk_len),
                             _ptr(out), _ptr(lse), int(nthreads))
    return out, lse


def append(k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None, block_size=16):
    """Return new (k_cache, v_cache) numpy arrays (raw storage) with the new
    token's K/V of every (b, j) written at position seq_lens_before[b]."""
    kn, kd = _raw(k_new)
    vn, vd = _raw(v_new)
    kc, kcd = _raw(k_cache)
    vc, vcd = _raw(v_cache)
    dt = _same_dtype(kd, vd, kcd, vcd)
    kc = kc.copy()
    vc = vc.copy()
    sl = _i32(seq_lens_before)
    B, g, d = kn.shape
    if block_table is None:
        t_cap = kc.shape[2]
        bt, max_blocks, bsz = None, 0, 0
        if B and (sl.min() < 0 or sl.max() >= t_cap):
            raise ValueError("append position outside the cache")
    else:
        bt = _i32(block_table)
        max_blocks = bt.shape[1]
        bsz = kc.shape[2]
        t_cap = 0
        blk = sl // bsz
        if B and (sl.min() < 0 or blk.max() >= max_blocks or
                  any(not 0 <= bt[b, blk[b]] < kc.shape[0] for b in range(B))):
            raise ValueError("append position outside the pool")
    _load().kvo_append(_ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), dt,
                       _ptr(bt) if bt is not None else None, max_blocks, bsz,
                       _ptr(sl), B, g, d, t_cap)
    return kc, vc


def kv_cache_bytes(layers: int, batch: int, kv_heads: int, tokens: int, head_dim: int,
                   elem_bytes: int) -> int:
    """Closed-form KV cache size: 2 (K and V) x layers x batch x KV heads x
    tokens x head_dim x element bytes.  The zwjcode.cn page (section 02) gives
    the element count 2*L*N*H*T*d; the limoncc.com page (section 二) and the
    plumephp.com page (section 3.2) give the byte form."""
    return 2 * layers * batch * kv_heads * tokens * head_dim * elem_bytes


def _multi_position(before, t):
    """Position of new token t of a sequence that had ``before`` cached ones."""
    return before + t


def _multi_visible(before, t):
    """Positions new token t sees: the cached ones and new tokens 0..t."""
    return before + t + 1


def append_multi(k_new, v_new, k_cache, v_cache, seq_lens_before, block_table=None):
    """k_new, v_new [B,g,n,d]: token t of sequence b is written at position
    seq_lens_before[b] + t.  Returns new (k_cache, v_cache) raw numpy arrays."""
    kn, _ = _raw(k_new)
    vn, _ = _raw(v_new)
    before = _i32(seq_lens_before)
    kc, vc = k_cache, v_cache
    for t in range(kn.shape[2]):
        kc, vc = append(np.ascontiguousarray(kn[:, :, t]), np.ascontiguousarray(vn[:, :, t]), kc, vc,
                        _multi_position(before, t).astype(np.int32), block_table)
    return kc, vc


def decode_multi(q, k, v, seq_lens_before, scale, block_table=None, block_size=16, nthreads=0):
    """q [B,h,n,d]: query token t of sequence b attends, through the single
    token definition above, to the positions it sees (``_multi_visible``) of a
    cache that already holds every new token.  Returns out [B,h,n,d] and lse
    [B,h,n], float64."""
    qa, _ = _raw(q)
    before = _i32(seq_lens_before)
    B, h, n, d = qa.shape
    out = np.zeros((B, h, n, d), dtype=np.float64)
    lse = np.zeros((B, h, n), dtype=np.float64)
    for t in range(n):
        o, l = decode(np.ascontiguousarray(qa[:, :, t]), k, v,
                      _multi_visible(before, t).astype(np.int32), scale, block_table=block_table,
                      block_size=block_size, nthreads=nthreads)
        out[:, :, t] = o
        lse[:, :, t] = l
    return out, lse


def decode_range(q, k, v, starts, seq_lens, scale, block_table=None, block_size=16, nthreads=0):
    """Like ``decode`` over positions [starts[b], seq_lens[b]) only."""
    qa, qd = _raw(q)
    ka, kd = _raw(k)
    va, vd = _raw(v)
    dt = _same_dtype(qd, kd, vd)
    st = _i32(starts)
    sl = _i32(seq_lens)
    B, h, d = qa.shape
    if block_table is None:
        _, g, t_cap, _ = ka.shape
        bt, max_blocks, bsz = None, 0, 0
    else:
        bt = _i32(block_table)
        _, g, bsz, _ = ka.shape
        assert bsz == block_size
        max_blocks = bt.shape[1]
        t_cap = 0
    out = np.zeros((B, h, d), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    sc = float(np.float32(scale))
    _load().kvo_decode_range(_ptr(qa), _ptr(ka), _ptr(va), dt,
                             _ptr(bt) if bt is not None else None, max_blocks, bsz,
                             _ptr(st), _ptr(sl), B, h, g, d, t_cap, sc, _ptr(out), _ptr(lse),
                             int(nthreads))
    return out, lse


def _window_start(visible, window):
    """First position a token sees when it sees ``visible`` positions under a
    sliding window of ``window`` (0: no window)."""
    if window <= 0:
        return np.zeros_like(visible)
    return np.maximum(visible - window, 0)


def _ring_slot(p, t_cap):
    return p % t_cap


def append_window(k_new, v_new, k_cache, v_cache, seq_lens_before, ring=False, block_table=None):
    """Write n new tokens per sequence (k_new, v_new [B,g,n,d]) at positions
    seq_lens_before[b] + t; a ring cache (contiguous [B,g,t_cap,d]) keeps
    position p in slot p mod t_cap.  Returns raw numpy caches."""
    if not ring:
        return append_multi(k_new, v_new, k_cache, v_cache, seq_lens_before, block_table)
    kn, _ = _raw(k_new)
    vn, _ = _raw(v_new)
    t_cap = _raw(k_cache)[0].shape[2]
    before = _i32(seq_lens_before)
    kc, vc = k_cache, v_cache
    for t in range(kn.shape[2]):
        slot = _ring_slot(_multi_position(before, t), t_cap).astype(np.int32)
        kc, vc = append(np.ascontiguousarray(kn[:, :, t]), np.ascontiguousarray(vn[:, :, t]), kc, vc,
                        slot)
    return kc, vc


def _linearize_ring(cache_raw, lo, hi):
    """[B,g,max(hi),d] raw array holding position p of sequence b (lo[b] <= p
    < hi[b]) taken from ring slot p mod t_cap; other positions are zero."""
    B, g, t_cap, d = cache_raw.shape
    L = int(max(int(np.max(hi)) if len(hi) else 0, 1))
    lin = np.zeros((B, g, L, d), dtype=cache_raw.dtype)
    for b in range(B):
        p = np.arange(int(lo[b]), int(hi[b]))
        lin[b, :, p] = np.moveaxis(cache_raw[b][:, _ring_slot(p, t_cap)], 1, 0)
    return lin


def decode_window(q, k, v, seq_lens_before, scale, window, ring=False, block_table=None,
                  block_size=16, nthreads=0):
    """q [B,h,n,d]: token t of sequence b sits at position seq_lens_before[b]
    + t and attends to positions max(0, x + 1 - window) .. x (window 0: all
    of 0 .. x) of a cache that already holds every new token (a ring cache
    when ``ring``).  Returns out [B,h,n,d], lse [B,h,n] (float64)."""
    qa, _ = _raw(q)
    before = _i32(seq_lens_before)
    B, h, n, d = qa.shape
    out = np.zeros((B, h, n, d), dtype=np.float64)
    lse = np.zeros((B, h, n), dtype=np.float64)
    for t in range(n):
        hi = _multi_visible(before, t).astype(np.int32)
        lo = _window_start(hi, window).astype(np.int32)
        kk, vv = k, v
        if ring:
            kk = _linearize_ring(_raw(k)[0], lo, hi)
            vv = _linearize_ring(_raw(v)[0], lo, hi)
        o, l = decode_range(np.ascontiguousarray(qa[:, :, t]), kk, vv, lo, hi, scale,
                            block_table=None if ring else block_table, block_size=block_size,
                            nthreads=nthreads)
        out[:, :, t] = o
        lse[:, :, t] = l
    return out, lse


def copy_blocks(k_pool, v_pool, pairs):
    """Copy physical block src to dst (all KV heads, K and V) for every
    (src, dst) in ``pairs``; pairs naming a block outside the pool are
    skipped.  Returns new raw numpy pools."""
    kp, _ = _raw(k_pool)
    vp, _ = _raw(v_pool)
    kp, vp = kp.copy(), vp.copy()
    nb = kp.shape[0]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= src < nb and 0 <= dst < nb:
            kp[dst] = kp[src]
            vp[dst] = vp[src]
    return kp, vp


def fork_tables(tables, seq_lens, parent):
    """Row b of the result is row parent[b] of ``tables`` (and its length):
    the forked requests share their parent's physical blocks."""
    t = _i32(tables)
    sl = _i32(seq_lens)
    par = _i32(parent).astype(np.int64)
    return t[par].copy(), sl[par].copy()


def gather_cache(k_cache, v_cache, parent, seq_lens, k_dst=None, v_dst=None):
    """Contiguous caches re-ranked by parent: position p < seq_lens[parent[b]]
    of sequence b is position p of sequence parent[b].  Positions past that
    length keep what k_dst / v_dst held (zero when not given).  Returns raw
    numpy caches [len(parent), g, t_cap, d]."""
    kc, _ = _raw(k_cache)
    vc, _ = _raw(v_cache)
    sl = _i32(seq_lens)
    par = _i32(parent).astype(np.int64)
    if k_dst is None:
        ko = np.zeros((len(par),) + kc.shape[1:], dtype=kc.dtype)
        vo = np.zeros_like(ko)
    else:
        ko, vo = _raw(k_dst)[0].copy(), _raw(v_dst)[0].copy()
    for b, pb in enumerate(par):
        L = int(sl[pb])
        ko[b, :, :L] = kc[pb, :, :L]
        vo[b, :, :L] = vc[pb, :, :L]
    return ko, vo


def e4m3_values():
    """float64 value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_encode(y):
    """Codes (uint8) of float32 values y: nearest E4M3 value, ties to the even
    code, |y| > 448 saturating to 448, NaN to 0x7F with y's sign, and the sign
    kept for values that round to zero."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    pos = e4m3_values()[:127]                 # codes 0..126: 0 .. 448, increasing
    a_sat = np.minimum(a, 448.0)
    hi = np.searchsorted(pos, a_sat, side="left")   # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - pos[lo]
    d_hi = pos[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pos[hi] == a_sat, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = np.where(np.isnan(a), np.uint8(0x7F), code).astype(np.uint8)
    return (code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def quantize_fp8(x, scale, head_axis):
    """E4M3 codes of bf16/float32 values x with one float32 scale per KV head
    (``scale`` [g], indexed along ``head_axis`` of x): code of x / scale,
    the quotient taken in float32."""
    xa, xd = _raw(x)
    xf = xa.astype(np.uint32) << 16 if xd == BF16 else xa
    xf = xf.view(np.float32) if xd == BF16 else xf
    sc = np.asarray(scale, dtype=np.float32)
    shape = [1] * xf.ndim
    shape[head_axis] = -1
    return e4m3_encode((xf / sc.reshape(shape)).astype(np.float32))


def append_fp8(k_new, v_new, k_codes, v_codes, k_scale, v_scale, seq_lens_before,
               block_table=None, ring=False):
    """Quantise n new tokens per sequence (k_new, v_new [B,g,n,d] bf16) and
    write their codes at positions seq_lens_before[b] + t of uint8 caches
    (contiguous [B,g,t_cap,d] or pools [NB,g,bs,d] through block_table; a
    ring cache keeps position p in slot p mod t_cap).  Returns new uint8
    caches."""
    kq = quantize_fp8(k_new, k_scale, 1)
    vq = quantize_fp8(v_new, v_scale, 1)
    kc = np.array(k_codes, dtype=np.uint8, copy=True)
    vc = np.array(v_codes, dtype=np.uint8, copy=True)
    before = _i32(seq_lens_before)
    bt = None if block_table is None else _i32(block_table)
    B, g, n, _ = kq.shape
    for b in range(B):
        for t in range(n):
            p = int(before[b]) + t
            if bt is None:
                slot = _ring_slot(p, kc.shape[2]) if ring else p
                if not 0 <= slot < kc.shape[2]:
                    raise ValueError("append position outside the cache")
                kc[b, :, slot] = kq[b, :, t]
                vc[b, :, slot] = vq[b, :, t]
            else:
                bs = kc.shape[2]
                blk = int(bt[b, p // bs])
                kc[blk, :, p % bs] = kq[b, :, t]
                vc[blk, :, p % bs] = vq[b, :, t]
    return kc, vc


def dequantize_fp8(codes, scale, head_axis):
    """float64 values of E4M3 codes with one float32 scale per KV head
    (``scale`` [g], indexed along ``head_axis``): the code's value times its
    head's scale.  Both factors are exact in float64 and so is their product
    (at most 4 + 24 significant bits)."""
    x = e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    return x * sc.reshape(shape)


def widen(x):
    """float64 copy of bf16 / float32 values (exact)."""
    a, code = _raw(x)
    if code == BF16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, dtype=np.float64)


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale, block_table=None,
               block_size=16, nthreads=0):
    """Single-token attention over FP8 caches: dequantise, then the plain
    definition.  K = code * k_scale[j] and V = code * v_scale[j] in float64
    (``dequantize_fp8``), the bf16 queries widened to float64, and ``decode``
    over those values with the same float32 score scale."""
    k = dequantize_fp8(k_codes, k_scale, 1)
    v = dequantize_fp8(v_codes, v_scale, 1)
    return decode(widen(q), k, v, seq_lens, scale, block_table=block_table,
                  block_size=block_size, nthreads=nthreads)


def decode_fp8_window(q, k_codes, v_codes, k_scale, v_scale, seq_lens_before, scale, window=0,
                      ring=False, block_table=None, block_size=16, nthreads=0):
    """Several query tokens per sequence (q [B,h,n,d] bf16) over FP8 caches
    that already hold them, with an optional sliding window (0: none) and
    ring cache: dequantise (``dequantize_fp8``), then ``decode_window`` over
    the dequantised values.  Returns out [B,h,n,d], lse [B,h,n]."""
    k = dequantize_fp8(k_codes, k_scale, 1)
    v = dequantize_fp8(v_codes, v_scale, 1)
    return decode_window(widen(q), k, v, seq_lens_before, scale, window, ring=ring,
                         block_table=block_table, block_size=block_size, nthreads=nthreads)


def dequantize_fp8_blocks(codes, scale):
    """float64 values of a paged pool of E4M3 codes [NB, g, bs, d] with one
    float32 scale per (physical block, KV head), ``scale`` [NB, g]: code
    value times its block's scale (exact in float64)."""
    x = e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return x * sc[:, :, None, None]


def append_fp8_block_scaled(k_new, v_new, k_codes, v_codes, k_scale, v_scale, seq_lens_before,
                            block_table):
    """Quantise n new tokens per sequence (k_new, v_new [B,g,n,d] bf16) into
    paged pools [NB,g,bs,d] with per-(block, KV head) scales [NB, g]: token t
    of sequence b goes to position seq_lens_before[b] + t as the code of the
    float32 quotient x / scale[blk, j] of its target block.  Positions whose
    table entry is not a block of the pool are skipped.  Returns new pools."""
    kc = np.array(k_codes, dtype=np.uint8, copy=True)
    vc = np.array(v_codes, dtype=np.uint8, copy=True)
    ks = np.asarray(k_scale, dtype=np.float32)
    vs = np.asarray(v_scale, dtype=np.float32)
    before = _i32(seq_lens_before)
    bt = _i32(block_table)
    nb, g, bs, _ = kc.shape

    def floats(x):
        a, code = _raw(x)
        return (a.astype(np.uint32) << 16).view(np.float32) if code == BF16 else a
    kf, vf = floats(k_new), floats(v_new)
    B, _, n, _ = kf.shape
    for b in range(B):
        for t in range(n):
            p = int(before[b]) + t
            if p // bs >= bt.shape[1]:
                continue
            blk = int(bt[b, p // bs])
            if not 0 <= blk < nb:
                continue
            for j in range(g):
                kc[blk, j, p % bs] = e4m3_encode((kf[b, j, t] / ks[blk, j]).astype(np.float32))
                vc[blk, j, p % bs] = e4m3_encode((vf[b, j, t] / vs[blk, j]).astype(np.float32))
    return kc, vc


def decode_fp8_block_scaled(q, k_codes, v_codes, k_scale, v_scale, seq_lens_before, scale,
                            block_table, block_size, window=0, nthreads=0):
    """n query tokens per sequence (q [B,h,n,d] bf16) over paged FP8 pools
    with per-(block, KV head) scales that already hold them: dequantise
    (``dequantize_fp8_blocks``), then ``decode_window`` over the values.
    Returns out [B,h,n,d], lse [B,h,n]."""
    k = dequantize_fp8_blocks(k_codes, k_scale)
    v = dequantize_fp8_blocks(v_codes, v_scale)
    return decode_window(widen(q), k, v, seq_lens_before, scale, window, block_table=block_table,
                         block_size=block_size, nthreads=nthreads)
