"""CPU-only: the fp64 oracle against its pins, the closed-form KV sizes, and
a mutation check that every planted mistake in the oracle fails a pin."""
from __future__ import annotations

import ctypes
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import kvc_workloads as W
import oracle
import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Closed-form KV cache sizes the pages print (tests/golden/kv_cache_sizes.json).
def test_kv_cache_bytes_printed_cases():
    with open(os.path.join(HERE, "golden", "kv_cache_sizes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        n = oracle.kv_cache_bytes(c["layers"], c["batch"], c["kv_heads"], c["tokens"],
                                  c["head_dim"], c["elem_bytes"])
        assert n == c["bytes_exact"], c["citation"]
        unit = c["printed_unit"]
        if unit.startswith("GB (read as GiB)"):
            assert n / 2 ** 30 == c["printed"], c["citation"]
        else:  # bytes / (1000 * 1024^2), printed to one decimal
            assert round(n / (1000 * 2 ** 20), 1) == c["printed"], c["citation"]


def test_kv_cache_bytes_exercise_and_ratios():
    # zwjcode.cn section 17 exercise: 24 layers, N=4, H=16, T=2048, d=64, fp16.
    elems = oracle.kv_cache_bytes(24, 4, 16, 2048, 64, 1)
    assert elems == 402_653_184
    assert oracle.kv_cache_bytes(24, 4, 16, 2048, 64, 2) == 3 * 2 ** 28  # 0.75 GiB
    assert oracle.kv_cache_bytes(24, 4, 4, 2048, 64, 2) * 4 == oracle.kv_cache_bytes(
        24, 4, 16, 2048, 64, 2)
    # limoncc.com section 三 3.3: h=64, g=8 shrinks the cache to 1/8;
    # plumephp.com section 5.1: MQA : GQA : MHA = 1 : 8 : 64.
    sizes = [oracle.kv_cache_bytes(80, 1, kv, 4096, 128, 2) for kv in (1, 8, 64)]
    assert sizes[1] == 8 * sizes[0] and sizes[2] == 64 * sizes[0]


def test_workload_caches_match_closed_form():
    """The allocated caches of the generated workloads hold exactly
    2 x B x g x capacity x d x elem_bytes bytes (one layer)."""
    w = W.WORKLOADS["tiny_gqa_f32"]
    x = W.make_contiguous(w)
    nbytes = x["k_cache"].numel() * 4 + x["v_cache"].numel() * 4
    assert nbytes == oracle.kv_cache_bytes(1, w.B, w.g, x["t_cap"], w.d, 4)
    w2 = W.Workload("p", B=3, h=4, g=2, d=8, dtype="bf16", T_range=(10, 40), paged=True, seed=5)
    xp = W.make_paged(w2)
    nb = xp["num_blocks"]
    assert xp["k_pool"].numel() * 2 * 2 == oracle.kv_cache_bytes(1, 1, w2.g, nb * 16, w2.d, 2)


# ----------------------------------------------------------------------------
# Mutation check: plant a plausible mistake in a copy of the oracle source,
# build it, and require that at least one pin fails.
MUTATIONS = {
    "head_map_mod_g": ("int j = (int)(((long)i * g) / h);", "int j = (int)(i % g);"),
    "drop_scale": ("s[p - p0] = scale * dot;", "s[p - p0] = dot;"),
    "exp_sign": ("double w = exp(s[p - p0] - m);", "double w = exp(m - s[p - p0]);"),
    "lse_drops_max": ("lse[bi] = m + log(l);", "lse[bi] = log(l);"),
    "len_off_by_one": ("starts ? starts[b] : 0, seq_lens[b], h, g, d, t_cap, scale, s, acc, &m, &l);",
                       "starts ? starts[b] : 0, seq_lens[b] - (seq_lens[b] > 1), h, g, d, t_cap, "
                       "scale, s, acc, &m, &l);"),
    "window_start_off_by_one": ("starts ? starts[b] : 0, seq_lens[b]",
                                "starts ? starts[b] + 1 : 0, seq_lens[b]"),
    "pv_reads_k": ("acc[k] += w * load_elem(vc, row * d + k, dtype);",
                   "acc[k] += w * load_elem(kc, row * d + k, dtype);"),
    "paged_offset": ("int offset = p % block_size;", "int offset = (p + 1) % block_size;"),
    # pool read as [num_blocks, block_size, g, d] instead of [num_blocks, g, block_size, d]
    "paged_pool_layout": ("return ((size_t)physical * g + j) * (size_t)block_size + (size_t)offset;",
                          "return ((size_t)physical * block_size + offset) * (size_t)g + (size_t)j;"),
    "append_pos_minus_one": ("int pos = seq_lens_before[b];",
                             "int pos = seq_lens_before[b] > 0 ? seq_lens_before[b] - 1 : 0;"),
    # contiguous K read as [B, g, d, t_cap] (transposed) instead of [B, g, t_cap, d]
    "k_transposed": ("dot += load_elem(q, qbase + k, dtype) * load_elem(kc, row * d + k, dtype);",
                     "dot += load_elem(q, qbase + k, dtype) * load_elem(kc, block_table ? row * d + k"
                     " : (((size_t)b * g + j) * d + k) * (size_t)t_cap + p, dtype);"),
    # q of head i read from head i + 1 (mod h): an index slip in the query operand
    "q_head_slip": ("size_t qbase = ((size_t)b * h + i) * (size_t)d;",
                    "size_t qbase = ((size_t)b * h + (i + 1) % h) * (size_t)d;"),
    "split_weight_no_exp": ("double w = exp(plse[c] - M);", "double w = plse[c] - M + 1.0;"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kvc_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutant = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutant)
    lib_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(lib_path), str(csrc),
                    "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle.configure(ctypes.CDLL(str(lib_path)))
    failed = []
    try:
        for pin in P.ALL_PINS:
            try:
                pin()
            except (AssertionError, Exception):  # noqa: BLE001 - any failure counts
                failed.append(pin.__name__)
    finally:
        oracle._lib = saved
    assert failed, f"no pin caught the planted mistake {name}"


# Plausible mistakes in the several-new-tokens composition (positions and
# visibility), each of which the multi-query pin must catch.  Every variant
# stays inside the pin's cache capacity (t_cap = prefix + n + 3).
MULTI_MUTATIONS = {
    "top_left_alignment": ("_multi_visible", lambda before, t: t + 1),
    "excludes_itself": ("_multi_visible", lambda before, t: before + t),
    "ignores_token_index": ("_multi_visible", lambda before, t: before + 1),
    "sees_next_token": ("_multi_visible", lambda before, t: before + t + 2),
    "append_shifted": ("_multi_position", lambda before, t: before + t + 1),
    "append_all_at_prefix_end": ("_multi_position", lambda before, t: before),
}


@pytest.mark.parametrize("name", sorted(MULTI_MUTATIONS))
def test_planted_multi_query_mistake_is_caught(name, monkeypatch):
    attr, fn = MULTI_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    with pytest.raises(Exception):
        P.pin_multi_query_equals_causal_prefill()


# Plausible mistakes in the window and ring compositions.
WINDOW_MUTATIONS = {
    "window_one_short": ("_window_start", lambda vis, w: np.maximum(vis - w + 1, 0) if w > 0
                         else np.zeros_like(vis)),
    "window_one_long": ("_window_start", lambda vis, w: np.maximum(vis - w - 1, 0) if w > 0
                        else np.zeros_like(vis)),
    "window_ignored": ("_window_start", lambda vis, w: np.zeros_like(vis)),
    "ring_slot_shifted": ("_ring_slot", lambda p, t_cap: (p + 1) % t_cap),
}


@pytest.mark.parametrize("name", sorted(WINDOW_MUTATIONS))
def test_planted_window_mistake_is_caught(name, monkeypatch):
    attr, fn = WINDOW_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    failed = 0
    for pin in (P.pin_sliding_window, P.pin_ring_cache_equals_linear):
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts
            failed += 1
    assert failed, f"no window pin caught {name}"


def _copy_blocks_k_only(k_pool, v_pool, pairs):
    kp, _ = oracle._raw(k_pool)
    vp, _ = oracle._raw(v_pool)
    kp, vp = kp.copy(), vp.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= src < kp.shape[0] and 0 <= dst < kp.shape[0]:
            kp[dst] = kp[src]
    return kp, vp


def _gather_whole_rows(k_cache, v_cache, parent, seq_lens):
    kc, _ = oracle._raw(k_cache)
    vc, _ = oracle._raw(v_cache)
    par = np.asarray(parent, dtype=np.int64)
    return kc[par].copy(), vc[par].copy()


def _fork_by_index(tables, seq_lens, parent):
    t = oracle._i32(tables)
    sl = oracle._i32(seq_lens)
    idx = np.arange(len(parent)) % t.shape[0]
    return t[idx].copy(), sl[idx].copy()


BLOCK_MUTATIONS = {
    "copy_blocks_k_only": ("copy_blocks", _copy_blocks_k_only),
    "gather_whole_rows": ("gather_cache", _gather_whole_rows),
    "fork_by_index": ("fork_tables", _fork_by_index),
}


@pytest.mark.parametrize("name", sorted(BLOCK_MUTATIONS))
def test_planted_block_op_mistake_is_caught(name, monkeypatch):
    attr, fn = BLOCK_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    failed = 0
    for pin in (P.pin_fork_copy_on_write_isolation, P.pin_beam_gather):
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts
            failed += 1
    assert failed, f"no block-op pin caught {name}"


def _encode_ties_odd(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    pos = oracle.e4m3_values()[:127]
    hi = np.minimum(np.searchsorted(pos, a, side="left"), 126)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (pos[hi] - a < a - pos[lo]) | ((pos[hi] - a == a - pos[lo]) & (hi % 2 == 1))
    code = np.where(pos[hi] == a, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return (code | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def _encode_no_saturation(y):
    y = np.asarray(y, dtype=np.float32)
    code = _ORIG_ENCODE(y)
    return np.where(np.abs(y) > 448, np.uint8(0x7F) | (code & 0x80), code).astype(np.uint8)


_ORIG_ENCODE = oracle.e4m3_encode


def _quantize_by_multiply(x, scale, head_axis):
    xa, xd = oracle._raw(x)
    xf = (xa.astype(np.uint32) << 16).view(np.float32) if xd == oracle.BF16 else xa
    sc = np.asarray(scale, dtype=np.float32)
    shape = [1] * xf.ndim
    shape[head_axis] = -1
    return oracle.e4m3_encode((xf * sc.reshape(shape)).astype(np.float32))


def _dequantize_dividing(codes, scale, head_axis):
    x = oracle.e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    return x / sc.reshape(shape)


def _dequantize_first_head_scale(codes, scale, head_axis):
    x = oracle.e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    return x * float(np.asarray(scale, dtype=np.float32)[0])


def _fp8_window_one_short(q, kc, vc, ks, vs, before, scale, window=0, ring=False,
                          block_table=None, block_size=16, nthreads=0):
    return _ORIG_FP8_WINDOW(q, kc, vc, ks, vs, before, scale, max(window - 1, 0) if window else 0,
                            ring=ring, block_table=block_table, block_size=block_size)


def _append_fp8_ring_shifted(k_new, v_new, kc, vc, ks, vs, before, block_table=None, ring=False):
    shift = 1 if ring else 0
    return _ORIG_APPEND_FP8(k_new, v_new, kc, vc, ks, vs, np.asarray(before) + shift,
                            block_table=block_table, ring=ring)


def _dequantize_blocks_head_scale(codes, scale):
    x = oracle.e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return x * sc[0][None, :, None, None]   # block 0's scales for every block


def _dequantize_blocks_transposed(codes, scale):
    x = oracle.e4m3_values()[np.asarray(codes, dtype=np.uint8)]
    sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
    nb, g = sc.shape
    return x * sc.T.reshape(-1)[: nb * g].reshape(nb, g)[:, :, None, None]


_ORIG_FP8_WINDOW = oracle.decode_fp8_window
_ORIG_APPEND_FP8 = oracle.append_fp8

FP8_MUTATIONS = {
    "ties_to_odd": ("e4m3_encode", _encode_ties_odd),
    "no_saturation": ("e4m3_encode", _encode_no_saturation),
    "scale_multiplies": ("quantize_fp8", _quantize_by_multiply),
    "dequantise_divides": ("dequantize_fp8", _dequantize_dividing),
    "dequantise_one_scale": ("dequantize_fp8", _dequantize_first_head_scale),
    "fp8_window_one_short": ("decode_fp8_window", _fp8_window_one_short),
    "fp8_ring_slot_shifted": ("append_fp8", _append_fp8_ring_shifted),
    "block_scales_of_block_0": ("dequantize_fp8_blocks", _dequantize_blocks_head_scale),
    "block_scales_transposed": ("dequantize_fp8_blocks", _dequantize_blocks_transposed),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    failed = 0
    for pin in (P.pin_fp8_format, P.pin_fp8_dequantised_attention, P.pin_fp8_multi_and_window,
                P.pin_fp8_block_scales):
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts
            failed += 1
    assert failed, f"no fp8 pin caught {name}"
