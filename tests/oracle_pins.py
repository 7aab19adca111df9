"""Pins that tie the CPU fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees.  They
are run by tests/test_oracle.py directly and again by the mutation test,
which plants plausible mistakes in copies of the oracle source and checks that
at least one pin fails for every mistake.

Pages:
  [P1] "大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com)
  [P2] "从KV cache共享到批量调度：注意力机制下的隔离问题与口令实验" (0539edu.com)
  [P3] "每生成一个词为何又重算全文？KV Cache 的增量解码" (zwjcode.cn)
  [P4] "KV Cache 优化与注意力机制加速：FlashAttention / PagedAttention" (plumephp.com)
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import kvc_workloads as W
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f64(t):
    return t.to(torch.float64)


def sdpa_reference(q, k, v, lengths, scale):
    """torch scaled_dot_product_attention in fp64 on the CPU, GQA through
    ``enable_gqa`` ([P3] section 06 and 15), invalid positions masked out.
    q [B,h,d], k/v [B,g,T,d]; returns out [B,h,d], and lse computed by
    torch.logsumexp over the masked scores (library routines only)."""
    B, h, d = q.shape
    T = k.shape[2]
    qq = _f64(q).unsqueeze(2)                  # [B,h,1,d]
    kk, vv = _f64(k), _f64(v)
    valid = torch.arange(T).view(1, T) < torch.as_tensor(lengths).view(-1, 1)  # [B,T]
    mask = valid.view(B, 1, 1, T)
    out = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale,
                                         enable_gqa=True).squeeze(2)
    g = k.shape[1]
    kx = kk.repeat_interleave(h // g, dim=1)   # [B,h,T,d]
    scores = torch.matmul(qq, kx.transpose(-1, -2).contiguous()).squeeze(2) * scale  # [B,h,T]
    scores = scores.masked_fill(~valid.view(B, 1, T), float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return out.numpy(), lse.numpy()


# ----------------------------------------------------------------------------
# [P3] section 04: the d = 1 worked example.
def pin_d1_worked_example():
    g = _golden("d1_worked_example.json")
    k = np.zeros((1, 1, 4, 1), np.float32)
    v = np.zeros((1, 1, 4, 1), np.float32)
    k[0, 0, :2, 0] = g["k_prefill"]
    v[0, 0, :2, 0] = g["v_prefill"]
    kc, vc = oracle.append(np.full((1, 1, 1), g["k_new"], np.float32),
                           np.full((1, 1, 1), g["v_new"], np.float32), k, v, [2])
    assert kc[0, 0, :3, 0].tolist() == g["k_after_append"]
    assert vc[0, 0, :3, 0].tolist() == g["v_after_append"]
    out, lse = oracle.decode(np.full((1, 1, 1), g["q"], np.float32), kc, vc, [3], g["scale"])
    tol_o = 0.5 * 10 ** (-g["output_printed_decimals"])
    assert abs(out[0, 0, 0] - g["output_printed"]) <= tol_o, out[0, 0, 0]
    # The softmax weights themselves: with V = identity rows, out = weights.
    kk = np.zeros((1, 1, 3, 3), np.float32)
    kk[0, 0, :, 0] = g["k_after_append"]
    eye = np.eye(3, dtype=np.float32).reshape(1, 1, 3, 3)
    qq = np.array([[[g["q"], 0.0, 0.0]]], np.float32)
    w, _ = oracle.decode(qq, kk, eye, [3], g["scale"])
    tol_w = 0.5 * 10 ** (-g["softmax_printed_decimals"])
    assert np.all(np.abs(w[0, 0] - np.array(g["softmax_printed"])) <= tol_w), w[0, 0]
    # The page's own arithmetic: o = sum(printed weight * V) = printed output.
    assert abs(float(np.dot(g["softmax_printed"], g["v_after_append"])) - g["output_printed"]) < 1e-9
    # lse = ln(sum exp(scores)) for the printed scores.
    assert abs(lse[0, 0] - math.log(sum(math.exp(s) for s in g["scores_printed"]))) < 1e-12


# ----------------------------------------------------------------------------
# Library cross-check: fp64 SDPA with enable_gqa ([P3] sections 06, 15).
def pin_sdpa_crosscheck():
    cases = [
        (W.WORKLOADS["tiny_gqa_f32"], None),
        (W.Workload("t1", B=3, h=8, g=2, d=32, dtype="bf16", T_range=(1, 70), seed=11), None),
        (W.Workload("t2", B=2, h=6, g=6, d=8, dtype="f32", T=17, seed=12), None),
        (W.Workload("t3", B=2, h=5, g=1, d=64, dtype="bf16", T=40, seed=13), None),
    ]
    for w, _ in cases:
        x = W.make_contiguous(w)
        L = x["seq_lens_before"]
        out, lse = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
        sc = float(np.float32(x["scale"]))
        ro, rl = sdpa_reference(x["q"], x["k_cache"], x["v_cache"], L, sc)
        assert np.max(np.abs(out - ro)) < 1e-12, (w.name, np.max(np.abs(out - ro)))
        assert np.max(np.abs(lse - rl)) < 1e-12, (w.name, np.max(np.abs(lse - rl)))


# ----------------------------------------------------------------------------
# [P1] section 三 3.3 and the repeat_kv helper of section 四 4.1: GQA(h, g) on
# the cache equals MHA(h, h) on the cache with every KV head repeated m times
# (contiguous groups), bit for bit.
def pin_gqa_equals_mha_on_expanded_cache():
    w = W.Workload("e", B=2, h=12, g=3, d=16, dtype="bf16", T_range=(5, 50), seed=21)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    o1, l1 = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    m = w.h // w.g
    ke = x["k_cache"].repeat_interleave(m, dim=1).contiguous()
    ve = x["v_cache"].repeat_interleave(m, dim=1).contiguous()
    o2, l2 = oracle.decode(x["q"], ke, ve, L, x["scale"])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# [P4] section 5.1: MQA has one KV head; every query head is then a plain
# single-head attention over that head.
def pin_mqa_is_per_head_single_attention():
    w = W.Workload("mq", B=2, h=4, g=1, d=8, dtype="f32", T=9, seed=22)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    o, l = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    for i in range(w.h):
        oi, li = oracle.decode(x["q"][:, i:i + 1].contiguous(), x["k_cache"], x["v_cache"], L,
                               x["scale"])
        assert np.array_equal(o[:, i], oi[:, 0]) and np.array_equal(l[:, i], li[:, 0])


# MHA (g = h): head i reads KV head i, i.e. a plain batched single-head attention.
def pin_mha_head_i_reads_kv_head_i():
    w = W.Workload("mh", B=1, h=3, g=3, d=4, dtype="f32", T=6, seed=23)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    o, _ = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    for i in range(w.h):
        oi, _ = oracle.decode(x["q"][:, i:i + 1].contiguous(),
                              x["k_cache"][:, i:i + 1].contiguous(),
                              x["v_cache"][:, i:i + 1].contiguous(), L, x["scale"])
        assert np.array_equal(o[:, i], oi[:, 0])


# ----------------------------------------------------------------------------
# [P4] sections 4.2-4.3: the paged layout holds the same logical cache, so the
# result equals the contiguous one exactly.
def pin_paged_equals_contiguous():
    bs = 16
    w = W.Workload("pg", B=4, h=8, g=2, d=16, dtype="bf16", T_range=(1, 60), seed=31)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    table, nb = W.make_block_table(L, bs, perm_seed=32, extra_blocks=3)
    kp = W.scatter_to_pool(x["k_cache"], L, table, nb, bs)
    vp = W.scatter_to_pool(x["v_cache"], L, table, nb, bs)
    o1, l1 = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    o2, l2 = oracle.decode(x["q"], kp, vp, L, x["scale"], block_table=table, block_size=bs)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # block size other than 16 ([P2] section 5.3 names 8 and 32 too)
    for bs2 in (8, 32):
        t2, nb2 = W.make_block_table(L, bs2, perm_seed=33)
        kp2 = W.scatter_to_pool(x["k_cache"], L, t2, nb2, bs2)
        vp2 = W.scatter_to_pool(x["v_cache"], L, t2, nb2, bs2)
        o3, l3 = oracle.decode(x["q"], kp2, vp2, L, x["scale"], block_table=t2, block_size=bs2)
        assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


# ----------------------------------------------------------------------------
# [P3] section 07: decoding token by token over the cache reproduces every
# row of a full causal forward.  The full forward is torch SDPA in fp64 with
# is_causal=True (square, so its alignment is unambiguous).
def pin_incremental_equals_full_causal():
    for (N, H, G, T, d, seed) in [(2, 4, 4, 6, 4, 0), (2, 8, 2, 9, 8, 1)]:
        gen = torch.Generator().manual_seed(seed)
        q = torch.randn(N, H, T, d, generator=gen)
        k = torch.randn(N, G, T, d, generator=gen)
        v = torch.randn(N, G, T, d, generator=gen)
        sc = float(np.float32(1.0 / math.sqrt(d)))
        full = F.scaled_dot_product_attention(_f64(q), _f64(k), _f64(v), is_causal=True,
                                              scale=sc, enable_gqa=True).numpy()
        kc = np.zeros((N, G, T, d), np.float32)
        vc = np.zeros((N, G, T, d), np.float32)
        for t in range(T):
            before = [t] * N
            kc, vc = oracle.append(k[:, :, t].contiguous(), v[:, :, t].contiguous(), kc, vc, before)
            o, _ = oracle.decode(q[:, :, t].contiguous(), kc, vc, [t + 1] * N, sc)
            assert np.max(np.abs(o - full[:, :, t])) < 1e-12, (t, np.max(np.abs(o - full[:, :, t])))
        # after T steps the cache holds every position ([P3] section 07 checks
        # the cache shape (2, 4, 6, 4) for its 2 x 6 x 16 input with 4 heads)
        assert np.array_equal(kc, k.numpy()) and np.array_equal(vc, v.numpy())
        if (N, H, T, d) == (2, 4, 6, 4):
            assert kc.shape == (2, 4, 6, 4)


# ----------------------------------------------------------------------------
# [P4] sections 2.2, 2.3, 2.5: chunked partial results merged by log-sum-exp
# equal the unsplit result.
def pin_split_merge_equals_unsplit():
    w = W.Workload("sp", B=3, h=4, g=2, d=16, dtype="bf16", T_range=(0, 130), seed=41)
    lengths = torch.tensor([0, 1, 130], dtype=torch.int32)
    x = W.make_contiguous(w, lengths=lengths)
    L = x["seq_lens_before"]
    o, l = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    for chunk in (1, 2, 7, 64, 130, 1000):
        os_, ls = oracle.decode_split(x["q"], x["k_cache"], x["v_cache"], L, x["scale"], chunk)
        assert np.max(np.abs(os_ - o)) < 1e-13, chunk
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(ls))
        assert np.max(np.abs(ls[fin] - l[fin])) < 1e-13, chunk


# ----------------------------------------------------------------------------
# Closed forms of the softmax definition ([P4] section 2.2).
def pin_closed_forms():
    w = W.Workload("cf", B=2, h=4, g=2, d=8, dtype="f32", T_range=(3, 40), seed=51)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    # scale = 0: uniform weights, out = mean of the valid V rows, lse = ln L.
    o, l = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, 0.0)
    for b in range(w.B):
        Lb = int(L[b])
        for i in range(w.h):
            j = i * w.g // w.h
            mean = x["v_cache"][b, j, :Lb].double().mean(0).numpy()
            assert np.max(np.abs(o[b, i] - mean)) < 1e-12
            assert abs(l[b, i] - math.log(Lb)) < 1e-12
    # every V row equal to one vector v: out = v whatever the scores.
    vc = x["v_cache"].clone()
    vrow = torch.randn(w.B, w.g, 1, w.d, generator=torch.Generator().manual_seed(52))
    vc[:] = vrow
    o, _ = oracle.decode(x["q"], x["k_cache"], vc, L, x["scale"])
    for b in range(w.B):
        for i in range(w.h):
            assert np.max(np.abs(o[b, i] - vrow[b, i * w.g // w.h, 0].double().numpy())) < 1e-12
    # needle: one key aligned with q at a large multiple; its weight is
    # 1/(1 + sum_{p != n} exp(s_p - s_n)), so out is V[n] up to that bound.
    kc = x["k_cache"].clone()
    for b in range(w.B):
        Lb = int(L[b])
        n = (7 * b + 3) % Lb
        for j in range(w.g):
            qs = x["q"][b, j * (w.h // w.g)]
            kc[b, j, n] = 60.0 * qs / qs.norm()
    o, _ = oracle.decode(x["q"], kc, x["v_cache"], L, x["scale"])
    for b in range(w.B):
        Lb = int(L[b])
        n = (7 * b + 3) % Lb
        for j in range(w.g):
            i = j * (w.h // w.g)
            assert np.max(np.abs(o[b, i] - x["v_cache"][b, j, n].double().numpy())) < 1e-6


# A sequence of length 0 ([P2] section 3.3 warns that one empty request can
# corrupt a whole batch): its rows are 0 with lse = -inf and the other
# sequences are unaffected.
def pin_zero_length_rows():
    w = W.Workload("z", B=3, h=4, g=2, d=8, dtype="bf16", T=10, seed=61)
    lengths = torch.tensor([10, 0, 7], dtype=torch.int32)
    x = W.make_contiguous(w, lengths=lengths)
    o, l = oracle.decode(x["q"], x["k_cache"], x["v_cache"], lengths, x["scale"])
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(l[1]))
    for b in (0, 2):
        ob, lb = oracle.decode(x["q"][b:b + 1].contiguous(), x["k_cache"][b:b + 1].contiguous(),
                               x["v_cache"][b:b + 1].contiguous(), lengths[b:b + 1], x["scale"])
        assert np.array_equal(o[b], ob[0]) and np.array_equal(l[b], lb[0])


# Positions at or beyond a sequence's length are never read ([P3] section
# 10): poisoning them with NaN changes nothing.
def pin_unwritten_slots_invisible():
    w = W.Workload("u", B=2, h=4, g=2, d=8, dtype="bf16", T_range=(1, 30), seed=71)
    x0 = W.make_contiguous(w, fill=0.0)
    xn = W.make_contiguous(w, fill=float("nan"))
    L = x0["seq_lens_before"]
    o0, l0 = oracle.decode(x0["q"], x0["k_cache"], x0["v_cache"], L, x0["scale"])
    o1, l1 = oracle.decode(xn["q"], xn["k_cache"], xn["v_cache"], L, xn["scale"])
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


# ----------------------------------------------------------------------------
# Append ([P1] section 四 4.1 concat along the sequence axis; [P3] section 08
# position = current cache length): exactly the target slots change.
def pin_append_writes_only_target_slots():
    w = W.Workload("ap", B=3, h=4, g=2, d=8, dtype="bf16", T_range=(0, 40), seed=81)
    lengths = torch.tensor([0, 15, 40], dtype=torch.int32)
    x = W.make_contiguous(w, lengths=lengths, t_cap=48)
    kc, vc = oracle.append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], lengths)
    k0 = x["k_cache"].view(torch.int16).numpy().view(np.uint16)
    v0 = x["v_cache"].view(torch.int16).numpy().view(np.uint16)
    kn = x["k_new"].view(torch.int16).numpy().view(np.uint16)
    vn = x["v_new"].view(torch.int16).numpy().view(np.uint16)
    expect_k, expect_v = k0.copy(), v0.copy()
    for b in range(w.B):
        expect_k[b, :, int(lengths[b])] = kn[b]
        expect_v[b, :, int(lengths[b])] = vn[b]
    assert np.array_equal(kc, expect_k) and np.array_equal(vc, expect_v)
    # paged: the slot is block_table[b, pos // bs], offset pos % bs
    bs = 16
    table, nb = W.make_block_table(lengths + 1, bs, perm_seed=82)
    kp = W.scatter_to_pool(x["k_cache"], lengths, table, nb, bs)
    vp = W.scatter_to_pool(x["v_cache"], lengths, table, nb, bs)
    kp2, vp2 = oracle.append(x["k_new"], x["v_new"], kp, vp, lengths, block_table=table)
    ek = kp.view(torch.int16).numpy().view(np.uint16).copy()
    ev = vp.view(torch.int16).numpy().view(np.uint16).copy()
    for b in range(w.B):
        pos = int(lengths[b])
        phys = int(table[b, pos // bs])
        ek[phys, :, pos % bs] = kn[b]
        ev[phys, :, pos % bs] = vn[b]
    assert np.array_equal(kp2, ek) and np.array_equal(vp2, ev)


# ----------------------------------------------------------------------------
# Brute force on the tiny workload: plain Python floats, one position at a
# time, straight from softmax(q K^T scale) V.
def pin_tiny_brute_force():
    w = W.WORKLOADS["tiny_gqa_f32"]
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    o, l = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, x["scale"])
    q = x["q"].double().tolist()
    K = x["k_cache"].double().tolist()
    V = x["v_cache"].double().tolist()
    sc = float(np.float32(x["scale"]))
    for b in range(w.B):
        for i in range(w.h):
            j = i // (w.h // w.g)
            s = [sc * sum(a * c for a, c in zip(q[b][i], K[b][j][p])) for p in range(int(L[b]))]
            e = [math.exp(z) for z in s]
            tot = sum(e)
            ref = [sum(e[p] * V[b][j][p][k] for p in range(len(e))) / tot for k in range(w.d)]
            assert max(abs(a - c) for a, c in zip(o[b, i], ref)) < 1e-12
            assert abs(l[b, i] - math.log(tot)) < 1e-12


# The scale enters as the float32 value the GPU receives.
def pin_scale_is_float32_value():
    w = W.Workload("s32", B=1, h=2, g=1, d=4, dtype="f32", T=5, seed=91)
    x = W.make_contiguous(w)
    L = x["seq_lens_before"]
    o1, l1 = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, 0.1)
    o2, l2 = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, float(np.float32(0.1)))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.decode(x["q"], x["k_cache"], x["v_cache"], L, 0.2)
    assert not np.array_equal(l1, l3)


# ----------------------------------------------------------------------------
# Several new tokens at once ([P1] 5.2: prefill of new tokens after a cached
# prefix; [P4] 5.3: draft tokens verified in one pass).  Appending them after
# the prefix and attending with each token's own visible length reproduces
# the last rows of a full causal forward over prefix + new tokens (torch SDPA
# in fp64, is_causal on the square problem, so its alignment is unambiguous);
# lse matches torch.logsumexp over the same causal scores.  Paged = contiguous.
def pin_multi_query_equals_causal_prefill():
    for (N, H, G, P, n, d, seed) in [(2, 8, 2, 7, 5, 8, 10), (1, 4, 4, 0, 6, 4, 11),
                                     (3, 6, 1, 20, 1, 16, 12), (2, 4, 2, 33, 3, 8, 13)]:
        gen = torch.Generator().manual_seed(seed)
        S = P + n
        q = torch.randn(N, H, S, d, generator=gen)
        k = torch.randn(N, G, S, d, generator=gen)
        v = torch.randn(N, G, S, d, generator=gen)
        sc = float(np.float32(1.0 / math.sqrt(d)))
        full = F.scaled_dot_product_attention(_f64(q), _f64(k), _f64(v), is_causal=True,
                                              scale=sc, enable_gqa=True).numpy()
        kx = _f64(k).repeat_interleave(H // G, dim=1)
        scores = torch.matmul(_f64(q), kx.transpose(-1, -2).contiguous()) * sc      # [N,H,S,S]
        causal = torch.ones(S, S, dtype=torch.bool).tril()
        full_lse = torch.logsumexp(scores.masked_fill(~causal, float("-inf")), dim=-1).numpy()
        t_cap = S + 3
        kc = np.zeros((N, G, t_cap, d), np.float32)
        vc = np.zeros((N, G, t_cap, d), np.float32)
        kc[:, :, :P] = k[:, :, :P].numpy()
        vc[:, :, :P] = v[:, :, :P].numpy()
        before = [P] * N
        kc, vc = oracle.append_multi(k[:, :, P:].contiguous(), v[:, :, P:].contiguous(), kc, vc,
                                     before)
        assert np.array_equal(kc[:, :, :S], k.numpy()) and np.array_equal(vc[:, :, :S], v.numpy())
        assert not kc[:, :, S:].any() and not vc[:, :, S:].any()
        o, l = oracle.decode_multi(q[:, :, P:].contiguous(), kc, vc, before, sc)
        assert np.max(np.abs(o - full[:, :, P:])) < 1e-12, np.max(np.abs(o - full[:, :, P:]))
        assert np.max(np.abs(l - full_lse[:, :, P:])) < 1e-12
        # paged: the same logical cache through a shuffled block table
        lens = torch.full((N,), S, dtype=torch.int32)
        table, nb = W.make_block_table(lens, 4, perm_seed=seed, extra_blocks=2)
        kp = W.scatter_to_pool(torch.from_numpy(kc), lens, table, nb, 4)
        vp = W.scatter_to_pool(torch.from_numpy(vc), lens, table, nb, 4)
        op, lp = oracle.decode_multi(q[:, :, P:].contiguous(), kp, vp, before, sc,
                                     block_table=table, block_size=4)
        assert np.array_equal(op, o) and np.array_equal(lp, l)


# ----------------------------------------------------------------------------
# Sliding window ([P4] 5.2; [P3] section 10): the token at position x sees the
# last `window` positions up to x.  Pinned by (1) the plain definition on a
# cache cut down to those positions, (2) a window at least as long as the
# context equal to full attention, (3) a window of 1: out is the token's own
# V and lse its own score, (4) a ring cache of t_cap slots (position p in
# slot p mod t_cap) filled step by step gives the linear cache's results.
def _truncated_decode(q_t, k, v, lo, hi, scale):
    """Single-token attention over positions [lo[b], hi[b]) by copying them
    to the front of a fresh cache and attending to all of it."""
    B, g, _, d = k.shape
    L = max(int(max(hi - lo)), 1)
    kt = torch.zeros(B, g, L, d, dtype=k.dtype)
    vt = torch.zeros(B, g, L, d, dtype=v.dtype)
    for b in range(B):
        kt[b, :, : hi[b] - lo[b]] = k[b, :, lo[b]:hi[b]]
        vt[b, :, : hi[b] - lo[b]] = v[b, :, lo[b]:hi[b]]
    return oracle.decode(q_t, kt, vt, torch.as_tensor(hi - lo, dtype=torch.int32), scale)


def pin_sliding_window():
    gen = torch.Generator().manual_seed(21)
    B, h, g, d, n, t_cap = 4, 6, 2, 8, 3, 64
    before = np.array([0, 5, 17, 50], dtype=np.int32)
    q = torch.randn(B, h, n, d, generator=gen)
    k = torch.randn(B, g, t_cap, d, generator=gen)
    v = torch.randn(B, g, t_cap, d, generator=gen)
    sc = float(np.float32(0.3))
    for window in (1, 2, 7, 16, 53):
        o, l = oracle.decode_window(q, k, v, before, sc, window)
        for t in range(n):
            hi = before + t + 1
            lo = np.maximum(hi - window, 0)
            ot, lt = _truncated_decode(q[:, :, t].contiguous(), k, v, lo, hi, sc)
            assert np.array_equal(o[:, :, t], ot) and np.array_equal(l[:, :, t], lt), (window, t)
            if window == 1:
                for b in range(B):
                    x = hi[b] - 1
                    for i in range(h):
                        j = i * g // h
                        assert np.array_equal(o[b, i, t], v[b, j, x].double().numpy())
                        s = sc * float(torch.dot(q[b, i, t].double(), k[b, j, x].double()))
                        assert abs(l[b, i, t] - s) < 1e-12
    o_full, l_full = oracle.decode_multi(q, k, v, before, sc)
    o_w, l_w = oracle.decode_window(q, k, v, before, sc, 10 ** 6)
    assert np.array_equal(o_full, o_w) and np.array_equal(l_full, l_w)
    o_0, l_0 = oracle.decode_window(q, k, v, before, sc, 0)
    assert np.array_equal(o_full, o_0) and np.array_equal(l_full, l_0)


def pin_ring_cache_equals_linear():
    gen = torch.Generator().manual_seed(22)
    B, h, g, d, window, steps, n = 2, 4, 2, 8, 5, 12, 2
    for t_cap in (window + n - 1, window + n + 2):
        lin_k = np.zeros((B, g, steps * n + 4, d), np.float32)
        lin_v = np.zeros_like(lin_k)
        ring_k = np.zeros((B, g, t_cap, d), np.float32)
        ring_v = np.zeros_like(ring_k)
        before = np.array([0, 3], dtype=np.int32)
        for step in range(steps):
            kn = torch.randn(B, g, n, d, generator=gen)
            vn = torch.randn(B, g, n, d, generator=gen)
            q = torch.randn(B, h, n, d, generator=gen)
            lin_k, lin_v = oracle.append_window(kn, vn, lin_k, lin_v, before)
            ring_k, ring_v = oracle.append_window(kn, vn, ring_k, ring_v, before, ring=True)
            o1, l1 = oracle.decode_window(q, lin_k, lin_v, before, 0.5, window)
            o2, l2 = oracle.decode_window(q, ring_k, ring_v, before, 0.5, window, ring=True)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), (t_cap, step)
            # the ring holds exactly the last t_cap positions of each sequence
            for b in range(B):
                end = before[b] + n
                for p in range(max(0, end - t_cap), end):
                    assert np.array_equal(ring_k[b, :, p % t_cap], lin_k[b, :, p])
            before = before + n


# ----------------------------------------------------------------------------
# Shared prefixes with copy-on-write ([P4] 4.3; [P2] 3.2: a shared block is
# copied before a request writes into it, so requests never see each other's
# tokens) and beam re-ranking ([P3] 11).  Three requests fork one prompt's
# block table; each appends its own tokens, copying the last shared block
# first; every request's attention equals attention over its own private
# contiguous cache, and the prompt blocks stay shared and unchanged.
def pin_fork_copy_on_write_isolation():
    gen = torch.Generator().manual_seed(31)
    g, d, h, bs, P = 2, 8, 4, 4, 10          # 10-token prompt: blocks 0, 1 full, 2 partial
    prompt_k = torch.randn(g, P, d, generator=gen)
    prompt_v = torch.randn(g, P, d, generator=gen)
    nb = 12
    kp = np.zeros((nb, g, bs, d), np.float32)
    vp = np.zeros_like(kp)
    for lb in range(3):
        n = min(bs, P - lb * bs)
        kp[lb, :, :n] = prompt_k[:, lb * bs: lb * bs + n].numpy()
        vp[lb, :, :n] = prompt_v[:, lb * bs: lb * bs + n].numpy()
    table0 = np.array([[0, 1, 2, -1]], np.int32)
    tables, lens = oracle.fork_tables(table0, [P], [0, 0, 0])
    assert np.array_equal(tables, np.repeat(table0, 3, 0)) and list(lens) == [P] * 3
    # requests 1 and 2 write into the shared block 2: copy it first (COW)
    kp, vp = oracle.copy_blocks(kp, vp, [(2, 3), (2, 4)])
    tables[1, 2], tables[2, 2] = 3, 4
    new_k = torch.randn(3, g, 1, d, generator=gen)
    new_v = torch.randn(3, g, 1, d, generator=gen)
    kp, vp = oracle.append_multi(new_k, new_v, kp, vp, lens, block_table=tables)
    # blocks 0 and 1 are still shared and hold the prompt; block 2 holds
    # request 0's token, blocks 3 and 4 the others'
    for lb in range(2):
        assert np.array_equal(kp[lb], prompt_k[:, lb * bs:(lb + 1) * bs].numpy())
    q = torch.randn(3, h, 1, d, generator=gen)
    o, l = oracle.decode_multi(q, kp, vp, lens, 0.5, block_table=tables, block_size=bs)
    for r in range(3):
        kc = torch.cat([prompt_k, new_k[r, :, :, :]], 1).unsqueeze(0).contiguous()
        vc = torch.cat([prompt_v, new_v[r, :, :, :]], 1).unsqueeze(0).contiguous()
        orr, lr = oracle.decode(q[r:r + 1, :, 0].contiguous(), kc, vc, [P + 1], 0.5)
        assert np.array_equal(o[r:r + 1, :, 0], orr) and np.array_equal(l[r:r + 1, :, 0], lr)
    # out-of-pool pairs are skipped; copying a block onto itself changes nothing
    kq, vq = oracle.copy_blocks(kp, vp, [(0, nb), (-1, 5), (1, 1)])
    assert np.array_equal(kq, kp) and np.array_equal(vq, vp)


def pin_beam_gather():
    gen = torch.Generator().manual_seed(32)
    B, g, T, d = 4, 2, 9, 4
    kc = torch.randn(B, g, T, d, generator=gen)
    vc = torch.randn(B, g, T, d, generator=gen)
    lens = torch.tensor([9, 3, 0, 6], dtype=torch.int32)
    parent = [3, 3, 0, 1, 2]
    ko, vo = oracle.gather_cache(kc, vc, parent, lens)
    assert ko.shape == (5, g, T, d)
    for b, pb in enumerate(parent):
        L = int(lens[pb])
        assert np.array_equal(ko[b, :, :L], kc[pb, :, :L].numpy())
        assert not ko[b, :, L:].any() and not vo[b, :, L:].any()
        assert np.array_equal(vo[b, :, :L], vc[pb, :, :L].numpy())
    # re-ranked beams attend to their parents' histories
    q = torch.randn(5, 4, d, generator=gen)
    o, l = oracle.decode(q, ko, vo, lens[parent], 0.7)
    for b, pb in enumerate(parent):
        o1, l1 = oracle.decode(q[b:b + 1], kc[pb:pb + 1].contiguous(), vc[pb:pb + 1].contiguous(),
                               lens[pb:pb + 1], 0.7)
        assert np.array_equal(o[b:b + 1], o1) and np.array_equal(l[b:b + 1], l1)
    # the paged form: forking the block tables by parent (no data moves)
    # gives the same attention as gathering the contiguous caches
    table, nb = W.make_block_table(lens, 4, perm_seed=33, extra_blocks=1)
    kp = W.scatter_to_pool(kc, lens, table, nb, 4)
    vp = W.scatter_to_pool(vc, lens, table, nb, 4)
    ft, fl = oracle.fork_tables(table, lens, parent)
    assert list(fl) == [int(lens[pb]) for pb in parent]
    op, lp = oracle.decode(q, kp, vp, fl, 0.7, block_table=ft, block_size=4)
    assert np.array_equal(op, o) and np.array_equal(lp, l)


# ----------------------------------------------------------------------------
# FP8 E4M3 cache ([P4] 2.5: FP8 attention; [P3] 14: low-bit K/V).  The
# format's closed-form points, round trips, ties to even, saturation and the
# sign of zero; torch's own float8_e4m3fn conversion agrees wherever it is
# finite (below 464); attention over the dequantised caches equals torch SDPA
# in float64 over torch's dequantisation of the same codes.
def pin_fp8_format():
    v = oracle.e4m3_values()
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0xB8] == -1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and v[0x80] == 0 and np.signbit(v[0x80])
    assert np.all(np.diff(v[:127]) > 0)
    finite = [c for c in range(256) if not np.isnan(v[c])]
    assert np.array_equal(oracle.e4m3_encode(v[finite].astype(np.float32)), np.array(finite, np.uint8))
    enc = oracle.e4m3_encode
    assert list(enc([1.0625, 1.1875, 500.0, 1e30, 448.0, 460.0, -1e-9, 2.0 ** -10, 1.5 * 2.0 ** -10])) \
        == [0x38, 0x3A, 0x7E, 0x7E, 0x7E, 0x7E, 0x80, 0x00, 0x01]
    # every midpoint between neighbours, random values, against torch
    mids = ((v[:126] + v[1:127]) / 2).astype(np.float32)
    gen = torch.Generator().manual_seed(41)
    rnd = (torch.randn(20000, generator=gen) * torch.exp(torch.randn(20000, generator=gen) * 3))
    ys = np.concatenate([mids, -mids, rnd.numpy().astype(np.float32)])
    ys = ys[np.abs(ys) < 464]
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc(ys), ref)


def pin_fp8_dequantised_attention():
    gen = torch.Generator().manual_seed(42)
    B, h, g, T, d = 3, 8, 2, 50, 16
    q = torch.randn(B, h, d, generator=gen)
    k = torch.randn(B, g, T, d, generator=gen) * 3
    v = torch.randn(B, g, T, d, generator=gen) * 2
    ks = np.array([0.05, 0.2], np.float32)
    vs = np.array([0.01, 0.5], np.float32)
    kc = oracle.quantize_fp8(k, ks, 1)
    vc = oracle.quantize_fp8(v, vs, 1)
    # the codes are torch's conversion of the float32 quotient (all in range)
    kq = (k / torch.from_numpy(ks).view(1, g, 1, 1)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(kc, kq.numpy())
    lens = [50, 7, 1]
    sc = 0.25
    o, l = oracle.decode_fp8(q, kc, vc, ks, vs, lens, sc)
    kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(ks).double().view(1, g, 1, 1)
    vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(vs).double().view(1, g, 1, 1)
    ro, rl = sdpa_reference(q, kd, vd, lens, sc)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12
    # paged = contiguous; and the append writes the codes of the new token
    lt = torch.tensor(lens, dtype=torch.int32)
    table, nb = W.make_block_table(lt, 4, perm_seed=43, extra_blocks=1)
    kp = W.scatter_to_pool(torch.from_numpy(kc), lt, table, nb, 4).numpy()
    vp = W.scatter_to_pool(torch.from_numpy(vc), lt, table, nb, 4).numpy()
    op, lp = oracle.decode_fp8(q, kp, vp, ks, vs, lens, sc, block_table=table, block_size=4)
    assert np.array_equal(op, o) and np.array_equal(lp, l)
    kn = torch.randn(B, g, 1, d, generator=gen)
    k2, v2 = oracle.append_fp8(kn, kn, kc, vc, ks, vs, [6, 0, 1])
    for b, p in enumerate([6, 0, 1]):
        assert np.array_equal(k2[b, :, p], oracle.quantize_fp8(kn, ks, 1)[b, :, 0])
        assert np.array_equal(v2[b, :, p], oracle.quantize_fp8(kn, vs, 1)[b, :, 0])
    changed = (k2 != kc).any(axis=(1, 3))
    assert changed.sum() <= B * 1 and not changed[0, 7:].any()


def pin_fp8_multi_and_window():
    """Several tokens per sequence over FP8 caches (window 0), and with a
    sliding window and a ring cache: every token's row equals torch SDPA in
    float64 over torch's dequantisation of the positions it sees."""
    gen = torch.Generator().manual_seed(44)
    B, h, g, d, n = 3, 4, 2, 16, 5
    before = [0, 6, 23]
    t_cap = 32
    ks = np.array([0.04, 0.3], np.float32)
    vs = np.array([0.02, 0.6], np.float32)
    q = torch.randn(B, h, n, d, generator=gen).to(torch.bfloat16)
    kn = torch.randn(B, g, n, d, generator=gen).to(torch.bfloat16)
    vn = torch.randn(B, g, n, d, generator=gen).to(torch.bfloat16)
    kc0 = oracle.quantize_fp8(torch.randn(B, g, t_cap, d, generator=gen) * 2, ks, 1)
    vc0 = oracle.quantize_fp8(torch.randn(B, g, t_cap, d, generator=gen) * 3, vs, 1)
    kc, vc = oracle.append_fp8(kn, vn, kc0, vc0, ks, vs, before)
    # the n new codes are those of the bf16 rows, and nothing else moved
    for b in range(B):
        for t in range(n):
            assert np.array_equal(kc[b, :, before[b] + t], oracle.quantize_fp8(kn, ks, 1)[b, :, t])
    kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(ks).double().view(1, g, 1, 1)
    vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64) * \
        torch.from_numpy(vs).double().view(1, g, 1, 1)
    sc = 0.3
    qf = q.to(torch.float64)
    for window in (0, 1, 4, 100):
        o, l = oracle.decode_fp8_window(q, kc, vc, ks, vs, before, sc, window)
        for b in range(B):
            for t in range(n):
                x = before[b] + t
                lo = max(0, x + 1 - window) if window else 0
                for i in range(h):
                    j = i * g // h
                    s_ = (kd[b, j, lo:x + 1] @ qf[b, i, t]) * float(np.float32(sc))
                    w = torch.softmax(s_, 0)
                    ro = w @ vd[b, j, lo:x + 1]
                    assert torch.max(torch.abs(torch.from_numpy(o[b, i, t]) - ro)) < 1e-12
                    assert abs(l[b, i, t] - float(torch.logsumexp(s_, 0))) < 1e-12
    # a ring of 8 slots written step by step gives the linear cache's rows
    window, ring_cap = 4, 8
    kr = np.zeros((B, g, ring_cap, d), np.uint8)
    vr = np.zeros((B, g, ring_cap, d), np.uint8)
    lin_k = np.zeros((B, g, 64, d), np.uint8)
    lin_v = np.zeros((B, g, 64, d), np.uint8)
    lens = np.array([0, 2, 9], np.int32)
    for step in range(6):
        kn = torch.randn(B, g, 3, d, generator=gen).to(torch.bfloat16)
        vn = torch.randn(B, g, 3, d, generator=gen).to(torch.bfloat16)
        qs = torch.randn(B, h, 3, d, generator=gen).to(torch.bfloat16)
        kr, vr = oracle.append_fp8(kn, vn, kr, vr, ks, vs, lens, ring=True)
        lin_k, lin_v = oracle.append_fp8(kn, vn, lin_k, lin_v, ks, vs, lens)
        o1, l1 = oracle.decode_fp8_window(qs, kr, vr, ks, vs, lens, sc, window, ring=True)
        o2, l2 = oracle.decode_fp8_window(qs, lin_k, lin_v, ks, vs, lens, sc, window)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), step
        lens = lens + 3


def pin_fp8_block_scales():
    """Paged FP8 pools with a scale per (block, KV head): the appended codes
    are torch's float8_e4m3fn conversion of x / (its block's scale); with
    every block of a head at the head's scale the result equals the
    per-head reference exactly; with random block scales every row equals
    torch SDPA in float64 over torch's per-block dequantisation."""
    gen = torch.Generator().manual_seed(45)
    B, h, g, d, bs, n = 3, 4, 2, 16, 4, 3
    before = torch.tensor([0, 5, 10], dtype=torch.int32)
    table, nb = W.make_block_table(before + n, bs, perm_seed=46, extra_blocks=1)
    kc = oracle.quantize_fp8(torch.randn(nb, g, bs, d, generator=gen) * 2, np.ones(g, np.float32), 1)
    vc = kc.copy()[::-1].copy()
    kb = (torch.rand(nb, g, generator=gen) * 0.5 + 0.02).numpy().astype(np.float32)
    vb = (torch.rand(nb, g, generator=gen) * 0.5 + 0.02).numpy().astype(np.float32)
    kn = (torch.randn(B, g, n, d, generator=gen) * 0.3).to(torch.bfloat16)
    vn = (torch.randn(B, g, n, d, generator=gen) * 0.3).to(torch.bfloat16)
    k2, v2 = oracle.append_fp8_block_scaled(kn, vn, kc, vc, kb, vb, before, table)
    for b in range(B):
        for t in range(n):
            p = int(before[b]) + t
            blk = int(table[b, p // bs])
            want = (kn[b, :, t].float() / torch.from_numpy(kb[blk]).view(g, 1)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(k2[blk, :, p % bs], want)
    q = torch.randn(B, h, n, d, generator=gen).to(torch.bfloat16)
    sc = 0.35
    # all blocks of head j at that head's scale: the per-head reference
    hk = np.array([0.07, 0.4], np.float32)
    hv = np.array([0.3, 0.05], np.float32)
    o1, l1 = oracle.decode_fp8_block_scaled(q, k2, v2, np.tile(hk, (nb, 1)), np.tile(hv, (nb, 1)),
                                            before, sc, table, bs)
    o2, l2 = oracle.decode_fp8_window(q, k2, v2, hk, hv, before, sc, 0, block_table=table,
                                      block_size=bs)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # random block scales against torch's per-block dequantisation
    o, l = oracle.decode_fp8_block_scaled(q, k2, v2, kb, vb, before, sc, table, bs)
    kd = torch.from_numpy(k2).view(torch.float8_e4m3fn).double() * \
        torch.from_numpy(kb).double().view(nb, g, 1, 1)
    vd = torch.from_numpy(v2).view(torch.float8_e4m3fn).double() * \
        torch.from_numpy(vb).double().view(nb, g, 1, 1)
    qf = q.double()
    for b in range(B):
        for t in range(n):
            x = int(before[b]) + t
            rows = [int(table[b, p // bs]) for p in range(x + 1)]
            for i in range(h):
                j = i * g // h
                kk = torch.stack([kd[rows[p], j, p % bs] for p in range(x + 1)])
                vv = torch.stack([vd[rows[p], j, p % bs] for p in range(x + 1)])
                s_ = (kk @ qf[b, i, t]) * float(np.float32(sc))
                ro = torch.softmax(s_, 0) @ vv
                assert torch.max(torch.abs(torch.from_numpy(o[b, i, t]) - ro)) < 1e-12
                assert abs(l[b, i, t] - float(torch.logsumexp(s_, 0))) < 1e-12


ALL_PINS = [
    pin_d1_worked_example,
    pin_sdpa_crosscheck,
    pin_gqa_equals_mha_on_expanded_cache,
    pin_mqa_is_per_head_single_attention,
    pin_mha_head_i_reads_kv_head_i,
    pin_paged_equals_contiguous,
    pin_incremental_equals_full_causal,
    pin_split_merge_equals_unsplit,
    pin_closed_forms,
    pin_zero_length_rows,
    pin_unwritten_slots_invisible,
    pin_append_writes_only_target_slots,
    pin_tiny_brute_force,
    pin_scale_is_float32_value,
    pin_multi_query_equals_causal_prefill,
    pin_sliding_window,
    pin_ring_cache_equals_linear,
    pin_fork_copy_on_write_isolation,
    pin_beam_gather,
    pin_fp8_format,
    pin_fp8_dequantised_attention,
    pin_fp8_multi_and_window,
    pin_fp8_block_scales,
]
