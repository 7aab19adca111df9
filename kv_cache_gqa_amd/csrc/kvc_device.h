// kvc_device.h -- device-side helpers shared by the libkvc kernels (gfx950,
// wave64).  Scores are kept in base 2: s2 = (scale * log2 e) * q.k, so that
// exp(s - m) = exp2(s2 - m2) maps onto v_exp_f32 directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_internal.h"

namespace kvc {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 pair (little-endian: element 2k in the low half) to two floats.  A
// bf16 value is the high half of the float with the same value.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves inside a row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<kDppMirror>(x);
    return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

// Max (sum) of x over the four lanes l, l^16, l^32, l^48 of a wavefront,
// every lane getting the result, with the gfx950 cross-row swaps instead of
// LDS permutes.  v_permlane16_swap of x with itself gives rows (0, 0, 2, 2)
// in its first result and (1, 1, 3, 3) in its second; v_permlane32_swap
// gives the low half twice and the high half twice.
__device__ __forceinline__ float max_rows4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16-byte global load through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (global_load_dwordx4 ... nt).  Every K/V byte of a
// decode step is read exactly once; marking the loads non-temporal keeps
// them from displacing useful cache lines and measured 6.7-6.9 TB/s on
// MI355X for this access pattern, against 5.9-6.1 TB/s for plain loads.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// 8-byte streaming load (global_load_dwordx2 ... nt).
__device__ __forceinline__ uint2 ld8_stream(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint2 ld8(const void* p) {
    return *reinterpret_cast<const uint2*>(p);
}

// ---- OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// no infinities, S.1111.111 = NaN, largest finite 448) ----

// Two codes (bytes 0-1 of w, or 2-3 when hi) as two bf16 in one 32-bit
// word, low half first.  Exact: every E4M3 value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    const auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// Eight codes (bytes of c, in order) as eight bf16.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c) {
    return make_uint4(e4m3x2_to_bf16x2<false>(c.x), e4m3x2_to_bf16x2<true>(c.x),
                      e4m3x2_to_bf16x2<false>(c.y), e4m3x2_to_bf16x2<true>(c.y));
}

// One code as float.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}

// Code of a float: the nearest E4M3 value with ties to the even code,
// magnitudes above 448 saturating to 448, NaN to S.1111.111, the sign kept
// (also for values that round to zero).  Below 2^-6 the values are the
// multiples of 2^-9, so the code is rint(|y| * 512) (exact scaling, ties to
// even); above, the float's mantissa is rounded to 3 bits at bit 20 (ties
// to even) and its exponent rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t ua = u & 0x7FFFFFFFu;
    const float a = __uint_as_float(ua);
    // |y| >= 2^-6: keep 3 mantissa bits, rounding the 20 dropped bits to
    // nearest even (a carry moves into the exponent); rebias 127 -> 7.
    const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
    const uint32_t normal = min((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u), 0x7Eu);
    // |y| < 2^-6: subnormal codes are multiples of 2^-9, rounded to even.
    const uint32_t sub = (uint32_t)rintf(fminf(a, 0.015625f) * 512.0f);
    uint32_t code = a < 0.015625f ? sub : normal;
    code = a >= 448.0f ? 0x7Eu : code;
    code = a != a ? 0x7Fu : code;
    return sign | code;
}

// Codes of eight bf16 values (w: element 2k in the low half of word k) as
// eight bytes, each the code of the float32 quotient x / scale -- the same
// quotient and encoder as the stored codes of an appended token.
__device__ __forceinline__ uint2 e4m3_encode8(uint4 w, float scale) {
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        c[k] = e4m3_encode(__uint_as_float(x[k] << 16) / scale) |
               (e4m3_encode(__uint_as_float(x[k] & 0xFFFF0000u) / scale) << 8);
    return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

// Merge two online-softmax states (m2, l, acc) in base 2.  -inf maxima
// (no positions seen) are handled so that no (-inf) - (-inf) is formed.
__device__ __forceinline__ void rescale_pair(float ma, float mb, float& fa, float& fb, float& mnew) {
    mnew = fmaxf(ma, mb);
    float ref = (mnew == kNegInf) ? 0.0f : mnew;
    fa = fast_exp2(ma - ref);
    fb = fast_exp2(mb - ref);
}

// Where a segment's m result rows go.  Final rows: out/lse of the query
// heads, natural-log lse.  Partial rows: normalised O and base-2 lse.
struct SegDst {
    float* o;
    float* lse;
    long o_stride;    // floats between consecutive rows
    long lse_stride;
    bool final_;
};

__device__ __forceinline__ SegDst final_dst(const DecodeArgs& a, int b, int j, int row0 = 0) {
    const long row = (long)b * a.h + (long)j * a.m + row0;
    return SegDst{a.out + row * a.d, a.lse + row, (long)a.d, 1, true};
}

// Chunked mode: chunk c of the rows of (b, j) from row0 on; a single chunk
// writes final rows.
__device__ __forceinline__ SegDst chunk_dst(const DecodeArgs& a, int b, int j, int c, int row0 = 0) {
    if (a.num_chunks == 1) return final_dst(a, b, j, row0);
    const long row = (long)b * a.h + (long)j * a.m + row0;
    return SegDst{a.part_o + (row * a.num_chunks + c) * a.d, a.part_lse + row * a.num_chunks + c,
                  (long)a.num_chunks * a.d, (long)a.num_chunks, false};
}

// A chunk that starts past the end of its unit: its `rows` partial rows get
// lse = -inf (weight 0), so that the merge reads every chunk's record at
// once without first reading the sequence length.
__device__ __forceinline__ void mark_empty_rows(const SegDst& dst, int rows, int tid) {
    if (tid < rows) dst.lse[(long)tid * dst.lse_stride] = kNegInf;
}

// Stream mode: record `slot` (0 = first segment, 1 = last) of this work-group.
__device__ __forceinline__ SegDst stream_dst(const DecodeArgs& a, int slot) {
    const long rec = ((long)blockIdx.x * 2 + slot) * a.m;
    return SegDst{a.part_o + rec * a.d, a.part_lse + rec, (long)a.d, 1, false};
}

// Clamp a device-side length to [0, cap].
__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Attended length from a raw seq_lens entry: the entry, plus the new token
// when the call also appends it, clamped to [0, cap_len].
__device__ __forceinline__ int attended_len(const DecodeArgs& a, int raw) {
    const long L = (long)raw + a.len_add;
    return L < 0 ? 0 : (L > a.cap_len ? a.cap_len : (int)L);
}

// Positions query token t (of the n per sequence) sees, from the raw
// seq_lens entry: raw + len_add - (n - 1 - t), clamped to [0, cap_len].  The
// last token sees the whole attended length.
__device__ __forceinline__ int visible_len(const DecodeArgs& a, int raw, int t) {
    const long L = (long)raw + a.len_add - (a.n - 1 - t);
    return L < 0 ? 0 : (L > a.cap_len ? a.cap_len : (int)L);
}

// First position a token sees when it sees `visible` positions.
__device__ __forceinline__ int window_lo(const DecodeArgs& a, int visible) {
    return a.window > 0 ? max(visible - a.window, 0) : 0;
}

// Positions [lo, hi) that some query row of a sequence reads: hi is the
// attended length (what the last token sees), lo what the first token's
// window starts at.
struct PosRange {
    int lo, hi;
};
__device__ __forceinline__ PosRange unit_range(const DecodeArgs& a, int raw) {
    return PosRange{window_lo(a, visible_len(a, raw, 0)), attended_len(a, raw)};
}

// Cache slot of position p in a contiguous cache: p, or p mod t_cap for a
// ring cache.
__device__ __forceinline__ int cache_slot(const DecodeArgs& a, int p) {
    return a.ring ? p % a.t_cap : p;
}

// bf16, d = D: write the appended tokens at positions [lo, hi) of unit
// (b, j) into their cache slots.  Position p holds new token p - raw of
// k_new / v_new [B, g, n, d].  Each of the `nthreads` threads moves 16-byte
// pieces (D/4 per position: D/8 of K, D/8 of V).  Paged: a position whose
// block-table entry is not a valid block is skipped, as the append entry
// point skips it.
template <int D>
__device__ __forceinline__ void store_new_rows_bf16(const DecodeArgs& a, int b, int j, int raw, int lo,
                                                    int hi, int tid, int nthreads) {
    constexpr int kC = D / 8;  // 16-byte chunks per row
    const long unit = (long)b * a.g + j;
    for (int idx = tid; idx < (hi - lo) * 2 * kC; idx += nthreads) {
        const int p = lo + idx / (2 * kC);
        const int part = idx % (2 * kC);
        long row;
        if (a.block_table != nullptr) {
            const int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
            if (phys < 0 || phys >= a.num_blocks) continue;
            row = ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
        } else {
            row = unit * a.t_cap + cache_slot(a, p);
        }
        const bool is_v = part >= kC;
        const int c = part % kC;
        const uint4* src = reinterpret_cast<const uint4*>(is_v ? a.v_new : a.k_new) +
                           (unit * a.n + (p - raw)) * kC + c;
        uint4* dst = reinterpret_cast<uint4*>(const_cast<void*>(is_v ? a.v : a.k)) + row * kC + c;
        *dst = *src;
    }
}
__device__ __forceinline__ void store_new_rows_bf16_d128(const DecodeArgs& a, int b, int j, int raw,
                                                         int lo, int hi, int tid, int nthreads) {
    store_new_rows_bf16<128>(a, b, j, raw, lo, hi, tid, nthreads);
}

// Transposing 8-byte LDS read (gfx950 ds_read_b64_tr_b16): within each
// 16-lane group, lanes 4r..4r+3 read 8 contiguous bytes each of one row r
// (r = 0..3), and lane i receives element i of each of the four rows -- one
// column of four rows, the MFMA operand layout of a transposed matrix.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)((__attribute__((address_space(3))) unsigned char*)p));
    return __builtin_bit_cast(uint2, r);
}

// D = A B + C on the matrix cores, 16x16 fp32 result from 16x32 bf16 A and
// 32x16 bf16 B (v_mfma_f32_16x16x32_bf16).  Lane l holds row l % 16 of A and
// column l % 16 of B, elements 8*(l/16) .. +8 of the 32-long k dimension;
// it receives rows 4*(l/16) .. +4 of column l % 16 of D.
__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS writes of a wavefront visible to all its lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// FP8 cache, d = D: quantise the appended tokens at positions [lo, hi) of
// unit (b, j) (bf16 rows of k_new / v_new, position p = row p - raw) and
// write their codes into their cache slots.  One code per thread and step
// (2*D per position: D of K, then D of V).  Paged: positions whose
// block-table entry is not a valid block are skipped.
template <int D>
__device__ __forceinline__ void store_new_rows_fp8(const DecodeArgs& a, int b, int j, int raw, int lo,
                                                   int hi, int tid, int nthreads) {
    const long unit = (long)b * a.g + j;
    for (int idx = tid; idx < (hi - lo) * 2 * D; idx += nthreads) {
        const int p = lo + idx / (2 * D);
        const bool is_v = (idx % (2 * D)) >= D;
        const int e = idx % D;
        long row;
        long sidx = j;
        if (a.block_table != nullptr) {
            const int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
            if (phys < 0 || phys >= a.num_blocks) continue;
            row = ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
            if (a.block_scales) sidx = (long)phys * a.g + j;
        } else {
            row = unit * a.t_cap + cache_slot(a, p);
        }
        const uint16_t x = reinterpret_cast<const uint16_t*>(is_v ? a.v_new : a.k_new)
                               [(unit * a.n + (p - raw)) * D + e];
        const float sc = is_v ? a.v_scale[sidx] : a.k_scale[sidx];
        unsigned char* dst = reinterpret_cast<unsigned char*>(const_cast<void*>(is_v ? a.v : a.k));
        dst[row * D + e] = (unsigned char)e4m3_encode(__uint_as_float((uint32_t)x << 16) / sc);
    }
}
__device__ __forceinline__ void store_new_rows_fp8_d128(const DecodeArgs& a, int b, int j, int raw,
                                                        int lo, int hi, int tid, int nthreads) {
    store_new_rows_fp8<128>(a, b, j, raw, lo, hi, tid, nthreads);
}

// d = 128: the bf16 pairs at dims 2*lane, 2*lane + 1 of unit (b, j)'s
// first new K row (.x) and V row (.y).
__device__ __forceinline__ uint2 new_row_pair_d128(const DecodeArgs& a, int b, int j, int lane) {
    const long row = ((long)b * a.g + j) * a.n;
    return make_uint2(reinterpret_cast<const uint32_t*>(a.k_new)[row * 64 + lane],
                      reinterpret_cast<const uint32_t*>(a.v_new)[row * 64 + lane]);
}

// Index of the FP8 scale of position p of unit (b, j): the KV head's, or
// with per-block scales that of its (block, KV head), the block id clamped
// into the pool as the kernels' reads clamp it.
__device__ __forceinline__ long fp8_scale_index(const DecodeArgs& a, int b, int j, int p) {
    if (!a.block_scales) return j;
    int ph = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
    ph = ph < 0 ? 0 : (ph >= a.num_blocks ? a.num_blocks - 1 : ph);
    return (long)ph * a.g + j;
}

// FP8 cache, d = 128, one new token per sequence: the codes of the new K
// row (bytes 0..127 of `codes`) and V row (128..255) for the scales at
// index sidx (fp8_scale_index of the new position), written
// to the calling wavefront's LDS area `codes` by its 64 lanes from their
// pairs (new_row_pair_d128), with the same quotient and encoder as
// store_new_rows_fp8_d128, so they equal what that call stores.  The caller
// syncs the wavefront (wave_lds_sync) before reading them.
__device__ __forceinline__ void new_row_codes_fp8_d128(const DecodeArgs& a, long sidx, int lane,
                                                       uint2 pair, unsigned char* codes) {
    const uint32_t kx = pair.x, vx = pair.y;
    const float ks = a.k_scale[sidx], vs = a.v_scale[sidx];
    const uint32_t kc = e4m3_encode(__uint_as_float(kx << 16) / ks) |
                        (e4m3_encode(__uint_as_float(kx & 0xFFFF0000u) / ks) << 8);
    const uint32_t vc = e4m3_encode(__uint_as_float(vx << 16) / vs) |
                        (e4m3_encode(__uint_as_float(vx & 0xFFFF0000u) / vs) << 8);
    reinterpret_cast<uint16_t*>(codes)[lane] = (uint16_t)kc;
    reinterpret_cast<uint16_t*>(codes + 128)[lane] = (uint16_t)vc;
}

}  // namespace kvc
