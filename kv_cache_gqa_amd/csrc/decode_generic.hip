// decode_generic.hip -- decode attention for any head_dim <= 256, float32 or
// bf16, any group size, contiguous or paged.  The path for shapes the
// specialised bf16/d=128 kernels do not cover (the fp32 d=16 workload, the
// d=1 worked example).
//
// One wavefront per (chunk, query head, sequence).  Lane k holds dims k,
// k+64, k+128, k+192.  Positions are visited one at a time: the partial dot
// products are summed across the wave, then the online-softmax update of
// "KV Cache 优化与注意力机制加速" (plumephp.com) section 2.2 is applied:
// m' = max(m, s), l' = l exp(m - m') + exp(s - m'), acc' = acc exp(m - m') +
// exp(s - m') V_p, all in base 2.  Query head i reads KV head
// floor(i*g/h) ("大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com),
// section 三 3.3).
#include "kvc_device.h"

namespace kvc {

template <typename T>
__device__ __forceinline__ float load_f(const T* p, long idx);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, long idx) { return p[idx]; }
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, long idx) {
    return __uint_as_float((uint32_t)p[idx] << 16);
}
template <>
__device__ __forceinline__ float load_f<uint8_t>(const uint8_t* p, long idx) {
    return e4m3_to_f32(p[idx]);  // FP8 E4M3 code
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += shfl_xor_f(x, 16);
    x += shfl_xor_f(x, 32);
    return x;
}

// TQ: query element type; T: cache element type (uint8_t: FP8 E4M3 codes
// with a float32 scale per KV head, folded into the query and the output).
template <typename TQ, typename T>
__global__ void __launch_bounds__(64) decode_generic_kernel(DecodeArgs a) {
    const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int d = a.d;
    const int j = (int)(((long)i * a.g) / a.h);
    const int raw = a.seq_lens[b];
    const PosRange ur = unit_range(a, raw);  // chunks cover [lo, hi)
    const int c0 = ur.lo + c * a.chunk_len;
    const bool single = a.num_chunks == 1;
    if (c0 >= ur.hi && !single) {  // past the end: a record of weight 0 for the merge
        if (lane == 0) a.part_lse[((long)b * a.h + i) * a.num_chunks + c] = kNegInf;
        return;
    }
    // row i is token i % n, which sees [window_lo(vis), vis)
    const int vis = visible_len(a, raw, i % a.n);
    const int p0 = max(c0, window_lo(a, vis));
    const int p1 = min(min(c0 + a.chunk_len, ur.hi), vis);

    const TQ* q = (const TQ*)a.q;
    const T* K = (const T*)a.k;
    const T* V = (const T*)a.v;
    const float k_sc = a.kv8 ? a.k_scale[j] : 1.0f;
    const float v_sc = a.kv8 ? a.v_scale[j] : 1.0f;
    float qv[4], acc[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int dim = lane + 64 * kk;
        qv[kk] = dim < d ? load_f(q, ((long)b * a.h + i) * d + dim) * (a.scale_log2e * k_sc) : 0.0f;
        acc[kk] = 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    const long contig_base = ((long)b * a.g + j) * a.t_cap;
    for (int p = p0; p < p1; ++p) {
        long row;
        if (a.block_table != nullptr) {
            int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
            phys = phys < 0 ? 0 : (phys >= a.num_blocks ? a.num_blocks - 1 : phys);
            row = ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
        } else {
            row = contig_base + cache_slot(a, p);
        }
        float part = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) part += qv[kk] * load_f(K, row * d + dim);
        }
        const float s = wave_sum(part);
        const float mnew = fmaxf(m, s);
        const float alpha = fast_exp2(m - mnew);  // m = -inf on the first position -> 0
        const float pw = fast_exp2(s - mnew);
        l = l * alpha + pw;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) acc[kk] = acc[kk] * alpha + pw * load_f(V, row * d + dim);
        }
        m = mnew;
    }

    const long row_out = (long)b * a.h + i;
    if (single) {
        const float inv = l > 0.0f ? v_sc / l : 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.out[row_out * d + dim] = acc[kk] * inv;
        }
        if (lane == 0) a.lse[row_out] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : kNegInf;
    } else {
        const long prow = row_out * a.num_chunks + c;
        const float inv = l > 0.0f ? v_sc / l : 0.0f;  // l = 0: nothing visible in this chunk
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.part_o[prow * d + dim] = acc[kk] * inv;
        }
        if (lane == 0) a.part_lse[prow] = l > 0.0f ? m + fast_log2(l) : kNegInf;
    }
}

hipError_t launch_decode_generic(const DecodeArgs& a, int dtype, hipStream_t s) {
    dim3 grid((unsigned)a.num_chunks, (unsigned)a.h, (unsigned)a.B);
    if (a.kv8) {
        decode_generic_kernel<uint16_t, uint8_t><<<grid, dim3(64), 0, s>>>(a);
    } else if (dtype == 0) {
        decode_generic_kernel<float, float><<<grid, dim3(64), 0, s>>>(a);
    } else {
        decode_generic_kernel<uint16_t, uint16_t><<<grid, dim3(64), 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace kvc
