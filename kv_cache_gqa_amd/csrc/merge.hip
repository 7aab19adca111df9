// merge.hip -- combine per-chunk partial results by log-sum-exp.
//
// Each chunk c of a sequence produced O_c (already divided by its own l_c)
// and lse2_c = m_c + log2 l_c (base 2).  The merge is the rescaling identity
// behind the online softmax of "KV Cache 优化与注意力机制加速"
// (plumephp.com) section 2.2, applied across the chunks that section 2.5's
// sequence-dimension parallelism creates:
//   M = max_c lse2_c,  w_c = 2^(lse2_c - M),
//   out = sum_c w_c O_c / sum_c w_c,  lse = (M + log2 sum_c w_c) ln 2.
// Only chunks that hold positions of the sequence are read; a sequence of
// length 0 gets out = 0 and lse = -inf.
//
// One wavefront per (sequence, query head) row.
#include "kvc_device.h"

namespace kvc {

// Chunks are consumed eight at a time with all their loads issued together,
// so the latency of reading a row's partials is paid once per eight chunks.
constexpr int kMergeBatch = 8;

__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.B * a.h) return;
    const int lane = threadIdx.x & 63;
    const int d = a.d;
    const int C = a.num_chunks;
    const int b = (int)(row / a.h);
    const int L = clamp_len(a.seq_lens[b], a.cap_len);
    const int nc = (L + a.chunk_len - 1) / a.chunk_len;
    const float* pl = a.part_lse + row * C;

    float M = kNegInf;
    for (int c = lane; c < nc; c += 64) M = fmaxf(M, pl[c]);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) M = fmaxf(M, shfl_xor_f(M, mask));
    const float ref = (M == kNegInf) ? 0.0f : M;

    // Lane k holds dims 2k, 2k+1 (d <= 128, even) or k, k+64, k+128, k+192.
    const bool pairs = (d % 2 == 0) && d <= 128;
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    const float* po = a.part_o + row * C * d;
    for (int c0 = 0; c0 < nc; c0 += kMergeBatch) {
        float w[kMergeBatch], v[kMergeBatch][4];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int c = c0 + k;
            const bool ok = c < nc;
            w[k] = ok ? pl[c] : kNegInf;
            const float* src = po + (long)(ok ? c : 0) * d;
            if (pairs) {
                float2 t = make_float2(0.0f, 0.0f);
                if (ok && 2 * lane < d) t = *reinterpret_cast<const float2*>(src + 2 * lane);
                v[k][0] = t.x; v[k][1] = t.y; v[k][2] = 0.0f; v[k][3] = 0.0f;
            } else {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int dim = lane + 64 * kk;
                    v[k][kk] = (ok && dim < d) ? src[dim] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const float wk = fast_exp2(w[k] - ref);  // -inf -> 0 for absent chunks
            wsum += wk;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) o[kk] += wk * v[k][kk];
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    if (pairs) {
        if (2 * lane < d)
            *reinterpret_cast<float2*>(a.out + row * d + 2 * lane) = make_float2(o[0] * inv, o[1] * inv);
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.out[row * d + dim] = o[kk] * inv;
        }
    }
    if (lane == 0) a.lse[row] = wsum > 0.0f ? (M + fast_log2(wsum)) * kLn2 : kNegInf;
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    const long rows = (long)a.B * a.h;
    merge_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvc
