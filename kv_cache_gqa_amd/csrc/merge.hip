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
#include "kvc_schedule.h"

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

// Stream mode: unit u = (b, j) occupies global positions [U, U + L).  If its
// first and last positions belong to the same work-group, that work-group
// wrote the final rows itself.  Otherwise work-groups pa..pb each hold one
// partial record of it: record slot 1 of pa when pa's range starts before U
// (u is then pa's last segment), slot 0 otherwise.  Work-groups with an empty
// range are skipped.  Length-0 sequences get out = 0, lse = -inf here.
__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) x += __shfl_xor(x, mask, 64);
    return x;
}

__global__ void __launch_bounds__(256) merge_stream_kernel(DecodeArgs a) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long)a.B * a.h) return;
    const int lane = threadIdx.x & 63;
    const int d = a.d, m = a.m;
    const int b = (int)(row / a.h);
    const int i = (int)(row % a.h);
    const int j = i / m, r = i % m;
    const long long L = clamp_len(a.seq_lens[b], a.cap_len);
    const bool pairs = (d % 2 == 0) && d <= 128;
    if (L == 0) {
        if (pairs) {
            if (2 * lane < d) *reinterpret_cast<float2*>(a.out + row * d + 2 * lane) = make_float2(0.f, 0.f);
        } else {
            for (int dim = lane; dim < d; dim += 64) a.out[row * d + dim] = 0.0f;
        }
        if (lane == 0) a.lse[row] = kNegInf;
        return;
    }
    long long before = 0, all = 0;
    for (int bb = lane; bb < a.B; bb += 64) {
        const long long Lb = clamp_len(a.seq_lens[bb], a.cap_len);
        all += Lb;
        if (bb < b) before += Lb;
    }
    before = wave_sum_ll(before);
    all = wave_sum_ll(all);
    const long long P = a.num_wgs;
    const long long total = (long long)a.g * all;
    const long long U = (long long)a.g * before + (long long)j * L;
    const long long pa = stream_owner(U, total, P);
    const long long pb = stream_owner(U + L - 1, total, P);
    if (pa == pb) return;  // one work-group covered the whole unit
    const bool pa_last = stream_start(pa, total, P) < U;
    auto rec = [&](long long q) -> long long {
        return (q * 2 + ((q == pa && pa_last) ? 1 : 0)) * m + r;
    };
    auto empty = [&](long long q) -> bool {
        return stream_start(q, total, P) >= stream_start(q + 1, total, P);
    };

    float M = kNegInf;
    for (long long q = pa + lane; q <= pb; q += 64)
        if (!empty(q)) M = fmaxf(M, a.part_lse[rec(q)]);
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) M = fmaxf(M, shfl_xor_f(M, mask));
    const float ref = (M == kNegInf) ? 0.0f : M;

    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    for (long long q0 = pa; q0 <= pb; q0 += kMergeBatch) {
        float w[kMergeBatch], v[kMergeBatch][4];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const long long q = q0 + k;
            const bool ok = q <= pb && !empty(q);
            const long long rr = ok ? rec(q) : 0;
            w[k] = ok ? a.part_lse[rr] : kNegInf;
            const float* src = a.part_o + rr * d;
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
            const float wk = fast_exp2(w[k] - ref);
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

hipError_t launch_merge_stream(const DecodeArgs& a, hipStream_t s) {
    const long rows = (long)a.B * a.h;
    merge_stream_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    const long rows = (long)a.B * a.h;
    merge_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvc
