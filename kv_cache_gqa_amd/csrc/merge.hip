// merge.hip -- combine per-chunk partial results by log-sum-exp.
//
// Each chunk c of a sequence produced O_c (already divided by its own l_c)
// and lse2_c = m_c + log2 l_c (base 2).  The merge is the rescaling identity
// behind the online softmax of "KV Cache 优化与注意力机制加速"
// (plumephp.com) section 2.2, applied across the chunks that section 2.5's
// sequence-dimension parallelism creates:
//   M = max_c lse2_c,  w_c = 2^(lse2_c - M),
//   out = sum_c w_c O_c / sum_c w_c,  lse = (M + log2 sum_c w_c) ln 2.
// Chunked plans: every chunk has a record (chunks past the end of a unit
// hold lse = -inf), so a row's records are all loaded at once; a sequence of
// length 0 gets out = 0 and lse = -inf.
#include "kvc_schedule.h"

namespace kvc {

// Chunks/records are consumed eight at a time: the lse and O loads of a
// batch are all issued together and folded in with online rescaling, so a
// row costs one round trip to memory per eight partial results.
constexpr int kMergeBatch = 8;

// Lane k holds dims 2k, 2k+1 (d <= 128 and even) or k, k+64, k+128, k+192.
struct MergeAcc {
    float M = kNegInf;
    float wsum = 0.0f;
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // Fold in a batch of partial results: lse (base 2) and lane values v.
    __device__ void add(const float (&lse)[kMergeBatch], const float (&v)[kMergeBatch][4]) {
        float bm = M;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lse[k]);
        const float ref = (bm == kNegInf) ? 0.0f : bm;
        const float f = fast_exp2(M - ref);  // 0 while nothing was added
        wsum *= f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) o[kk] *= f;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const float w = fast_exp2(lse[k] - ref);  // -inf -> 0 for absent entries
            wsum += w;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) o[kk] += w * v[k][kk];
        }
        M = bm;
    }
};

__device__ __forceinline__ void load_lane(const float* src, bool ok, int lane, int d, bool pairs,
                                          float (&v)[4]) {
    if (pairs) {
        float2 t = make_float2(0.0f, 0.0f);
        if (ok && 2 * lane < d) t = *reinterpret_cast<const float2*>(src + 2 * lane);
        v[0] = t.x; v[1] = t.y; v[2] = 0.0f; v[3] = 0.0f;
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            v[kk] = (ok && dim < d) ? src[dim] : 0.0f;
        }
    }
}

__device__ __forceinline__ void write_row(const DecodeArgs& a, long row, int lane, bool pairs,
                                          const MergeAcc& acc) {
    const int d = a.d;
    const float inv = acc.wsum > 0.0f ? 1.0f / acc.wsum : 0.0f;
    if (pairs) {
        if (2 * lane < d)
            *reinterpret_cast<float2*>(a.out + row * d + 2 * lane) =
                make_float2(acc.o[0] * inv, acc.o[1] * inv);
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.out[row * d + dim] = acc.o[kk] * inv;
        }
    }
    if (lane == 0) a.lse[row] = acc.wsum > 0.0f ? (acc.M + fast_log2(acc.wsum)) * kLn2 : kNegInf;
}

// Chunked plans: one work-group per (sequence, query head) row.  Thread t
// owns V dims (e = t % nE, nE = d / V) of the chunks c = cg, cg + G, ...
// (cg = t / nE, G = 256 / nE chunk groups), folds them in eight per round
// trip with online rescaling, and the G partial states are combined through
// LDS.  All loads of a row are independent of each other, so a row costs
// about one memory round trip.  The O of a record of weight 0 is not used
// (chunks past the end leave it unwritten).
template <int V>
__device__ __forceinline__ void merge_row_chunked(const DecodeArgs& a, long row) {
    __shared__ float sm_m[256];
    __shared__ float sm_w[256];
    __shared__ float sm_o[256 * 4];
    const int d = a.d, C = a.num_chunks;
    const int nE = d / V;
    const int G = 256 / nE;
    const int t = threadIdx.x;
    const int cg = t / nE, e = t - (t / nE) * nE;
    const int nc = C;
    if (cg < G) {
        float M = kNegInf, W = 0.0f, o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = 0.0f;
        for (int c0 = cg; c0 < nc; c0 += G * kMergeBatch) {
            float lse[kMergeBatch], x[kMergeBatch][V];
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const int c = c0 + k * G;
                const bool ok = c < nc;
                const long rec = row * C + (ok ? c : 0);
                lse[k] = ok ? a.part_lse[rec] : kNegInf;
                const float* src = a.part_o + rec * d + e * V;
                if constexpr (V == 4) {
                    const float4 q4 = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
                    x[k][0] = q4.x;
                    x[k][1] = q4.y;
                    x[k][2] = q4.z;
                    x[k][3] = q4.w;
                } else {
                    x[k][0] = ok ? src[0] : 0.0f;
                }
            }
            float bm = M;
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lse[k]);
            const float ref = (bm == kNegInf) ? 0.0f : bm;
            const float f = fast_exp2(M - ref);
            W *= f;
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] *= f;
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const float w = fast_exp2(lse[k] - ref);  // 0 for absent and empty chunks
                W += w;
#pragma unroll
                for (int v = 0; v < V; ++v) o[v] += w > 0.0f ? w * x[k][v] : 0.0f;
            }
            M = bm;
        }
        if (e == 0) {
            sm_m[cg] = M;
            sm_w[cg] = W;
        }
#pragma unroll
        for (int v = 0; v < V; ++v) sm_o[cg * d + e * V + v] = o[v];
    }
    __syncthreads();
    for (int dim = t; dim < d; dim += 256) {
        float Mx = kNegInf;
        for (int q = 0; q < G; ++q) Mx = fmaxf(Mx, sm_m[q]);
        const float ref = (Mx == kNegInf) ? 0.0f : Mx;
        float Wt = 0.0f, ot = 0.0f;
        for (int q = 0; q < G; ++q) {
            const float f = fast_exp2(sm_m[q] - ref);
            Wt += sm_w[q] * f;
            ot += sm_o[q * d + dim] * f;
        }
        a.out[row * d + dim] = Wt > 0.0f ? ot / Wt : 0.0f;
        if (dim == 0) a.lse[row] = Wt > 0.0f ? (Mx + fast_log2(Wt)) * kLn2 : kNegInf;
    }
}

__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a) {
    const long row = blockIdx.x;
    if (a.d % 4 == 0) merge_row_chunked<4>(a, row);
    else merge_row_chunked<1>(a, row);
}

// Stream mode: unit u = (b, j) occupies global positions [U, U + L).  If its
// first and last positions belong to the same work-group, that work-group
// wrote the final rows itself.  Otherwise work-groups pa..pb each hold one
// partial record of it: record slot 1 of pa when pa's range starts before U
// (u is then pa's last segment), slot 0 otherwise.  Work-groups with an empty
// range are skipped.  Length-0 sequences get out = 0, lse = -inf here.
//
// One work-group per unit: the prefix sums of the lengths and the unit's
// span of work-groups are found once per unit (64-bit divisions: computed
// per row they dominated the pass at many rows per unit), the records'
// slots go to shared memory, and each thread folds one (row, 4 dims) item of
// the unit's m rows over them, eight records per round trip.  The block has
// as many threads as items (rounded up to wavefronts, at most 1024); more
// items loop.  Head dimension a multiple of 4 (64, 128, 256 in stream plans).
constexpr int kMergeStreamThreads = 1024;

__global__ void __launch_bounds__(kMergeStreamThreads) merge_stream_kernel(DecodeArgs a) {
    __shared__ long long cum[kStreamMaxB + 1];
    __shared__ int slot_of[kMergeStreamThreads];  // per record of a batch: q * 2 + slot, or -1
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int b = blockIdx.x / a.g, j = blockIdx.x % a.g;
    const int m = a.m, d = a.d, nq = d / 4;
    const int items = m * nq;
    const long row0 = (long)b * a.h + (long)j * m;
    stream_prefix(a, cum);  // ends with a barrier
    if (cum[b + 1] == cum[b]) {
        for (int it = tid; it < items; it += nthr) {
            const int r = it / nq, q4 = it - r * nq;
            *reinterpret_cast<float4*>(a.out + (row0 + r) * d + 4 * q4) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (q4 == 0) a.lse[row0 + r] = kNegInf;
        }
        return;
    }
    const UnitSpan sp = unit_span(a, cum, b, j);
    if (sp.pa == sp.pb) return;  // one work-group covered the whole unit
    for (int it0 = 0; it0 < items; it0 += nthr) {
        const int it = it0 + tid;
        const bool act = it < items;
        const int r = act ? it / nq : 0, q4 = act ? it - r * nq : 0;
        float M = kNegInf, W = 0.0f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (long long q0 = sp.pa; q0 <= sp.pb; q0 += nthr) {
            const int cnt = (int)min((long long)nthr, sp.pb - q0 + 1);
            __syncthreads();  // the previous batch's slots are read
            if (tid < cnt) {
                const long long q = q0 + tid;
                slot_of[tid] = sp.empty(q) ? -1 : (int)sp.record(q, 1, 0);
            }
            __syncthreads();
            if (!act) continue;
            for (int k0 = 0; k0 < cnt; k0 += kMergeBatch) {
                float lse[kMergeBatch];
                float4 x[kMergeBatch];
#pragma unroll
                for (int k = 0; k < kMergeBatch; ++k) {
                    const int sl = k0 + k < cnt ? slot_of[k0 + k] : -1;
                    const long rec = (long)(sl < 0 ? 0 : sl) * m + r;
                    lse[k] = sl >= 0 ? a.part_lse[rec] : kNegInf;
                    x[k] = sl >= 0 ? *reinterpret_cast<const float4*>(a.part_o + rec * d + 4 * q4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                float bm = M;
#pragma unroll
                for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lse[k]);
                const float ref = (bm == kNegInf) ? 0.0f : bm;
                const float f = fast_exp2(M - ref);  // 0 while nothing was added
                W *= f;
                o.x *= f; o.y *= f; o.z *= f; o.w *= f;
#pragma unroll
                for (int k = 0; k < kMergeBatch; ++k) {
                    const float w = fast_exp2(lse[k] - ref);  // 0 for absent records
                    W += w;
                    o.x += w * x[k].x; o.y += w * x[k].y; o.z += w * x[k].z; o.w += w * x[k].w;
                }
                M = bm;
            }
        }
        if (!act) continue;
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        *reinterpret_cast<float4*>(a.out + (row0 + r) * d + 4 * q4) =
            make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        if (q4 == 0) a.lse[row0 + r] = W > 0.0f ? (M + fast_log2(W)) * kLn2 : kNegInf;
    }
}

hipError_t launch_merge_stream(const DecodeArgs& a, hipStream_t s) {
    if (a.d % 4 != 0 || a.B > kStreamMaxB) return hipErrorInvalidValue;
    const long items = (long)a.m * (a.d / 4);
    const long rounded = (items + 63) / 64 * 64;
    const int threads = (int)(rounded < kMergeStreamThreads ? rounded : kMergeStreamThreads);
    merge_stream_kernel<<<dim3((unsigned)((long)a.B * a.g)), dim3(threads), 0, s>>>(a);
    return hipGetLastError();
}

// Chunked plans with d = 128 (every bf16 / FP8 head-dim-128 kernel): rows
// packed into work-groups.  A (row, chunk group) is 32 lanes of 4 dims; a
// row has G chunk groups (1, 2, 4 or 8 by the chunk count, so that no lane
// folds more than eight chunks for up to 64 chunks: one round trip to
// memory), and a 64-lane work-group holds 2 / G rows (G <= 2) or one row of
// 32*G lanes.  The G partial states of a row are combined through LDS.
template <int G>
__global__ void __launch_bounds__(G <= 2 ? 64 : 32 * G) merge128_kernel(DecodeArgs a) {
    constexpr int kRowsPerWg = G == 1 ? 2 : 1;
    __shared__ float sm_m[G];
    __shared__ float sm_w[G];
    __shared__ float4 sm_o[G][32];
    const int slot = threadIdx.x >> 5, lane = threadIdx.x & 31;
    const int grp = slot % G;
    const long row = (long)blockIdx.x * kRowsPerWg + slot / G;
    const long rows = (long)a.B * a.h;
    const int C = a.num_chunks;
    float M = kNegInf, W = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < rows) {
        for (int c0 = grp; c0 < C; c0 += G * kMergeBatch) {
            float lse[kMergeBatch];
            float4 x[kMergeBatch];
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const int c = c0 + k * G;
                const bool ok = c < C;
                const long rec = row * C + (ok ? c : 0);
                lse[k] = ok ? a.part_lse[rec] : kNegInf;
                x[k] = ok ? *reinterpret_cast<const float4*>(a.part_o + rec * 128 + 4 * lane)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            float bm = M;
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lse[k]);
            const float ref = (bm == kNegInf) ? 0.0f : bm;
            const float f = fast_exp2(M - ref);  // 0 while nothing was added
            W *= f;
            o.x *= f; o.y *= f; o.z *= f; o.w *= f;
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const float w = fast_exp2(lse[k] - ref);  // 0 for absent and empty chunks
                W += w;
                if (w > 0.0f) {  // the O of an empty chunk is never written
                    o.x += w * x[k].x; o.y += w * x[k].y; o.z += w * x[k].z; o.w += w * x[k].w;
                }
            }
            M = bm;
        }
    }
    if constexpr (G > 1) {
        if (lane == 0) {
            sm_m[grp] = M;
            sm_w[grp] = W;
        }
        sm_o[grp][lane] = o;
        __syncthreads();
        if (grp != 0) return;
        float Mx = kNegInf;
#pragma unroll
        for (int q = 0; q < G; ++q) Mx = fmaxf(Mx, sm_m[q]);
        const float ref = (Mx == kNegInf) ? 0.0f : Mx;
        W = 0.0f;
        o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const float f = fast_exp2(sm_m[q] - ref);
            const float4 y = sm_o[q][lane];
            W += sm_w[q] * f;
            o.x += f * y.x; o.y += f * y.y; o.z += f * y.z; o.w += f * y.w;
        }
        M = Mx;
    }
    if (row >= rows) return;
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    *reinterpret_cast<float4*>(a.out + row * 128 + 4 * lane) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (lane == 0) a.lse[row] = W > 0.0f ? (M + fast_log2(W)) * kLn2 : kNegInf;
}

template <int G>
static void launch_merge128(const DecodeArgs& a, long rows, hipStream_t s) {
    constexpr int kRowsPerWg = G == 1 ? 2 : 1;
    constexpr int kThreads = G <= 2 ? 64 : 32 * G;
    merge128_kernel<G><<<dim3((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg)), dim3(kThreads), 0,
                         s>>>(a);
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    const long rows = (long)a.B * a.h;
    if (a.d == 128) {
        const int C = a.num_chunks;
        if (C <= kMergeBatch) launch_merge128<1>(a, rows, s);
        else if (C <= 2 * kMergeBatch) launch_merge128<2>(a, rows, s);
        else if (C <= 4 * kMergeBatch) launch_merge128<4>(a, rows, s);
        else launch_merge128<8>(a, rows, s);
    } else {
        merge_kernel<<<dim3((unsigned)rows), dim3(256), 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace kvc
