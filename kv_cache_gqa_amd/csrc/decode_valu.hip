// decode_valu.hip -- bf16, head_dim 128, small query groups (m = h/g <= 3).
//
// One work-group of four wavefronts per (chunk, KV head j, sequence b).  The
// work-group serves all m query heads that share KV head j ("大语言模型研究15
// ——注意力机制优化之KV缓存" (limoncc.com) section 三 3.3: heads j*m..j*m+m-1
// use KV head j), so every K/V byte of the chunk is read from HBM once.
//
// Lane layout: lane l covers dims [8*(l%16), 8*(l%16)+8) of position
// (l/16) + 4u of the current 32-position sub-tile, u = 0..7.  One 16-byte
// load per lane per u reads four whole 256-byte K (or V) rows per wavefront
// instruction, fully coalesced.  q.k is v_dot2_f32_bf16 on the raw bf16
// pairs, summed over the 16 lanes of a row with DPP.  Each row of 16 lanes
// keeps its own online-softmax state (m, l, acc) ("KV Cache 优化与注意力机制
// 加速" (plumephp.com) section 2.2); the four row states of a wavefront and
// the four wavefronts are merged once at the end of the chunk.
#include "kvc_device.h"

namespace kvc {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;

template <bool PAGED>
__device__ __forceinline__ long kv_row(const DecodeArgs& a, const int* tbl, int blk0, long bj_base,
                                       int j, int p) {
    if (PAGED) {
        const int phys = tbl[(p >> a.log2_bs) - blk0];
        return ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
    }
    return bj_base + p;
}

}  // namespace

template <int M, bool PAGED>
__global__ void __launch_bounds__(256) decode_valu_kernel(DecodeArgs a) {
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int tsub = lane >> 4, ds = lane & 15;
    const int L = clamp_len(a.seq_lens[b], a.cap_len);
    const int p0 = c * a.chunk_len;
    const int p1 = min(p0 + a.chunk_len, L);
    const bool single = a.num_chunks == 1;
    if (p0 >= L && !single) return;

    __shared__ int tbl[PAGED ? kMaxTableSlice : 1];
    __shared__ float red_m[kWaves][M], red_l[kWaves][M];
    __shared__ float red_o[kWaves][M][kD];

    int blk0 = 0;
    if (PAGED) {
        blk0 = p0 >> a.log2_bs;
        const int nblk = p1 > p0 ? ((p1 - 1) >> a.log2_bs) - blk0 + 1 : 0;
        for (int t = tid; t < nblk; t += 256) {
            int ph = a.block_table[(long)b * a.max_blocks + blk0 + t];
            tbl[t] = ph < 0 ? 0 : (ph >= a.num_blocks ? a.num_blocks - 1 : ph);
        }
        __syncthreads();
    }

    const uint16_t* K = (const uint16_t*)a.k;
    const uint16_t* Vc = (const uint16_t*)a.v;
    const uint16_t* Q = (const uint16_t*)a.q;

    uint32_t qp[M][4];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const uint4 v = ld16(Q + (((long)b * a.h + (long)j * M + r) * kD + 8 * ds));
        qp[r][0] = v.x; qp[r][1] = v.y; qp[r][2] = v.z; qp[r][3] = v.w;
    }
    float mrun[M], lrun[M], acc[M][8];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        mrun[r] = kNegInf;
        lrun[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
    }
    const long bj_base = ((long)b * a.g + j) * a.t_cap;
    const float sl2 = a.scale_log2e;

    for (int t0 = p0 + wave * kTileTokens; t0 < p1; t0 += kWaves * kTileTokens) {
        uint4 kv[8], vv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = min(t0 + 4 * u + tsub, p1 - 1);
            const long row = kv_row<PAGED>(a, tbl, blk0, bj_base, j, p);
            kv[u] = ld16(K + row * kD + 8 * ds);
            vv[u] = ld16(Vc + row * kD + 8 * ds);
        }
        float s[M][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool valid = (t0 + 4 * u + tsub) < p1;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                float dot = dot2_bf16(qp[r][0], kv[u].x, 0.0f);
                dot = dot2_bf16(qp[r][1], kv[u].y, dot);
                dot = dot2_bf16(qp[r][2], kv[u].z, dot);
                dot = dot2_bf16(qp[r][3], kv[u].w, dot);
                dot = row16_sum(dot) * sl2;
                s[r][u] = valid ? dot : kNegInf;
            }
        }
        float pr[M][8];
#pragma unroll
        for (int r = 0; r < M; ++r) {
            float mt = s[r][0];
#pragma unroll
            for (int u = 1; u < 8; ++u) mt = fmaxf(mt, s[r][u]);
            const float mnew = fmaxf(mrun[r], mt);
            const float ref = (mnew == kNegInf) ? 0.0f : mnew;
            const float alpha = fast_exp2(mrun[r] - ref);
            mrun[r] = mnew;
            float lsum = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pr[r][u] = fast_exp2(s[r][u] - ref);
                lsum += pr[r][u];
            }
            lrun[r] = lrun[r] * alpha + lsum;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float vf[8] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y),
                                 bf16_hi(vv[u].y), bf16_lo(vv[u].z), bf16_hi(vv[u].z),
                                 bf16_lo(vv[u].w), bf16_hi(vv[u].w)};
#pragma unroll
            for (int r = 0; r < M; ++r) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] += pr[r][u] * vf[e];
            }
        }
    }

    // Merge the four rows of 16 lanes (positions interleaved by lane/16).
#pragma unroll
    for (int r = 0; r < M; ++r) {
#pragma unroll
        for (int mask = 16; mask <= 32; mask <<= 1) {
            const float mo = shfl_xor_f(mrun[r], mask);
            const float lo = shfl_xor_f(lrun[r], mask);
            float fa, fb, mnew;
            rescale_pair(mrun[r], mo, fa, fb, mnew);
            lrun[r] = lrun[r] * fa + lo * fb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ao = shfl_xor_f(acc[r][e], mask);
                acc[r][e] = acc[r][e] * fa + ao * fb;
            }
            mrun[r] = mnew;
        }
    }
    if (tsub == 0) {
#pragma unroll
        for (int r = 0; r < M; ++r) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[wave][r][8 * ds + e] = acc[r][e];
            if (ds == 0) {
                red_m[wave][r] = mrun[r];
                red_l[wave][r] = lrun[r];
            }
        }
    }
    __syncthreads();

    // Merge the four wavefronts and write the result (final or partial).
    for (int idx = tid; idx < M * kD; idx += 256) {
        const int r = idx / kD, dim = idx % kD;
        float mm = red_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, red_m[w][r]);
        const float ref = (mm == kNegInf) ? 0.0f : mm;
        float l = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(red_m[w][r] - ref);
            l += red_l[w][r] * f;
            o += red_o[w][r][dim] * f;
        }
        const long row_out = (long)b * a.h + (long)j * M + r;
        if (single) {
            a.out[row_out * kD + dim] = l > 0.0f ? o / l : 0.0f;
            if (dim == 0) a.lse[row_out] = l > 0.0f ? (mm + fast_log2(l)) * kLn2 : kNegInf;
        } else {
            const long prow = row_out * a.num_chunks + c;
            a.part_o[prow * kD + dim] = o / l;
            if (dim == 0) a.part_lse[prow] = mm + fast_log2(l);
        }
    }
}

hipError_t launch_decode_valu_bf16_d128(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.num_chunks, (unsigned)a.g, (unsigned)a.B);
    const bool paged = a.block_table != nullptr;
#define KVC_VALU_CASE(MM)                                                      \
    case MM:                                                                   \
        if (paged)                                                             \
            decode_valu_kernel<MM, true><<<grid, dim3(256), 0, s>>>(a);        \
        else                                                                   \
            decode_valu_kernel<MM, false><<<grid, dim3(256), 0, s>>>(a);       \
        break;
    switch (a.m) {
        KVC_VALU_CASE(1)
        KVC_VALU_CASE(2)
        KVC_VALU_CASE(3)
        KVC_VALU_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef KVC_VALU_CASE
    return hipGetLastError();
}

}  // namespace kvc
