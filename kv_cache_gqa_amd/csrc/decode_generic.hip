// decode_generic.hip -- decode attention for any head_dim <= 256, float32 or
// bf16, any group size, contiguous or paged.  The path for shapes the
// specialised bf16/d=128 kernels do not cover (the fp32 d=16 workload, the
// d=1 worked example).
//
// One work-group per (chunk, KV head j and a block of up to 16 of its m
// query rows, sequence), one wavefront per query row: the wavefronts of a
// work-group walk the same K/V positions together, so the rows of a KV
// head's group share each line the first of them brings in, and K/V is read
// from HBM once per KV head, not once per query head.  Query head i reads
// KV head floor(i*g/h) ("大语言模型研究15——注意力机制优化之KV缓存"
// (limoncc.com), section 三 3.3).
//
// Lane k holds dims k (head dims up to 64; positions in batches of sixteen)
// or k, k+64, k+128, k+192 (batches of eight, four for FP8 codes): one
// round trip to memory per batch.  For each batch the partial dot products
// are summed across the wave, then the online-softmax update of "KV Cache
// 优化与注意力机制加速" (plumephp.com) section 2.2 is applied once for the
// batch: m' = max(m, max_p s_p), l' = l exp(m - m') + sum_p exp(s_p - m'),
// acc' = acc exp(m - m') + sum_p exp(s_p - m') V_p, all in base 2.  A call
// that appends reads its new tokens (positions seq_lens[b] ..) from k_new /
// v_new (FP8: as their codes), and the first query row of each KV head's
// group writes its chunk's new positions into their cache slots.
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

// Four consecutive elements (index idx .. idx+3, idx a multiple of 4) as
// floats, in one vector load: 16 bytes of float32, 8 of bf16, 4 of codes.
template <typename T>
__device__ __forceinline__ void load4_f(const T* p, long idx, float (&x)[4]);
template <>
__device__ __forceinline__ void load4_f<float>(const float* p, long idx, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p + idx);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <>
__device__ __forceinline__ void load4_f<uint16_t>(const uint16_t* p, long idx, float (&x)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + idx);
    x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xFFFF0000u);
    x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load4_f<uint8_t>(const uint8_t* p, long idx, float (&x)[4]) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p + idx);
#pragma unroll
    for (int t = 0; t < 4; ++t) x[t] = e4m3_to_f32((v >> (8 * t)) & 0xFFu);
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += shfl_xor_f(x, 16);
    x += shfl_xor_f(x, 32);
    return x;
}

// The value a new element x takes in the cache: itself, or (FP8) the value
// of its code for the head's scale, as the FP8 append kernel stores it.
template <typename T>
__device__ __forceinline__ float new_value(float x, float scale) {
    if constexpr (sizeof(T) == 1) return e4m3_to_f32((uint8_t)e4m3_encode(x / scale));
    else return x;
}

// Query rows per work-group (one wavefront each).
constexpr int kGenericRows = 16;

// TQ: query element type; T: cache element type (uint8_t: FP8 E4M3 codes
// with a float32 scale per KV head, folded into the query and the output;
// k_new / v_new are then bf16, TQ).  NK: dims per lane (1: d <= 64; 4).
// LP > 0 (head dims that are multiples of 4): LP lanes per position, four
// dims each (one vector load per position and tensor), 64 / LP positions
// side by side, each lane group with its own online-softmax state, merged
// across the groups at the end; NK is then unused.
// Work-group (c, y, b) with y = j * RB + rb (RB = ceil(m / R) row blocks,
// R = min(m, kGenericRows) wavefronts): wavefront w takes query head
// i = j*m + rb*R + w, if that is below (j+1)*m.
template <typename TQ, typename T, int NK, int LP>
__global__ void __launch_bounds__(64 * kGenericRows) decode_generic_kernel(DecodeArgs a) {
    const int c = blockIdx.x, b = blockIdx.z;
    const int R = (int)(blockDim.x >> 6), RB = (a.m + R - 1) / R;
    const int j = (int)blockIdx.y / RB, rb = (int)blockIdx.y - j * RB;
    const int r = rb * R + (int)(threadIdx.x >> 6);
    if (r >= a.m) return;  // the last row block of a group may be partial
    const int i = j * a.m + r;  // query head: i * g / h = j
    const int lane = threadIdx.x & 63;
    const int d = a.d;
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
    // FP8 scales: per KV head (folded into q and the output), or per
    // (block, KV head) (applied per position)
    const bool bsc = a.kv8 && a.block_scales;
    const float k_sc = a.kv8 && !bsc ? a.k_scale[j] : 1.0f;
    const float v_sc = a.kv8 && !bsc ? a.v_scale[j] : 1.0f;
    // new tokens: element type of k_new / v_new, their rows, cache rows
    using TN = typename std::conditional<sizeof(T) == 1, TQ, T>::type;
    const bool appends = a.k_new != nullptr;
    const long new_base = ((long)b * a.g + j) * a.n - raw;  // k_new row of position p: new_base + p
    const long contig_base = ((long)b * a.g + j) * a.t_cap;
    if (appends && i == j * a.m) {
        // this chunk's new positions go to their cache slots (skipped, as the
        // append kernels skip them, when a paged table entry is not a block)
        const int s0 = max(c0, raw), s1 = min(c0 + a.chunk_len, ur.hi);
        for (int p = s0; p < s1; ++p) {
            long row;
            float wk = k_sc, wv = v_sc;  // the scales the new codes are made with
            if (a.block_table != nullptr) {
                const int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
                if (phys < 0 || phys >= a.num_blocks) continue;
                row = ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
                if (bsc) {
                    wk = a.k_scale[(long)phys * a.g + j];
                    wv = a.v_scale[(long)phys * a.g + j];
                }
            } else {
                row = contig_base + cache_slot(a, p);
            }
            for (int dim = lane; dim < d; dim += 64) {
                const long src = (new_base + p) * d + dim;
                if constexpr (sizeof(T) == 1) {
                    const float x = load_f((const TN*)a.k_new, src);
                    const float y = load_f((const TN*)a.v_new, src);
                    const_cast<T*>(K)[row * d + dim] = (T)e4m3_encode(x / wk);
                    const_cast<T*>(V)[row * d + dim] = (T)e4m3_encode(y / wv);
                } else {
                    const_cast<T*>(K)[row * d + dim] = ((const T*)a.k_new)[src];
                    const_cast<T*>(V)[row * d + dim] = ((const T*)a.v_new)[src];
                }
            }
        }
    }
    if constexpr (LP > 0) {
        // Lane group gs (of PP) takes positions pb + u*PP + gs of batch pb;
        // lane sub of the group holds dims 4*sub .. 4*sub+3.
        constexpr int PP = 64 / LP;
        constexpr int kPasses = sizeof(T) == 1 ? 4 : 8;  // positions per group and batch
        const int gs = lane / LP, dbase = 4 * (lane % LP);
        const bool on = dbase < d;  // d is a multiple of 4
        float qv[4], acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (on) load4_f(q, ((long)b * a.h + i) * d + dbase, qv);
#pragma unroll
        for (int t = 0; t < 4; ++t) qv[t] = on ? qv[t] * (a.scale_log2e * k_sc) : 0.0f;
        float m = kNegInf, l = 0.0f;
        for (int pb = p0; pb < p1; pb += PP * kPasses) {
            float kx[kPasses][4], vx[kPasses][4], ksp[kPasses], vsp[kPasses];
#pragma unroll
            for (int u = 0; u < kPasses; ++u) {
                const int p = min(pb + u * PP + gs, p1 - 1);  // past the end: the last position (masked)
                const bool fresh = appends && p >= raw;
                ksp[u] = vsp[u] = 1.0f;
                if (bsc) {
                    const long si = fp8_scale_index(a, b, j, p);
                    ksp[u] = a.k_scale[si];
                    vsp[u] = a.v_scale[si];
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) kx[u][t] = vx[u][t] = 0.0f;
                if (on) {
                    if (fresh) {
                        const long src = (new_base + p) * d + dbase;
                        load4_f((const TN*)a.k_new, src, kx[u]);
                        load4_f((const TN*)a.v_new, src, vx[u]);
                        const float nk = bsc ? ksp[u] : k_sc, nv = bsc ? vsp[u] : v_sc;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            kx[u][t] = new_value<T>(kx[u][t], nk);
                            vx[u][t] = new_value<T>(vx[u][t], nv);
                        }
                    } else {
                        long row;
                        if (a.block_table != nullptr) {
                            int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
                            phys = phys < 0 ? 0 : (phys >= a.num_blocks ? a.num_blocks - 1 : phys);
                            row = ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
                        } else {
                            row = contig_base + cache_slot(a, p);
                        }
                        load4_f(K, row * d + dbase, kx[u]);
                        load4_f(V, row * d + dbase, vx[u]);
                    }
                }
            }
            float sc[kPasses];
            float bmax = kNegInf;
#pragma unroll
            for (int u = 0; u < kPasses; ++u) {
                float part = qv[0] * kx[u][0] + qv[1] * kx[u][1] + qv[2] * kx[u][2] + qv[3] * kx[u][3];
#pragma unroll
                for (int off = 1; off < LP; off <<= 1) part += shfl_xor_f(part, off);
                sc[u] = pb + u * PP + gs < p1 ? part * ksp[u] : kNegInf;
                bmax = fmaxf(bmax, sc[u]);
            }
            // a group may see no position of a batch (the last one)
            const float mnew = fmaxf(m, bmax);
            const float ref = mnew == kNegInf ? 0.0f : mnew;
            const float alpha = fast_exp2(m - ref);  // 0 while nothing was seen
            l *= alpha;
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] *= alpha;
#pragma unroll
            for (int u = 0; u < kPasses; ++u) {
                const float pw = fast_exp2(sc[u] - ref);  // 0 for masked positions
                l += pw;
                const float pwv = pw * vsp[u];
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[t] += pwv * vx[u][t];
            }
            m = mnew;
        }
        // merge the PP groups' states (lanes with the same dims)
#pragma unroll
        for (int off = LP; off < 64; off <<= 1) {
            const float mo = shfl_xor_f(m, off), lo = shfl_xor_f(l, off);
            float fa, fb, mn;
            rescale_pair(m, mo, fa, fb, mn);
            l = l * fa + lo * fb;
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t] = acc[t] * fa + shfl_xor_f(acc[t], off) * fb;
            m = mn;
        }
        const long row_out = (long)b * a.h + i;
        const float inv = l > 0.0f ? v_sc / l : 0.0f;  // l = 0: nothing visible
        const float4 o4 = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        if (single) {
            if (lane < LP && on) *reinterpret_cast<float4*>(a.out + row_out * d + dbase) = o4;
            if (lane == 0) a.lse[row_out] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : kNegInf;
        } else {
            const long prow = row_out * a.num_chunks + c;
            if (lane < LP && on) *reinterpret_cast<float4*>(a.part_o + prow * d + dbase) = o4;
            if (lane == 0) a.part_lse[prow] = l > 0.0f ? m + fast_log2(l) : kNegInf;
        }
        return;
    }
    float qv[NK], acc[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int dim = lane + 64 * kk;
        qv[kk] = dim < d ? load_f(q, ((long)b * a.h + i) * d + dim) * (a.scale_log2e * k_sc) : 0.0f;
        acc[kk] = 0.0f;
    }
    float m = kNegInf, l = 0.0f;
    // Positions go in batches of kBatch: the K and V loads of a batch are
    // issued together, so a batch costs one memory round trip.
    constexpr int kBatch = NK == 1 ? 16 : (sizeof(T) == 1 ? 4 : 8);  // FP8: room for the conversions
    auto row_of = [&](int p, bool fresh) -> long {
        if (fresh) return new_base + p;  // a row of k_new / v_new
        if (a.block_table != nullptr) {
            int phys = a.block_table[(long)b * a.max_blocks + (p >> a.log2_bs)];
            phys = phys < 0 ? 0 : (phys >= a.num_blocks ? a.num_blocks - 1 : phys);
            return ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
        }
        return contig_base + cache_slot(a, p);
    };
    for (int pb = p0; pb < p1; pb += kBatch) {
        float kx[kBatch][NK], vx[kBatch][NK];
        float ksp[kBatch], vsp[kBatch];  // per-block scales of the batch's positions
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = min(pb + u, p1 - 1);  // past the end: repeat the last position (masked)
            const bool fresh = appends && p >= raw;  // uniform over the wavefront
            const long row = row_of(p, fresh);
            ksp[u] = vsp[u] = 1.0f;
            if (bsc) {
                const long si = fp8_scale_index(a, b, j, p);
                ksp[u] = a.k_scale[si];
                vsp[u] = a.v_scale[si];
            }
            const float nk = bsc ? ksp[u] : k_sc, nv = bsc ? vsp[u] : v_sc;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                const int dim = lane + 64 * kk;
                kx[u][kk] = vx[u][kk] = 0.0f;
                if (dim < d) {
                    if (fresh) {
                        kx[u][kk] = new_value<T>(load_f((const TN*)a.k_new, row * d + dim), nk);
                        vx[u][kk] = new_value<T>(load_f((const TN*)a.v_new, row * d + dim), nv);
                    } else {
                        kx[u][kk] = load_f(K, row * d + dim);
                        vx[u][kk] = load_f(V, row * d + dim);
                    }
                }
            }
        }
        float sc[kBatch];
        float bmax = kNegInf;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            float part = 0.0f;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) part += qv[kk] * kx[u][kk];
            sc[u] = pb + u < p1 ? wave_sum(part) * ksp[u] : kNegInf;
            bmax = fmaxf(bmax, sc[u]);
        }
        const float mnew = fmaxf(m, bmax);
        const float alpha = fast_exp2(m - mnew);  // m = -inf on the first batch -> 0
        l *= alpha;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc[kk] *= alpha;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const float pw = fast_exp2(sc[u] - mnew);  // 0 for masked positions
            l += pw;
            const float pwv = pw * vsp[u];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) acc[kk] += pwv * vx[u][kk];
        }
        m = mnew;
    }

    const long row_out = (long)b * a.h + i;
    if (single) {
        const float inv = l > 0.0f ? v_sc / l : 0.0f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.out[row_out * d + dim] = acc[kk] * inv;
        }
        if (lane == 0) a.lse[row_out] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : kNegInf;
    } else {
        const long prow = row_out * a.num_chunks + c;
        const float inv = l > 0.0f ? v_sc / l : 0.0f;  // l = 0: nothing visible in this chunk
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int dim = lane + 64 * kk;
            if (dim < d) a.part_o[prow * d + dim] = acc[kk] * inv;
        }
        if (lane == 0) a.part_lse[prow] = l > 0.0f ? m + fast_log2(l) : kNegInf;
    }
}

int generic_rows_per_wg(int m) { return m < kGenericRows ? m : kGenericRows; }

// Head dims that are multiples of 4 take four dims per lane and
// LP = max(4, d/4 rounded up to a power of 2) lanes per position; others one
// lane per dim (d <= 64) or four (d > 64).
template <typename TQ, typename T>
static void launch_generic(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if (a.d % 4 == 0) {
        const int q = a.d / 4;
        if (q <= 4) decode_generic_kernel<TQ, T, 1, 4><<<grid, block, 0, s>>>(a);
        else if (q <= 8) decode_generic_kernel<TQ, T, 1, 8><<<grid, block, 0, s>>>(a);
        else if (q <= 16) decode_generic_kernel<TQ, T, 1, 16><<<grid, block, 0, s>>>(a);
        else if (q <= 32) decode_generic_kernel<TQ, T, 1, 32><<<grid, block, 0, s>>>(a);
        else decode_generic_kernel<TQ, T, 1, 64><<<grid, block, 0, s>>>(a);
    } else if (a.d <= 64) {
        decode_generic_kernel<TQ, T, 1, 0><<<grid, block, 0, s>>>(a);
    } else {
        decode_generic_kernel<TQ, T, 4, 0><<<grid, block, 0, s>>>(a);
    }
}

hipError_t launch_decode_generic(const DecodeArgs& a, int dtype, hipStream_t s) {
    const int R = generic_rows_per_wg(a.m), RB = (a.m + R - 1) / R;
    if (a.waves != R || (long)a.g * RB > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.num_chunks, (unsigned)(a.g * RB), (unsigned)a.B);
    const dim3 block((unsigned)(64 * R));
    if (a.kv8) launch_generic<uint16_t, uint8_t>(a, grid, block, s);
    else if (dtype == 0) launch_generic<float, float>(a, grid, block, s);
    else launch_generic<uint16_t, uint16_t>(a, grid, block, s);
    return hipGetLastError();
}

}  // namespace kvc
