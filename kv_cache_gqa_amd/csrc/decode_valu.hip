// decode_valu.hip -- bf16 or FP8 caches, head_dim 128, small query groups
// (at most 3 query rows per KV head).
//
// A work-group of four wavefronts computes one segment at a time: the m
// query heads that share KV head j of sequence b ("大语言模型研究15——注意力
// 机制优化之KV缓存" (limoncc.com) section 三 3.3: heads j*m..j*m+m-1 use KV
// head j) over a range of positions, so every K/V byte is read from HBM once.
// With m <= 3 the product is too thin for the matrix cores; it runs on the
// vector ALUs.
//
// Lane layout: lane l covers dims [8*(l%16), 8*(l%16)+8) of position
// (l/16) + 4u of the current 32-position sub-tile, u = 0..7.  One 16-byte
// load per lane per u reads four whole 256-byte K (or V) rows per wavefront
// instruction (FP8: 8 bytes, four 128-byte rows), fully coalesced, as
// streaming (non-temporal) loads.  q.k is
// v_dot2_f32_bf16 on the raw bf16 pairs, summed over the 16 lanes of a row
// with DPP.  Each row of 16 lanes keeps its own online-softmax state (m, l,
// acc) ("KV Cache 优化与注意力机制加速" (plumephp.com) section 2.2); the four
// row states of a wavefront and the four wavefronts are merged once at the
// end of the segment.
//
// Two entry points share the segment code: a chunked grid (chunk, KV head,
// sequence) and the persistent stream grid of kvc_schedule.h.

#include "kvc_schedule.h"

namespace kvc {

namespace {

constexpr int kD = 128;

// GEN: several query tokens per sequence, sliding windows or ring caches
// (per-row visibility masks, ring-aware windows).
// Registers of one wavefront's tile: rows 4u + lane/16, dims 8*(lane%16)
// .. +8, as bf16 or (FP8 cache) as raw codes converted when used.
template <bool KV8>
struct ValuTile {
    uint4 k[8];
    uint4 v[8];
};
template <>
struct ValuTile<true> {
    uint2 k[8];
    uint2 v[8];
};

// KV8: 0 = bf16 cache; 1 = FP8 E4M3 codes with a float32 scale per KV
// head, folded into the score scale (K) and the output (V); 2 = FP8 codes
// with a scale per (physical block, KV head) of a paged pool, applied per
// position to the score (K) and to the weight of its V row.
template <int M, bool PAGED, int W, bool GEN, int KV8>
struct ValuEngine {
    static constexpr bool kF8 = KV8 != 0;
    static constexpr bool kBS = KV8 == 2;  // per-block scales
    static_assert(!kBS || PAGED, "per-block scales need a paged pool");
    struct Shared {
        int tbl[PAGED ? kMaxTableSlice : 1];
        float bsc[kBS ? 2 * kMaxTableSlice : 1];  // per block: K scale, then V scale
        float red_m[W][M];
        float red_l[W][M];
        float red_o[W][M][kD];
        // one new token's rows; with general features over an FP8 cache, the
        // codes of a tile of new tokens (32 rows of 128 K then 128 V codes)
        __attribute__((aligned(16))) unsigned char nrow[GEN && !KV8 ? 1 : W][GEN && KV8 ? 32 * 256 : 512];
    };

    // The M query heads of KV head j of sequence b over positions [s, e)
    // (possibly empty).  Called by all 64*W threads.
    __device__ static void segment(const DecodeArgs& a, Shared& sh, int b, int j, int s, int e,
                                   const SegDst& dst) {
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        const int tsub = lane >> 4, ds = lane & 15;
        __syncthreads();  // the previous segment is done with the shared memory

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
            for (int k = 0; k < 8; ++k) acc[r][k] = 0.0f;
        }
        const long bj_base = ((long)b * a.g + j) * a.t_cap;
        long cbase = bj_base;  // row of position 0 in the current window (ring: shifted)
        const float k_sc = KV8 == 1 ? a.k_scale[j] : 1.0f;  // FP8 head scales
        const float v_sc = KV8 == 1 ? a.v_scale[j] : 1.0f;
        const float sl2 = a.scale_log2e * k_sc;
        const int* tbl = sh.tbl;
        int blk0 = 0;
        int w1 = e;

        auto kv_row = [&](int p) -> long {
            if (PAGED) {
                const int phys = tbl[(p >> a.log2_bs) - blk0];
                return ((long)phys * a.g + j) * a.block_size + (p & (a.block_size - 1));
            }
            return cbase + p;
        };
        // Row r is token r % n, which sees positions [lim[r] - wlen, lim[r]):
        // p is visible when lim - 1 - p, as unsigned, is below wlen (the
        // window, or 2^31).
        const int raw = a.seq_lens[b];
        const unsigned wlen = GEN && a.window > 0 ? (unsigned)a.window : 0x80000000u;
        int lim[M];
#pragma unroll
        for (int r = 0; r < M; ++r) lim[r] = GEN ? visible_len(a, raw, r % a.n) : 0;

        // A call that appends writes its new tokens (positions raw ..
        // raw+n-1, the last ones of the unit) into their cache slots here,
        // once per unit, and attends to them as a last tile built from
        // k_new / v_new (FP8: from their codes, n = 1).
        const int fresh_lo = max(s, raw);
        const bool has_new = a.k_new != nullptr && fresh_lo < e;  // at most n <= 3 positions
        const int e_cache = has_new ? fresh_lo : e;
        if (has_new) {
            if (KV8) store_new_rows_fp8_d128(a, b, j, raw, fresh_lo, e, tid, 64 * W);
            else store_new_rows_bf16_d128(a, b, j, raw, fresh_lo, e, tid, 64 * W);
        }
        // The wavefront that takes the new tile.  With one new token (always
        // so without GEN) it loads the token's K and V rows now, one bf16
        // pair of each per lane, so that the last tile does not wait for
        // them; the tile is then built from those pairs through LDS.
        constexpr bool kNewPair = !GEN;
        const bool new_wave = has_new && wave == ((fresh_lo - s) / kTileTokens) % W;
        const uint2 new_pair = kNewPair && new_wave ? new_row_pair_d128(a, b, j, lane) : make_uint2(0u, 0u);
        // scale index of the one new token (FP8 single-token calls)
        const long new_sidx = kBS && kNewPair && has_new ? fp8_scale_index(a, b, j, raw) : (long)j;
        const long bj = (long)b * a.g + j;
        const uint16_t* KN = has_new ? (const uint16_t*)a.k_new + bj * a.n * kD : K;
        const uint16_t* VN = has_new ? (const uint16_t*)a.v_new + bj * a.n * kD : Vc;

        // Positions clamped to the window's last one (in bounds past the end).
        // The tile's K rows are loaded before its V rows, kept in that order
        // (FP8 caches, and bf16 without the general features, which measured
        // faster that way; the bf16 general-feature kernels measured faster
        // with the order left to the compiler): the scores consume K first,
        // so a wait for K leaves the V loads in flight.
        auto load_tile = [&](int t0, ValuTile<kF8>& tr) {
            long rows[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) rows[u] = kv_row(min(t0 + 4 * u + tsub, w1 - 1));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if constexpr (KV8) tr.k[u] = ld8_stream((const unsigned char*)a.k + rows[u] * kD + 8 * ds);
                else tr.k[u] = ld16_stream(K + rows[u] * kD + 8 * ds);
            }
            if constexpr (KV8 || !GEN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if constexpr (KV8) tr.v[u] = ld8_stream((const unsigned char*)a.v + rows[u] * kD + 8 * ds);
                else tr.v[u] = ld16_stream(Vc + rows[u] * kD + 8 * ds);
            }
        };
        // The appended tokens' tile at t0 (>= raw): position p is row p - raw
        // of the unit's k_new / v_new rows; positions clamp to w1 - 1.  With
        // one new token every position of the tile is that token: its rows
        // (FP8: their codes) go to this wavefront's LDS area first.
        auto load_new_tile = [&](int t0, ValuTile<kF8>& tr) {
            if constexpr (KV8 && kNewPair) {
                unsigned char* codes = sh.nrow[wave];
                new_row_codes_fp8_d128(a, new_sidx, lane, new_pair, codes);
                wave_lds_sync();
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    tr.k[u] = *reinterpret_cast<const uint2*>(codes + 8 * ds);
                    tr.v[u] = *reinterpret_cast<const uint2*>(codes + 128 + 8 * ds);
                }
            } else if constexpr (kNewPair) {
                unsigned char* rows = sh.nrow[wave];
                reinterpret_cast<uint32_t*>(rows)[lane] = new_pair.x;        // K row, 256 bytes
                reinterpret_cast<uint32_t*>(rows + 256)[lane] = new_pair.y;  // V row
                wave_lds_sync();
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    tr.k[u] = *reinterpret_cast<const uint4*>(rows + 16 * ds);
                    tr.v[u] = *reinterpret_cast<const uint4*>(rows + 256 + 16 * ds);
                }
            } else if constexpr (KV8) {
                // several new tokens over an FP8 cache: the wavefront
                // quantises the tile's new rows once (positions t0 ..
                // min(t0 + 32, w1) - 1, rows p - raw of k_new / v_new; items
                // of 8 values spread over its lanes) into its LDS area, row
                // i as 128 K codes then 128 V codes, with the quotient and
                // encoder of the cache's append; the tile is then read from
                // there, positions past the last clamped to it.
                unsigned char* codes = sh.nrow[wave];
                const int nrows = min(t0 + 32, w1) - t0;
                for (int it = lane; it < nrows * 32; it += 64) {
                    const int i = it >> 5, hv = (it >> 4) & 1, ch = it & 15;
                    const long r = (long)(t0 - raw) + i;
                    const long si = kBS ? fp8_scale_index(a, b, j, (int)(raw + r)) : (long)j;
                    const float sc = hv ? a.v_scale[si] : a.k_scale[si];
                    const uint16_t* row = (hv ? VN : KN) + r * kD + 8 * ch;
                    *reinterpret_cast<uint2*>(codes + i * 256 + hv * kD + 8 * ch) = e4m3_encode8(ld16(row), sc);
                }
                wave_lds_sync();
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = min(t0 + 4 * u + tsub, w1 - 1) - t0;
                    tr.k[u] = *reinterpret_cast<const uint2*>(codes + i * 256 + 8 * ds);
                    tr.v[u] = *reinterpret_cast<const uint2*>(codes + i * 256 + kD + 8 * ds);
                }
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const long r = min(t0 + 4 * u + tsub, w1 - 1) - raw;
                    tr.k[u] = ld16(KN + r * kD + 8 * ds);
                    tr.v[u] = ld16(VN + r * kD + 8 * ds);
                }
            }
        };
        auto as_bf16 = [&](const auto& x) -> uint4 {
            if constexpr (KV8) return e4m3x8_to_bf16(x);
            else return x;
        };
        // fresh: a tile of appended tokens (their scales are looked up, not
        // in the table slice)
        auto compute_tile = [&](int t0, const ValuTile<kF8>& tr, bool fresh) {
            // per-block scales of the lane's eight positions
            float sk[8], vf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sk[u] = sl2;
                vf[u] = 1.0f;
                if constexpr (kBS) {
                    const int p = min(t0 + 4 * u + tsub, w1 - 1);
                    if (fresh) {
                        const long si = fp8_scale_index(a, b, j, p);
                        sk[u] = sl2 * a.k_scale[si];
                        vf[u] = a.v_scale[si];
                    } else {
                        const int bi = (p >> a.log2_bs) - blk0;
                        sk[u] = sl2 * sh.bsc[bi];
                        vf[u] = sh.bsc[kMaxTableSlice + bi];
                    }
                }
            }
            float sc[M][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = t0 + 4 * u + tsub;
                const uint4 kb = as_bf16(tr.k[u]);
#pragma unroll
                for (int r = 0; r < M; ++r) {
                    float dot = dot2_bf16(qp[r][0], kb.x, 0.0f);
                    dot = dot2_bf16(qp[r][1], kb.y, dot);
                    dot = dot2_bf16(qp[r][2], kb.z, dot);
                    dot = dot2_bf16(qp[r][3], kb.w, dot);
                    dot = row16_sum(dot) * sk[u];
                    const bool vis = GEN ? (p < w1 && (unsigned)(lim[r] - 1 - p) < wlen) : p < w1;
                    sc[r][u] = vis ? dot : kNegInf;
                }
            }
            float pr[M][8];
#pragma unroll
            for (int r = 0; r < M; ++r) {
                float mt = sc[r][0];
#pragma unroll
                for (int u = 1; u < 8; ++u) mt = fmaxf(mt, sc[r][u]);
                const float mnew = fmaxf(mrun[r], mt);
                const float ref = (mnew == kNegInf) ? 0.0f : mnew;
                const float alpha = fast_exp2(mrun[r] - ref);
                mrun[r] = mnew;
                float lsum = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    pr[r][u] = fast_exp2(sc[r][u] - ref);
                    lsum += pr[r][u];
                }
                lrun[r] = lrun[r] * alpha + lsum;
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[r][k] *= alpha;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint4 vb = as_bf16(tr.v[u]);
                const float vfl[8] = {bf16_lo(vb.x), bf16_hi(vb.x), bf16_lo(vb.y), bf16_hi(vb.y),
                                      bf16_lo(vb.z), bf16_hi(vb.z), bf16_lo(vb.w), bf16_hi(vb.w)};
#pragma unroll
                for (int r = 0; r < M; ++r) {
                    const float w = kBS ? pr[r][u] * vf[u] : pr[r][u];
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[r][k] += w * vfl[k];
                }
            }
        };

        // Windows of at most kMaxChunk positions (block-table slice in LDS).
        for (int w0 = s; w0 < e_cache; w0 = w1) {
            w1 = min(e_cache, w0 + kMaxChunk);
            if (GEN && !PAGED && a.ring) {
                // a window never wraps around the ring: slot = p - wbase in it
                const int wbase = w0 - w0 % a.t_cap;
                w1 = min(w1, wbase + a.t_cap);
                cbase = bj_base - wbase;
            }
            if (PAGED) {
                blk0 = w0 >> a.log2_bs;
                const int nblk = ((w1 - 1) >> a.log2_bs) - blk0 + 1;
                for (int t = tid; t < nblk; t += 64 * W) {
                    int ph = a.block_table[(long)b * a.max_blocks + blk0 + t];
                    ph = ph < 0 ? 0 : (ph >= a.num_blocks ? a.num_blocks - 1 : ph);
                    sh.tbl[t] = ph;
                    if constexpr (kBS) {
                        sh.bsc[t] = a.k_scale[(long)ph * a.g + j];
                        sh.bsc[kMaxTableSlice + t] = a.v_scale[(long)ph * a.g + j];
                    }
                }
                __syncthreads();
            }
            const int stride = W * kTileTokens;
            int t0 = w0 + wave * kTileTokens;
            ValuTile<kF8> tA, tB;
            load_tile(t0, tA);
            for (;;) {
                if (t0 >= w1) break;
                load_tile(t0 + stride, tB);
                compute_tile(t0, tA, false);
                t0 += stride;
                if (t0 >= w1) break;
                load_tile(t0 + stride, tA);
                compute_tile(t0, tB, false);
                t0 += stride;
            }
            if (PAGED) __syncthreads();  // the next window rewrites the table slice
        }
        // The appended tokens (the last positions of the unit) are taken
        // last, as one tile by the wavefront next in turn.
        if (new_wave) {
            w1 = e;
            ValuTile<kF8> tr;
            load_new_tile(fresh_lo, tr);
            compute_tile(fresh_lo, tr, true);
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
                for (int k = 0; k < 8; ++k) {
                    const float ao = shfl_xor_f(acc[r][k], mask);
                    acc[r][k] = acc[r][k] * fa + ao * fb;
                }
                mrun[r] = mnew;
            }
        }
        if (tsub == 0) {
#pragma unroll
            for (int r = 0; r < M; ++r) {
#pragma unroll
                for (int k = 0; k < 8; ++k) sh.red_o[wave][r][8 * ds + k] = acc[r][k];
                if (ds == 0) {
                    sh.red_m[wave][r] = mrun[r];
                    sh.red_l[wave][r] = lrun[r];
                }
            }
        }
        __syncthreads();

        // Merge the W wavefronts and write the rows.
        for (int idx = tid; idx < M * kD; idx += 64 * W) {
            const int r = idx / kD, dim = idx % kD;
            float mm = sh.red_m[0][r];
#pragma unroll
            for (int w = 1; w < W; ++w) mm = fmaxf(mm, sh.red_m[w][r]);
            const float ref = (mm == kNegInf) ? 0.0f : mm;
            float l = 0.0f, o = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float f = fast_exp2(sh.red_m[w][r] - ref);
                l += sh.red_l[w][r] * f;
                o += sh.red_o[w][r][dim] * f;
            }
            dst.o[(long)r * dst.o_stride + dim] = l > 0.0f ? o * v_sc / l : 0.0f;  // FP8: V head scale
            if (dim == 0) {
                float v;
                if (dst.final_) v = l > 0.0f ? (mm + fast_log2(l)) * kLn2 : kNegInf;
                else v = l > 0.0f ? mm + fast_log2(l) : kNegInf;
                dst.lse[(long)r * dst.lse_stride] = v;
            }
        }
    }
};

}  // namespace

template <int M, bool PAGED, int W, bool GEN, int KV8>
__global__ void __launch_bounds__(64 * W) decode_valu_chunked(DecodeArgs a) {
    using E = ValuEngine<M, PAGED, W, GEN, KV8>;
    __shared__ typename E::Shared sh;
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    // chunks cover [lo, hi); without the general features lo = 0
    const PosRange ur = GEN ? unit_range(a, a.seq_lens[b])
                            : PosRange{0, attended_len(a, a.seq_lens[b])};
    const int p0 = ur.lo + c * a.chunk_len;
    const int p1 = min(p0 + a.chunk_len, ur.hi);
    const bool single = a.num_chunks == 1;
    if (p0 >= ur.hi && !single) {  // past the end: a record of weight 0 for the merge
        mark_empty_rows(chunk_dst(a, b, j, c), M, threadIdx.x);
        return;
    }
    E::segment(a, sh, b, j, p0, p1, chunk_dst(a, b, j, c));
}

template <int M, bool PAGED, int W, bool GEN, int KV8>
__global__ void __launch_bounds__(64 * W) decode_valu_stream(DecodeArgs a) {
    using E = ValuEngine<M, PAGED, W, GEN, KV8>;
    __shared__ typename E::Shared sh;
    __shared__ long long cum[kStreamMaxB + 1];
    stream_prefix(a, cum);
    stream_walk(a, cum, [&](int b, int j, int s, int e, bool complete, int slot) {
        const int lo = GEN ? unit_range(a, a.seq_lens[b]).lo : 0;  // walk offsets are relative to it
        E::segment(a, sh, b, j, lo + s, lo + e, complete ? final_dst(a, b, j) : stream_dst(a, slot));
    });
}

template <int M, bool PG, int KV>
static const void* valu_pick_kv(bool stream, bool gen) {
    if (stream)
        return gen ? (const void*)decode_valu_stream<M, PG, 4, true, KV>
                   : (const void*)decode_valu_stream<M, PG, 4, false, KV>;
    return gen ? (const void*)decode_valu_chunked<M, PG, 4, true, KV>
               : (const void*)decode_valu_chunked<M, PG, 4, false, KV>;
}

template <int M, bool PG>
static const void* valu_pick(bool stream, bool gen, int kv8) {
    if (kv8 == 2) {  // per-block scales: paged pools only
        if constexpr (PG) return valu_pick_kv<M, PG, 2>(stream, gen);
        else return nullptr;
    }
    return kv8 ? valu_pick_kv<M, PG, 1>(stream, gen) : valu_pick_kv<M, PG, 0>(stream, gen);
}

// Kernel function for (m, layout, split mode, wavefronts per work-group,
// general features, FP8 cache); nullptr when that combination is not built.
// Only 4-wavefront kernels: one wide work-group per (sequence, KV head)
// measured slower than split chunks plus a merge for these kernels (8, 12
// and 16 wavefronts, m = 1; 12 keeps the occupancy of three chunks but not
// their balance).
const void* valu_kernel(int m, bool paged, bool stream, int waves, bool gen, int kv8) {
    if (waves != 4) return nullptr;
    switch (m) {
        case 1: return paged ? valu_pick<1, true>(stream, gen, kv8) : valu_pick<1, false>(stream, gen, kv8);
        case 2: return paged ? valu_pick<2, true>(stream, gen, kv8) : valu_pick<2, false>(stream, gen, kv8);
        case 3: return paged ? valu_pick<3, true>(stream, gen, kv8) : valu_pick<3, false>(stream, gen, kv8);
        default: return nullptr;
    }
}

hipError_t launch_decode_valu_bf16_d128(const DecodeArgs& a, hipStream_t s) {
    const void* fn = valu_kernel(a.m, a.block_table != nullptr, a.stream != 0, a.waves,
                                 general_features(a), kv_mode(a));
    if (fn == nullptr) return hipErrorInvalidValue;
    const dim3 grid = a.stream ? dim3((unsigned)a.num_wgs)
                               : dim3((unsigned)a.num_chunks, (unsigned)a.g, (unsigned)a.B);
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    return hipLaunchKernel(fn, grid, dim3(64 * a.waves), args, 0, s);
}

}  // namespace kvc
