// prefill.hip -- bf16 caches, head_dim 128, more than 32 query rows per KV
// head: several new tokens per sequence attending at once (the new tokens
// of a prefill after a cached prefix, "大语言模型研究15——注意力机制优化之KV
// 缓存" (limoncc.com) section 5.2; draft tokens checked in one pass, "KV
// Cache 优化与注意力机制加速" (plumephp.com) section 5.3), or more than 32
// query heads per KV head.
//
// Query rows of one unit (sequence b, KV head j) are r = 0 .. m-1, m = (h/g)
// * n; row r is query head j*(h/g) + r / n, token r % n, and token t sees
// the positions below raw + len_add - (n - 1 - t): the causal mask of the
// whole sequence aligned to its bottom-right corner (the zwjcode.cn page,
// section 13, warns that a non-square is_causal mask is aligned top-left),
// cut to a sliding window when one is given.
//
// A work-group of W wavefronts serves 16*NQT*W consecutive rows of one unit
// over one range of positions, 64 positions (two 32-position tiles) per
// step.  A step's K and V are read from memory once per work-group into LDS
// (every thread moves 16-byte pieces; the next step's pieces are in
// registers while this step is computed, and with 256 rows per work-group
// the step after it is loading too; two LDS buffers, one barrier per step) and every wavefront reads them there for its own 16*NQT rows, so a
// unit's K/V is read once per row block instead of once per 32 rows.  Work-groups of the row blocks of
// one unit get ids eight apart: MI355X hands work-group ids to its eight
// XCDs in turn, so they run on one XCD at about the same time and share the
// K/V lines in its L2.
//
// Per wavefront and tile, on the matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulate), as in the single-token kernels:
//   S^T[16 pos x 16 rows] = K[16 pos x 128] . Q^T[128 x 16 rows]: the A
//     operand is read from LDS (lane l: 16 bytes of K row l % 16 at dims
//     32*ks + 8*(l/16)), the B operand is the wavefront's queries in
//     registers.
//   O^T[16 dims x 16 rows] += V^T[16 dims x 32 pos] . P^T[32 pos x 16 rows]:
//     the S^T result already sits in the B-operand layout (lane l holds
//     positions 4*(l/16) + v of both 16-position halves), and the A operand
//     comes from transposing LDS reads of the V tile.
//   An all-ones A operand gives the column sums of the bf16-rounded P.
// Online softmax per row in base 2 ("KV Cache 优化与注意力机制加速"
// (plumephp.com) section 2.2) with the lazy rescale of the single-token
// kernels: the running reference moves only when a step maximum passes it by
// more than 8; out = sum bf16(P) V / sum bf16(P); lse = m + log2 of the fp32
// sum of P.  Wavefronts own disjoint rows and see the same positions, so
// each writes its rows directly, no merge between wavefronts.
//
// A call that appends reads its new positions (raw .. raw+n-1) from k_new /
// v_new, and the work-group of the first row block writes them into the
// cache.

#include "kvc_schedule.h"

namespace kvc {

namespace {

constexpr float kLazyRescale = 8.0f;

// Sizes for head dimension D (64, 80, 96, 128 or 256; bf16 rows of 2*D
// bytes in 16-byte chunks).  The products run over kDP dims, D rounded up to
// a multiple of 32: at D = 80 dims 80..95 are zero in the staged K rows and
// in the queries, so they add nothing to the scores.  Staged rows of 80 or
// 96 dims take the 256-byte pitch of 128-dim rows (the other chunk slots of
// a row unused), so that they keep that layout's swizzles.
template <int D>
struct PfDims {
    static constexpr int kDP = (D + 31) / 32 * 32;            // dims of the score product
    static constexpr int kRowB = 2 * D;                       // bytes of one K or V row
    static constexpr int kPitch = (D == 80 || D == 96) ? 256 : kRowB;  // bytes between staged rows in LDS
    static constexpr int kTileB = kTileTokens * kPitch;       // one staged 32-position tile of K (or V)
    static constexpr int kKs = kDP / 32;                      // 32-dim steps of Q K^T
    static constexpr int kNt = D / 16;                        // 16-dim tiles of O

    // LDS offset of 16-byte chunk c of K row r.  An A-operand read touches
    // rows 0..15 at one chunk: with a pitch of 256 or 512 bytes the chunks
    // are XOR-swizzled by r % 16 (16 different slots of a 256-byte bank row;
    // a 96-dim row's chunks 0..11 land in slots 0..15); with 128-byte rows
    // two rows share a bank row, so the slot follows (r / 2) % 8 and the
    // row's half does the rest.  No conflict either way.
    __device__ static int k_off(int r, int c) {
        const int swz = D == 64 ? (r >> 1) & 7 : r & 15;
        return r * kPitch + ((c ^ swz) << 4);
    }
    // V rows: the swizzle of the transposing reads, rows R..R+3 (R = 4k) on
    // disjoint 32-byte slices of the 256-byte bank row, chunk pairs (2k,
    // 2k+1) kept adjacent.
    __device__ static int v_off(int r, int c) { return r * kPitch + ((c ^ ((r & 3) << 1)) << 4); }
};

// KV8: 0 = bf16 cache; 1 = FP8 E4M3 codes with a float32 scale per KV head.
// The codes are widened to bf16 when a tile is staged in LDS (exact: every
// E4M3 value is a bf16 value), so the tiles and products are those of bf16;
// the K scale is folded into the score scale and the V scale into the
// output.  New tokens (bf16 in k_new / v_new) are staged as the values of
// their codes, the same quotient and encoder the stored codes get.
template <int NQT, int W, bool PAGED, int D, int KV8>
struct PrefillEngine {
    using Dm = PfDims<D>;
    static constexpr int kRowB = Dm::kRowB;                // bytes of one staged (bf16) row
    static constexpr int kCacheRowB = KV8 ? D : 2 * D;     // bytes of one cached row
    static constexpr int kTileB = Dm::kTileB;
    static constexpr int kRowsPerWave = 16 * NQT;
    static constexpr int kRowsPerGroup = kRowsPerWave * W;
    // Positions per step: kSub tiles of 32, so that a barrier covers 64
    // positions and each wavefront has two independent score products in
    // flight (measured: 0.29 -> 0.33 of the matrix-core peak at 1024 rows,
    // D = 128).  With D = 256 one tile: two would need 128 KB of LDS per
    // work-group.
    static constexpr int kSub = D == 256 ? 1 : 2;
    static constexpr int kSpan = kSub * kTileTokens;
    // A piece is what one thread moves with one 16-byte load: 8 bf16
    // elements, or 16 FP8 codes (two staged chunks) when the step has at
    // least one K piece of that size per thread (else 8 codes, 8 bytes).
    // At D = 80 and 96 the wide pieces would leave an odd count per thread,
    // so 8 codes.  A staged row has kPPR pieces, the first kReal of them
    // from the row's D dims, the others (D = 80) zero.
    static constexpr bool kWide = KV8 && D != 80 && D != 96 && kSub * kTileTokens * (D / 16) >= 64 * W;
    static constexpr int kPE = kWide ? 16 : 8;                // elements per piece
    static constexpr int kPPR = Dm::kDP / kPE;                // pieces per staged row
    static constexpr int kReal = D / kPE;                     // pieces per row that hold its dims
    static constexpr int kPieceB = KV8 ? kPE : 16;            // cached bytes of one piece
    static constexpr int kStepPieces = 2 * kSub * kTileTokens * kPPR;  // K and V pieces per step
    static constexpr int kPer = kStepPieces / (64 * W);       // pieces per thread per step
    static_assert(kPer >= 2 && kPer * 64 * W == kStepPieces, "pieces must divide evenly");
    static_assert(kPer % 2 == 0, "a thread moves as many K pieces as V pieces");

    struct Shared {
        uint32_t tbl[PAGED ? kMaxTableSlice : 1];  // per block: row of its first position, head j
        __attribute__((aligned(16))) unsigned char k[2][kSub * kTileB];  // tile s at s * kTileB
        __attribute__((aligned(16))) unsigned char v[2][kSub * kTileB];
    };

    // Rows rb*kRowsPerGroup .. +kRowsPerGroup of unit (b, j) over positions
    // [s, e); results go to `dst` (row 0 of the unit there: a chunk's
    // records, a stream work-group's record slot, or the final rows).
    // Called by all 64*W threads; may be called again for another segment.
    __device__ static void run(const DecodeArgs& a, Shared& sh, int b, int j, int rb, int s, int e,
                               const SegDst& unit_dst) {
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        const int G = lane >> 4, col = lane & 15;
        const int row0 = rb * kRowsPerGroup + wave * kRowsPerWave;  // this wavefront's first row
        const int rows = min(a.m - row0, kRowsPerWave);             // may be <= 0
        const int raw = a.seq_lens[b];
        const long bj = (long)b * a.g + j;

        // B operands of Q K^T: row 16*qt + col, dims 32*ks + 8*G .. +8.
        const uint16_t* Q = (const uint16_t*)a.q;
        uint4 qb[NQT][Dm::kKs];
        int lim[NQT];  // positions below lim are visible to the lane's row
        const unsigned wlen = a.window > 0 ? (unsigned)a.window : 0x80000000u;
        // The wavefront's rows see positions in [lo_w, hi_w) between them;
        // every one of them sees [full_lo, full_hi), where no mask is needed.
        int hi_w = 0, lo_w = 0x7fffffff, full_lo = 0, full_hi = 0x7fffffff;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            const int qi = 16 * qt + col;
            const bool ok = qi < rows;
#pragma unroll
            for (int ks = 0; ks < Dm::kKs; ++ks)
                qb[qt][ks] = ok && 32 * ks + 8 * G < D
                                 ? ld16(Q + ((b * (long)a.h + (long)j * a.m + row0 + qi) * D + 32 * ks + 8 * G))
                                 : make_uint4(0u, 0u, 0u, 0u);
            lim[qt] = visible_len(a, raw, (row0 + qi) % a.n);
            if (ok) {
                const int wl = window_lo(a, lim[qt]);
                hi_w = max(hi_w, lim[qt]);
                lo_w = min(lo_w, wl);
                full_hi = min(full_hi, lim[qt]);
                full_lo = max(full_lo, wl);
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            hi_w = max(hi_w, __shfl_xor(hi_w, off, 64));
            lo_w = min(lo_w, __shfl_xor(lo_w, off, 64));
            full_hi = min(full_hi, __shfl_xor(full_hi, off, 64));
            full_lo = max(full_lo, __shfl_xor(full_lo, off, 64));
        }

        f32x4_t acc[NQT][Dm::kNt];
        f32x4_t lacc[NQT];  // sums of bf16-rounded P (normalise out)
        float lex[NQT];     // sums of fp32 P over this lane's positions (give lse)
        float mrun[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            mrun[qt] = kNegInf;
            lex[qt] = 0.0f;
            lacc[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < Dm::kNt; ++nt) acc[qt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        const float k_sc = KV8 ? a.k_scale[j] : 1.0f, v_sc = KV8 ? a.v_scale[j] : 1.0f;
        const float sl2 = a.scale_log2e * k_sc;

        // The appended tokens: positions raw .. come from k_new / v_new rows
        // (b, j, p - raw); the first row block's work-group writes this
        // range's new positions into the cache (the kernels never read the
        // cache there, so nothing waits for the writes).
        const bool appends = a.k_new != nullptr;
        if (appends && rb == 0 && max(s, raw) < e) {
            if constexpr (KV8) store_new_rows_fp8<D>(a, b, j, raw, max(s, raw), e, tid, 64 * W);
            else store_new_rows_bf16<D>(a, b, j, raw, max(s, raw), e, tid, 64 * W);
        }
        const char* knew = appends ? (const char*)a.k_new + bj * a.n * kRowB - (long)raw * kRowB : nullptr;
        const char* vnew = appends ? (const char*)a.v_new + bj * a.n * kRowB - (long)raw * kRowB : nullptr;

        // Several work-groups (row blocks) read each K/V line: ordinary loads
        // keep it in L2 for the others; a single reader streams.
        const bool reread = a.row_blocks > 1;
        int blk0 = 0, w1 = e;
        const char* kbase = (const char*)a.k;
        const char* vbase = (const char*)a.v;
        // Address of piece pc of K (or V) at position p: in k_new / v_new
        // (bf16) for appended positions, else in the cache.
        auto fresh_src = [&](bool isv, int p, int pc) -> const char* {
            return (isv ? vnew : knew) + (long)p * kRowB + 2 * kPE * pc;
        };
        auto cache_src = [&](bool isv, int p, int pc) -> const char* {
            const char* base = isv ? vbase : kbase;
            uint64_t row;
            if (PAGED) row = sh.tbl[(p >> a.log2_bs) - blk0] + (uint32_t)(p & (a.block_size - 1));
            else row = (uint64_t)(bj * a.t_cap + cache_slot(a, p));
            return base + row * kCacheRowB + kPieceB * pc;
        };
        auto src = [&](bool isv, int p, int pc) -> const void* {
            return appends && p >= raw ? fresh_src(isv, p, pc) : cache_src(isv, p, pc);
        };
        // staged pieces in registers: bf16 values, or (FP8) their codes
        std::conditional_t<KV8 != 0 && !kWide, uint2, uint4> pre[kPer];
        // Pieces of the step at t0 into registers: the thread's pieces k <
        // kPer/2 are of K, the others of V; piece k is row q / kPPR, piece q %
        // kPPR of the row with q = tid + (k % (kPer/2)) * 64*W; positions past
        // the range repeat its last one (masked).
        constexpr int kHalf = kPer / 2;
        // FP8: an appended position's bf16 values are quantised as they
        // arrive (the quotient and encoder of the stored codes), which waits
        // for those loads: one step per unit has them.
        auto load_tile = [&](int t0) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int q = tid + (k % kHalf) * 64 * W;
                const int p = min(t0 + q / kPPR, w1 - 1);
                const bool isv = k >= kHalf;
                if constexpr (kReal < kPPR) {
                    if (q % kPPR >= kReal) {  // padding dims: zero
                        if constexpr (KV8 && !kWide) pre[k] = make_uint2(0u, 0u);
                        else pre[k] = make_uint4(0u, 0u, 0u, 0u);
                        continue;
                    }
                }
                if constexpr (KV8) {
                    const float sc = isv ? v_sc : k_sc;
                    if (appends && p >= raw) {
                        const char* f = fresh_src(isv, p, q % kPPR);
                        if constexpr (kWide) {
                            const uint2 lo = e4m3_encode8(ld16(f), sc), hi = e4m3_encode8(ld16(f + 16), sc);
                            pre[k] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                        } else {
                            pre[k] = e4m3_encode8(ld16(f), sc);
                        }
                    } else {
                        const void* ptr = cache_src(isv, p, q % kPPR);
                        if constexpr (kWide) pre[k] = reread ? ld16(ptr) : ld16_stream(ptr);
                        else pre[k] = reread ? ld8(ptr) : ld8_stream(ptr);
                    }
                } else {
                    const void* ptr = src(isv, p, q % kPPR);
                    pre[k] = reread ? ld16(ptr) : ld16_stream(ptr);
                }
            }
        };
        // 16-byte staged chunk c of row r (within the step) of K or V, buffer buf
        auto chunk_at = [&](bool isv, int buf, int r, int c) -> uint4* {
            const int off = (r >> 5) * kTileB + (isv ? Dm::v_off(r & 31, c) : Dm::k_off(r & 31, c));
            return reinterpret_cast<uint4*>((isv ? sh.v[buf] : sh.k[buf]) + off);
        };
        auto stage_tile = [&](int buf) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int q = tid + (k % kHalf) * 64 * W;
                const int r = q / kPPR, pc = q % kPPR;
                const bool isv = k >= kHalf;
                if constexpr (KV8 && kWide) {
                    *chunk_at(isv, buf, r, 2 * pc) = e4m3x8_to_bf16(make_uint2(pre[k].x, pre[k].y));
                    *chunk_at(isv, buf, r, 2 * pc + 1) = e4m3x8_to_bf16(make_uint2(pre[k].z, pre[k].w));
                } else if constexpr (KV8) {
                    *chunk_at(isv, buf, r, pc) = e4m3x8_to_bf16(pre[k]);
                } else {
                    *chunk_at(isv, buf, r, pc) = pre[k];
                }
            }
        };

        auto compute_tile = [&](int t0, int buf) {
            f32x4_t S[kSub][NQT][2];
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                const unsigned char* kt = sh.k[buf] + u * kTileB;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                    for (int qt = 0; qt < NQT; ++qt) S[u][qt][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < Dm::kKs; ++ks) {
                        const uint4 ka = *reinterpret_cast<const uint4*>(kt + Dm::k_off(16 * tt + col, 4 * ks + G));
#pragma unroll
                        for (int qt = 0; qt < NQT; ++qt) S[u][qt][tt] = mfma_bf16(ka, qb[qt][ks], S[u][qt][tt]);
                    }
                }
            }
            // Every row of the wavefront sees the whole step: no mask.
            const bool full = t0 >= full_lo && t0 + kSpan <= min(full_hi, w1);
            uint4 pb[kSub][NQT];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                // sv[8u + 4tt + v]: position t0 + 32u + 16tt + 4G + v
                float sv[8 * kSub];
                if (full) {
#pragma unroll
                    for (int k = 0; k < 8 * kSub; ++k) sv[k] = S[k >> 3][qt][(k >> 2) & 1][k & 3] * sl2;
                } else {
#pragma unroll
                    for (int k = 0; k < 8 * kSub; ++k) {
                        const int p = t0 + 32 * (k >> 3) + 16 * ((k >> 2) & 1) + 4 * G + (k & 3);
                        const bool vis = p < w1 && (unsigned)(lim[qt] - 1 - p) < wlen;
                        sv[k] = vis ? S[k >> 3][qt][(k >> 2) & 1][k & 3] * sl2 : kNegInf;
                    }
                }
                float mt = sv[0];
#pragma unroll
                for (int k = 1; k < 8 * kSub; ++k) mt = fmaxf(mt, sv[k]);
                mt = max_rows4(mt);
                if (__any(mt > mrun[qt] + kLazyRescale)) {  // uniform branch
                    const float mnew = fmaxf(mrun[qt], mt);
                    const float r = (mnew == kNegInf) ? 0.0f : mnew;
                    const float alpha = fast_exp2(mrun[qt] - r);  // 0 while nothing was seen
                    mrun[qt] = mnew;
#pragma unroll
                    for (int nt = 0; nt < Dm::kNt; ++nt) acc[qt][nt] *= alpha;
                    lacc[qt] *= alpha;
                    lex[qt] *= alpha;
                }
                const float ref = (mrun[qt] == kNegInf) ? 0.0f : mrun[qt];
#pragma unroll
                for (int u = 0; u < kSub; ++u) {
                    float pv[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) pv[k] = fast_exp2(sv[8 * u + k] - ref);
                    lex[qt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                    pb[u][qt] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
                }
            }
            // PV: lane 16G + 4r + qd reads 8 bytes of V rows 4G + r and
            // 16 + 4G + r at dims 16*nt + 4*qd; the transposing read hands
            // lane 16G + i dim 16*nt + i of those rows.
            const int tr_r = (lane >> 2) & 3, tr_q = lane & 3;
            const int r0 = 4 * G + tr_r, r1 = 16 + 4 * G + tr_r;
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                const unsigned char* vt = sh.v[buf] + u * kTileB;
#pragma unroll
                for (int nt = 0; nt < Dm::kNt; ++nt) {
                    const int ch = 2 * nt + (tr_q >> 1), sub = (tr_q & 1) * 8;
                    const uint2 lo = lds_read_tr16(vt + Dm::v_off(r0, ch) + sub);
                    const uint2 hi = lds_read_tr16(vt + Dm::v_off(r1, ch) + sub);
                    const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                    for (int qt = 0; qt < NQT; ++qt) acc[qt][nt] = mfma_bf16(av, pb[u][qt], acc[qt][nt]);
                }
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) lacc[qt] = mfma_bf16(ones, pb[u][qt], lacc[qt]);
            }
        };

        // Windows of at most kMaxChunk positions, so that a window's slice
        // of the block table fits in LDS; within a window, tiles of 32.
        for (int w0 = s; w0 < e; w0 = w1) {
            w1 = min(e, w0 + kMaxChunk);
            if (PAGED) {
                blk0 = w0 >> a.log2_bs;
                const int nblk = ((w1 - 1) >> a.log2_bs) - blk0 + 1;
                for (int t = tid; t < nblk; t += 64 * W) {
                    int ph = a.block_table[(long)b * a.max_blocks + blk0 + t];
                    ph = ph < 0 ? 0 : (ph >= a.num_blocks ? a.num_blocks - 1 : ph);
                    sh.tbl[t] = ((uint32_t)ph * (uint32_t)a.g + (uint32_t)j) * (uint32_t)a.block_size;
                }
                __syncthreads();
            }
            int t0 = w0;
            load_tile(t0);
            stage_tile(0);
            if (t0 + kSpan < w1) load_tile(t0 + kSpan);
            __syncthreads();
            int buf = 0;
            for (; t0 < w1; t0 += kSpan) {
                // a wavefront whose rows see none of the step skips it
                const bool busy = rows > 0 && t0 < hi_w && t0 + kSpan > lo_w;
                // 8-wavefront work-groups (256 rows: the products bound the
                // step) stage the next step into the other LDS buffer (last
                // read before the previous barrier) and load the one after
                // it before this step's products, so that those loads are
                // in flight while it computes (the barrier waits for every
                // load in flight); the 4-wavefront shapes, bound by memory,
                // measured faster staging and loading after the products.
                if constexpr (W == 8) {
                    if (t0 + kSpan < w1) stage_tile(buf ^ 1);
                    if (t0 + 2 * kSpan < w1) load_tile(t0 + 2 * kSpan);
                    if (busy) compute_tile(t0, buf);
                } else {
                    if (busy) compute_tile(t0, buf);
                    if (t0 + kSpan < w1) stage_tile(buf ^ 1);
                    if (t0 + 2 * kSpan < w1) load_tile(t0 + 2 * kSpan);
                }
                __syncthreads();
                buf ^= 1;
            }
        }

        // lex holds this lane's positions only: sum the four row groups.
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) lex[qt] = sum_rows4(lex[qt]);
        if (rows <= 0) return;
        SegDst dst = unit_dst;
        dst.o += (long)row0 * dst.o_stride;
        dst.lse += (long)row0 * dst.lse_stride;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            const int qi = 16 * qt + col;
            if (qi >= rows) continue;
            const float lr = lacc[qt][0];
            const float inv = lr > 0.0f ? v_sc / lr : 0.0f;
#pragma unroll
            for (int nt = 0; nt < Dm::kNt; ++nt)
                *reinterpret_cast<f32x4_t*>(dst.o + (long)qi * dst.o_stride + 16 * nt + 4 * G) = acc[qt][nt] * inv;
            if (G == 0) {
                const float l = lex[qt];
                float v;
                if (dst.final_) v = l > 0.0f ? (mrun[qt] + fast_log2(l)) * kLn2 : kNegInf;
                else v = l > 0.0f ? mrun[qt] + fast_log2(l) : kNegInf;
                dst.lse[(long)qi * dst.lse_stride] = v;
            }
        }
    }
};

}  // namespace

// Resident wavefronts per SIMD the register allocator is asked to allow:
// two (a 64-position step holds up to 256 registers per lane).
constexpr int kPrefillWavesPerEu = 2;

// Grid: one work-group per (chunk, KV head, sequence, row block), as a 1-D
// grid.  Units u = (b*g + j)*C + c go in groups of eight (the last group may
// be narrower); within a group of width w, row block r of unit k has id
// r*w + k, so the row blocks of a unit get ids eight apart.
template <int NQT, int W, bool PAGED, int D, int KV8>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(kPrefillWavesPerEu)))
prefill_mfma(DecodeArgs a) {
    using E = PrefillEngine<NQT, W, PAGED, D, KV8>;
    __shared__ typename E::Shared sh;
    const long id = blockIdx.x;
    const long units = (long)a.num_chunks * a.g * a.B;
    const int R = a.row_blocks;
    const long grp = id / (8L * R), rem = id - grp * 8L * R;
    const long width = min(8L, units - grp * 8);
    const long u = grp * 8 + rem % width;
    const int rb = (int)(rem / width);
    const int c = (int)(u % a.num_chunks);
    const int j = (int)((u / a.num_chunks) % a.g);
    const int b = (int)(u / ((long)a.num_chunks * a.g));
    const PosRange ur = unit_range(a, a.seq_lens[b]);
    const int p0 = ur.lo + c * a.chunk_len;
    const int p1 = min(p0 + a.chunk_len, ur.hi);
    if (p0 >= ur.hi && a.num_chunks > 1) {  // past the end: records of weight 0 for the merge
        const int row0 = rb * E::kRowsPerGroup;
        mark_empty_rows(chunk_dst(a, b, j, c, row0), min(a.m - row0, E::kRowsPerGroup), threadIdx.x);
        return;
    }
    E::run(a, sh, b, j, rb, p0, p1, chunk_dst(a, b, j, c));
}

// Paged pools whose unit's rows fit one work-group: the persistent,
// position-balanced grid of kvc_schedule.h (ragged lengths), one segment
// after another per work-group; partial segments go to the work-group's
// record slots for the stream merge.
template <int NQT, int W, int D, int KV8>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(kPrefillWavesPerEu)))
prefill_stream(DecodeArgs a) {
    using E = PrefillEngine<NQT, W, true, D, KV8>;
    __shared__ typename E::Shared sh;
    __shared__ long long cum[kStreamMaxB + 1];
    stream_prefix(a, cum);
    stream_walk(a, cum, [&](int b, int j, int s, int e, bool complete, int slot) {
        const int lo = unit_range(a, a.seq_lens[b]).lo;  // walk offsets are relative to it
        E::run(a, sh, b, j, 0, lo + s, lo + e, complete ? final_dst(a, b, j) : stream_dst(a, slot));
    });
}

template <int NQT, int W, int D, int KV8>
static const void* prefill_pick(bool paged) {
    return paged ? (const void*)prefill_mfma<NQT, W, true, D, KV8> : (const void*)prefill_mfma<NQT, W, false, D, KV8>;
}

template <int D, int KV8>
static const void* prefill_kernel_d(int nqt, int waves, bool paged, bool stream) {
    if (stream) {  // paged pools, one row block per unit
        if (!paged || waves != 4) return nullptr;
        if (nqt == 1) return (const void*)prefill_stream<1, 4, D, KV8>;
        if constexpr (D != 256) {
            if (nqt == 2) return (const void*)prefill_stream<2, 4, D, KV8>;
        }
        return nullptr;
    }
    if (nqt == 1 && waves == 4) return prefill_pick<1, 4, D, KV8>(paged);
    if constexpr (D == 256) {  // 16 rows per wavefront only (64 accumulator registers per query tile)
        if (nqt == 1 && waves == 8) return prefill_pick<1, 8, D, KV8>(paged);
    } else if constexpr (D == 80 || D == 96) {  // four wavefronts only (eight would move 3 pieces per thread)
        if (nqt == 2 && waves == 4) return prefill_pick<2, 4, D, KV8>(paged);
    } else {
        if (nqt == 2 && waves == 4) return prefill_pick<2, 4, D, KV8>(paged);
        if (nqt == 2 && waves == 8) return prefill_pick<2, 8, D, KV8>(paged);
    }
    return nullptr;
}

// Kernel for (rows per wavefront tile count NQT, wavefronts W, layout, grid
// (chunks, or the stream grid of a paged pool), head dimension d, cache kind:
// 0 bf16, 1 FP8 with per-KV-head scales); nullptr when not built.
const void* prefill_kernel(int nqt, int waves, bool paged, bool stream, int d, int kv8) {
    if (kv8 == 0) {
        if (d == 64) return prefill_kernel_d<64, 0>(nqt, waves, paged, stream);
        if (d == 80) return prefill_kernel_d<80, 0>(nqt, waves, paged, stream);
        if (d == 96) return prefill_kernel_d<96, 0>(nqt, waves, paged, stream);
        if (d == 128) return prefill_kernel_d<128, 0>(nqt, waves, paged, stream);
        if (d == 256) return prefill_kernel_d<256, 0>(nqt, waves, paged, stream);
    } else if (kv8 == 1) {
        if (d == 64) return prefill_kernel_d<64, 1>(nqt, waves, paged, stream);
        if (d == 80) return prefill_kernel_d<80, 1>(nqt, waves, paged, stream);
        if (d == 96) return prefill_kernel_d<96, 1>(nqt, waves, paged, stream);
        if (d == 128) return prefill_kernel_d<128, 1>(nqt, waves, paged, stream);
        if (d == 256) return prefill_kernel_d<256, 1>(nqt, waves, paged, stream);
    }
    return nullptr;
}

hipError_t launch_prefill_mfma(const DecodeArgs& a, hipStream_t s) {
    const void* fn = prefill_kernel(a.nqt, a.waves, a.block_table != nullptr, a.stream != 0, a.d,
                                    kv_mode(a));
    if (fn == nullptr || a.row_blocks < 1 || (a.stream && a.row_blocks != 1)) return hipErrorInvalidValue;
    if ((long)a.row_blocks * 16 * a.nqt * a.waves < a.m) return hipErrorInvalidValue;
    const long wgs = a.stream ? (long)a.num_wgs : (long)a.num_chunks * a.g * a.B * a.row_blocks;
    if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    return hipLaunchKernel(fn, dim3((unsigned)wgs), dim3(64 * a.waves), args, 0, s);
}

}  // namespace kvc
