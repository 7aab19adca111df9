// decode_mfma.hip -- bf16 or FP8 caches, head_dim 128, 4 to 32 query rows
// per KV head (more rows run as 32-row slices).
//
// A work-group of W = 4 or 8 wavefronts computes one segment at a time: the
// m query heads j*m..j*m+m-1 (times n new tokens) that share KV head j of
// sequence b
// ("大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com) section 三 3.3)
// over a range of positions, so every K/V byte is read once.  With m >= 4 the
// group's queries times a tile of positions is a real dense product, so both
// products run on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32
// accumulate):
//
//   S^T[16 pos x 16 q] = K_tile[16 pos x 128] . Q^T[128 x 16 q]
//     A operand = K rows straight from HBM: lane l loads 16 bytes of row
//     (l % 16) at dims 32*ks + 8*(l/16); B operand = the group's queries,
//     loaded once per segment; queries >= m are zero columns.
//   O^T[16 dims x 16 q] += V^T[16 dims x 32 pos] . P^T[32 pos x 16 q]
//     the S^T result already sits in the B-operand layout this needs
//     (lane l holds positions 4*(l/16)+v of both 16-position halves), so P
//     never moves between lanes; V^T comes from a per-wavefront LDS copy of
//     the 32 V rows (XOR-swizzled 16-byte chunks).
//   A ninth product with an all-ones A operand gives lr = sum_p bf16(P[p, q]).
//
// Online softmax per query column in base 2 ("KV Cache 优化与注意力机制加速"
// (plumephp.com) section 2.2): the sub-tile maximum is reduced over the four
// row groups of the wavefront; when it passes the running reference m by
// more than 8 (base-2 units) for some column, O and the sums are rescaled by
// 2^(m - m') (otherwise the weights 2^(s - m) stay below 256 and nothing is
// rescaled);
// P is rounded to bf16 for the PV product.  Two sums are kept: lr (the
// rounded P, from the ones product) normalises out = sum bf16(P) V / lr, so
// the weights applied to V add up to one; l (the fp32 P, summed on the VALU)
// gives lse = m + log2 l without the bias the matrix-core sum of the rounded
// weights showed on MI355X (about 1e-3 in lse).
//
// V^T reads use ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3
// read 8 contiguous bytes each of one V row r, and lane i receives element i
// of each of the four rows -- one dim of four positions, the MFMA A layout.
//
// K and V are read with streaming (non-temporal) loads while the next
// 32-position sub-tile is in flight: double-buffered registers for 16 query
// rows, one set reloaded in place for 32 rows and for the 4-wavefront FP8
// kernels with per-head scales and no general features (register budget
// and residency at MfmaEngine and MfmaOccupancy below).  At the end of a segment the W wavefront states go to
// LDS and all threads combine them.
//
// Two entry points share the segment code: a chunked grid (chunk, KV head,
// sequence) and the persistent stream grid of kvc_schedule.h.

#include "kvc_schedule.h"

namespace kvc {

namespace {

constexpr int kD = 128;
// log2 of the largest softmax weight P before the reference maximum moves
constexpr float kLazyRescale = 8.0f;
constexpr int kVRowBytes = kD * 2;                      // 256
constexpr int kVStageBytes = kTileTokens * kVRowBytes;  // 8 KB per wavefront
constexpr int kOStride = kD + 4;                        // padded LDS row (floats)

// Shared memory of a W-wavefront work-group: one V stage per wavefront,
// reused after the walk for the wavefront states (one slot each).
template <int NQT, int W>
struct Lds {
    static constexpr int kSlotFloats = 16 * NQT * kOStride + 3 * 16 * NQT;
    static constexpr int kStageBytes = W * kVStageBytes;
    static constexpr int kMergeBytes = W * kSlotFloats * 4;
    static constexpr int kBytes = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
};

// XOR swizzle of the 16-byte chunk index of V row r.  One transposing read
// of a 16-lane group touches rows R..R+3 (R a multiple of 4) at the same
// 32-byte column slice; the swizzle puts those four slices on disjoint
// groups of eight banks.  It keeps chunk pairs (2k, 2k+1) adjacent.  The
// LDS serves two 16-lane groups together, and rows R..R+3 and R+4..R+7 land
// on the same banks: a two-way conflict, 32 stall cycles per tile (22 % of
// the LDS cycles, about 2 % of the kernel's time).  Layouts without it (the
// group parity in the swizzle, or a padded 4-row pitch) measured no faster
// in the whole-unit kernel and make the 4-wavefront stream kernels spill.
__device__ __forceinline__ int vswz(int r) { return (r & 3) << 1; }

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) { return mfma_bf16(a, b, c); }

// Registers of one wavefront's 32-position tile.  bf16: K rows as MFMA A
// operands (chunk ks: dims 32*ks + 8*G .. +8) and V rows 4u + G, dims
// 8*col .. +8.  FP8: the raw codes, converted to bf16 when the tile is used:
// K dims 64*hh + 16*G .. +16 per half hh (chunk ks = 2*hh + r takes bytes
// 8r .. 8r+7), V as for bf16.
template <bool KV8>
struct TileRegs {
    uint4 k[2][4];
    uint4 v[8];
};
template <>
struct TileRegs<true> {
    uint4 k[2][2];
    uint2 v[8];
};

// GEN: several query tokens per sequence, sliding windows or ring caches
// (per-row visibility masks, ring-aware windows).  Without it a row sees
// every position of its segment, which keeps the common path's registers.
// KV8: 0 = bf16 cache; 1 = FP8 E4M3 codes with a float32 scale per KV
// head: the codes are converted to bf16 exactly and the head's scales are
// folded into the score scale (K) and the output (V); 2 = FP8 codes with a
// scale per (physical block, KV head) of a paged pool: each lane's K scale
// multiplies its scores and its V scale the weights P of its positions
// before they are rounded for the PV product (the normalising sum stays
// that of the unscaled P).
template <int NQT, bool PAGED, int W, bool GEN, int KV8>
struct MfmaEngine {
    using L = Lds<NQT, W>;
    static constexpr bool kF8 = KV8 != 0;
    static constexpr bool kBS = KV8 == 2;  // per-block scales
    static_assert(!kBS || PAGED, "per-block scales need a paged pool");
    // One set of tile registers: with two query tiles (64 accumulator and 32
    // query registers per lane) it lets two wavefronts share a SIMD; in the
    // 4-wavefront FP8 kernels with a scale per KV head and no general
    // features, three (measured faster there: paged 0.617 vs 0.582 of
    // 8 TB/s).  The per-block-scale and general-feature FP8 kernels keep two
    // sets at two wavefronts per SIMD (block scales 0.521 vs 0.502, a
    // 1024-position window over a paged pool 0.408 vs 0.321): with one set
    // the compiler waits for every load in flight before each tile.
    static constexpr bool kSingleBuffer = NQT >= 2 || (KV8 == 1 && W == 4 && !GEN);
    struct Shared {
        uint32_t tbl[PAGED ? kMaxTableSlice : 1];  // per block: row of its first position, head j
        float4 bsc[kBS ? kMaxTableSlice : 1];      // per block: scale*log2e*K scale, V scale, 1 / V scale
        __attribute__((aligned(16))) unsigned char lds[L::kBytes];
    };

    // Query rows row0 .. row0 + 16*NQT - 1 (those below a.m) of KV head j
    // of sequence b over positions [s, e) (possibly empty).  Called by all
    // 64*W threads.
    __device__ static void segment(const DecodeArgs& a, Shared& sh, int b, int j, int s, int e,
                                   const SegDst& dst, int row0 = 0) {
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        const int G = lane >> 4, col = lane & 15;
        const int m = min(a.m - row0, 16 * NQT);  // rows of this slice
        __syncthreads();  // the previous segment is done with the shared memory

        const uint16_t* Q = (const uint16_t*)a.q;

        // B operand of Q K^T: query column 16*qt + col; chunk ks holds dims
        // 32*ks + 8*G .. +8 (bf16) or 64*(ks/2) + 16*G + 8*(ks%2) .. +8 (FP8:
        // the dims of the lane's K bytes).
        uint4 qb[NQT][4];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            const int qi = 16 * qt + col;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int dim0 = KV8 ? 64 * (ks >> 1) + 16 * G + 8 * (ks & 1) : 32 * ks + 8 * G;
                qb[qt][ks] = qi < m ? ld16(Q + (((long)b * a.h + (long)j * a.m + row0 + qi) * kD + dim0))
                                    : make_uint4(0u, 0u, 0u, 0u);
            }
        }

        f32x4_t acc[NQT][8];
        f32x4_t lacc[NQT];  // sum of bf16-rounded P (normalises out)
        float lex[NQT];     // sum of fp32 P over this lane's positions (gives lse)
        // per-block scales: sum over this lane's positions of the weights the
        // PV product applies, bf16(P * v_scale) / v_scale (normalises out)
        float lw[kBS ? NQT : 1];
        float mrun[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            mrun[qt] = kNegInf;
            lex[qt] = 0.0f;
            if constexpr (kBS) lw[qt] = 0.0f;
            lacc[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[qt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

        unsigned char* vst = sh.lds + wave * kVStageBytes;
        const long bj_base = ((long)b * a.g + j) * a.t_cap;
        const float k_sc = KV8 == 1 ? a.k_scale[j] : 1.0f;  // FP8 head scales
        const float v_sc = KV8 == 1 ? a.v_scale[j] : 1.0f;
        const float sl2 = a.scale_log2e * k_sc;
        int blk0 = 0;  // first block of the current window (paged)
        int w0 = s;  // start of the current window
        int w1 = e;  // end of the current window

        // Rows of K/V: paged, the row of position p in the pool (the table
        // slice holds each block's first row for head j; a pool of 2^32 rows
        // exceeds any device); contiguous, p - w0 from the window's first row
        // (kwin / vwin), so that a load is a uniform base plus a 32-bit
        // offset.  A lane reads bytes klane.. of K rows and vlane.. of V rows
        // (plus constant offsets): row_ptr(lane offset, r, constant).
        constexpr int kRowBytes = KV8 ? kD : 2 * kD;
        const char* kwin = (const char*)a.k;
        const char* vwin = (const char*)a.v;
        const uint32_t klane = 16 * G;                 // K chunk of the lane
        const uint32_t vlane = (KV8 ? 8 : 16) * col;  // V chunk of the lane
        auto kv_row = [&](int p) -> uint32_t {
            if (PAGED) return sh.tbl[(p >> a.log2_bs) - blk0] + (uint32_t)(p & (a.block_size - 1));
            return (uint32_t)(p - w0);
        };
        auto row_ptr = [&](const char* base, uint32_t lane_off, uint32_t r, int off) -> const void* {
            if (PAGED) {
                // one shift-and-add for the 64-bit address, kept in the
                // global address space
                using gchar = const __attribute__((address_space(1))) char;
                gchar* g = (gchar*)(((uint64_t)r << (KV8 ? 7 : 8)) + (uint64_t)base);
                return (const char*)(g + (lane_off + off));
            }
            return base + (r * (uint32_t)kRowBytes + lane_off) + off;
        };

        // Query column 16*qt + col is token (row0 + 16*qt + col) % n, which
        // sees positions [lim[qt] - wlen, lim[qt]): p is visible when
        // lim - 1 - p, as unsigned, is below wlen (the window, or 2^31).
        const int raw = a.seq_lens[b];
        const unsigned wlen = GEN && a.window > 0 ? (unsigned)a.window : 0x80000000u;
        int lim[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            lim[qt] = GEN ? visible_len(a, raw, (row0 + 16 * qt + col) % a.n) : 0;

        // A call that appends writes its new tokens (positions raw ..
        // raw+n-1, the last ones of the unit) into their cache slots here,
        // once per unit, and attends to them as last tiles built from
        // k_new / v_new (FP8: from their codes, n = 1).
        const int fresh_lo = max(s, raw);
        const bool has_new = a.k_new != nullptr && fresh_lo < e;
        const int e_cache = has_new ? fresh_lo : e;
        if (has_new) {
            if (KV8) store_new_rows_fp8_d128(a, b, j, raw, fresh_lo, e, tid, 64 * W);
            else store_new_rows_bf16_d128(a, b, j, raw, fresh_lo, e, tid, 64 * W);
        }
        // The new positions [fresh_lo, e) form tiles of 32 (more than one
        // when more than 32 new tokens reach this segment); new tile i goes
        // to wavefront (first + i) % W, first being the wavefront next in
        // turn after the cached tiles.  With one new token (always so
        // without GEN) the single new tile's wavefront loads the token's K
        // and V rows now, one bf16 pair of each per lane, so that the last
        // tile does not wait for them; the tile is then built from those
        // pairs through LDS.
        constexpr bool kNewPair = !GEN;
        const int new_first = ((fresh_lo - s) / kTileTokens) % W;
        bool new_wave;
        int new_i0 = 0;  // this wavefront's first new tile (several new tokens)
        if constexpr (kNewPair) {
            new_wave = has_new && wave == new_first;
        } else {
            const int new_tiles = has_new ? (e - fresh_lo + kTileTokens - 1) / kTileTokens : 0;
            new_i0 = (wave - new_first + W) % W;
            new_wave = new_i0 < new_tiles;
        }
        const uint2 new_pair = kNewPair && new_wave ? new_row_pair_d128(a, b, j, lane) : make_uint2(0u, 0u);
        // scale index of the one new token (FP8 single-token calls)
        const long new_sidx = kBS && kNewPair && has_new ? fp8_scale_index(a, b, j, raw) : (long)j;
        const long bj = (long)b * a.g + j;
        const uint16_t* KN = has_new ? (const uint16_t*)a.k_new + bj * a.n * kD : Q;
        const uint16_t* VN = has_new ? (const uint16_t*)a.v_new + bj * a.n * kD : Q;

        // Loads of the 32-position sub-tile at t0; positions are clamped to
        // the window's last one, so a sub-tile past the end stays in bounds.
        // K/V read once are streamed (non-temporal loads); when the rows are
        // cut into slices that each read the unit's K/V, ordinary loads keep
        // the lines in the caches for the other slices (measured 20 % faster
        // there, 10 % slower for single reads).  Only FP8 pools with
        // per-block scales take slices (other caches run more than 32 rows
        // on the multi-row kernel), so the others keep one load form: a
        // runtime choice puts every load in a branch, after which the
        // compiler waits for all loads in flight before each tile.
        const bool reread = NQT >= 2 && kBS && a.slices > 1;
        auto ld16_kv = [&](const void* p) { return reread ? ld16(p) : ld16_stream(p); };
        auto ld8_kv = [&](const void* p) { return reread ? ld8(p) : ld8_stream(p); };
        auto load_k = [&](int t0, TileRegs<kF8>& tr) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint32_t row = kv_row(min(t0 + 16 * tt + col, w1 - 1));
                if constexpr (KV8) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) tr.k[tt][hh] = ld16_kv(row_ptr(kwin, klane, row, 64 * hh));
                } else {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) tr.k[tt][ks] = ld16_kv(row_ptr(kwin, klane, row, 64 * ks));
                }
            }
        };
        // V rows 4u + G, chunk col: four whole rows per instruction.
        auto load_v = [&](int t0, TileRegs<kF8>& tr) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t row = kv_row(min(t0 + 4 * u + G, w1 - 1));
                if constexpr (KV8) tr.v[u] = ld8_kv(row_ptr(vwin, vlane, row, 0));
                else tr.v[u] = ld16_kv(row_ptr(vwin, vlane, row, 0));
            }
        };
        // K before V, kept in that order (the products consume K first; a
        // wait for K then leaves the V loads in flight).  The bf16
        // general-feature kernels measured faster with the order left to the
        // compiler (8 tokens per sequence: 0.778 vs 0.765 of 8 TB/s at 70B).
        auto load_tile = [&](int t0, TileRegs<kF8>& tr) {
            load_k(t0, tr);
            if constexpr (KV8 || !GEN) __builtin_amdgcn_sched_barrier(0);
            load_v(t0, tr);
        };
        // The appended tokens' tile at t0 (>= raw): position p is row p - raw
        // of the unit's k_new / v_new rows; positions clamp to w1 - 1.  With
        // one new token every position of the tile is that token: its rows
        // (FP8: their codes) go to this wavefront's V staging area first.
        auto load_new_tile = [&](int t0, TileRegs<kF8>& tr) {
            if constexpr (KV8 && kNewPair) {
                new_row_codes_fp8_d128(a, new_sidx, lane, new_pair, vst);
                wave_lds_sync();
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        tr.k[tt][hh] = *reinterpret_cast<const uint4*>(vst + 64 * hh + 16 * G);
#pragma unroll
                for (int u = 0; u < 8; ++u) tr.v[u] = *reinterpret_cast<const uint2*>(vst + 128 + 8 * col);
            } else if constexpr (kNewPair) {
                reinterpret_cast<uint32_t*>(vst)[lane] = new_pair.x;        // K row, 256 bytes
                reinterpret_cast<uint32_t*>(vst + 256)[lane] = new_pair.y;  // V row
                wave_lds_sync();
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        tr.k[tt][ks] = *reinterpret_cast<const uint4*>(vst + 64 * ks + 16 * G);
#pragma unroll
                for (int u = 0; u < 8; ++u) tr.v[u] = *reinterpret_cast<const uint4*>(vst + 256 + 16 * col);
            } else if constexpr (KV8) {
                // several new tokens over an FP8 cache: the wavefront
                // quantises the tile's new rows once (positions t0 ..
                // min(t0 + 32, w1) - 1, rows p - raw of k_new / v_new; items
                // of 8 values spread over its lanes) into its staging area,
                // row i as 128 K codes then 128 V codes, with the quotient
                // and encoder of the cache's append; the tile is then read
                // from there, positions past the last clamped to it.
                const int nrows = min(t0 + kTileTokens, w1) - t0;
                for (int it = lane; it < nrows * 32; it += 64) {
                    const int i = it >> 5, hv = (it >> 4) & 1, ch = it & 15;
                    const long r = (long)(t0 - raw) + i;
                    const long si = kBS ? fp8_scale_index(a, b, j, (int)(raw + r)) : (long)j;
                    const float sc = hv ? a.v_scale[si] : a.k_scale[si];
                    const uint16_t* row = (hv ? VN : KN) + r * kD + 8 * ch;
                    *reinterpret_cast<uint2*>(vst + i * kVRowBytes + hv * kD + 8 * ch) =
                        e4m3_encode8(ld16(row), sc);
                }
                wave_lds_sync();
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int i = min(t0 + 16 * tt + col, w1 - 1) - t0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        tr.k[tt][hh] = *reinterpret_cast<const uint4*>(vst + i * kVRowBytes + 64 * hh + 16 * G);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = min(t0 + 4 * u + G, w1 - 1) - t0;
                    tr.v[u] = *reinterpret_cast<const uint2*>(vst + i * kVRowBytes + kD + 8 * col);
                }
            } else {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const long r = min(t0 + 16 * tt + col, w1 - 1) - raw;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) tr.k[tt][ks] = ld16(KN + r * kD + 32 * ks + 8 * G);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const long r = min(t0 + 4 * u + G, w1 - 1) - raw;
                    tr.v[u] = ld16(VN + r * kD + 8 * col);
                }
            }
        };
        // MFMA A operand of K chunk ks of sub-tile tt.
        auto k_operand = [&](const TileRegs<kF8>& tr, int tt, int ks) -> uint4 {
            if constexpr (KV8) {
                const uint4 c = tr.k[tt][ks >> 1];
                return e4m3x8_to_bf16((ks & 1) ? make_uint2(c.z, c.w) : make_uint2(c.x, c.y));
            } else {
                return tr.k[tt][ks];
            }
        };
        auto v_row = [&](const TileRegs<kF8>& tr, int u) -> uint4 {
            if constexpr (KV8) return e4m3x8_to_bf16(tr.v[u]);
            else return tr.v[u];
        };

        // after_qk runs once the K registers are consumed, after_stage once
        // the V registers are (a single-buffered walk reloads them there).
        auto no_hook = [] {};
        // fresh: a tile of appended tokens (their scales are looked up, not
        // in the table slice)
        auto compute_tile = [&](int t0, const TileRegs<kF8>& tr, auto after_qk, auto after_stage,
                                bool fresh) {
            // per-block scales of the lane's eight positions 16*tt + 4*G + v
            // (a segment may start anywhere, so they may span two blocks)
            float sk[8], vf[8], rvf[8];  // rvf: 1 / vf (hardware reciprocal, shared by the query tiles)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sk[k] = sl2;
                vf[k] = 1.0f;
                rvf[k] = 1.0f;
            }
            if constexpr (kBS) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int p = min(t0 + 16 * (k >> 2) + 4 * G + (k & 3), w1 - 1);
                    if (fresh) {
                        const long si = fp8_scale_index(a, b, j, p);
                        sk[k] = sl2 * a.k_scale[si];
                        vf[k] = a.v_scale[si];
                        rvf[k] = __builtin_amdgcn_rcpf(vf[k]);
                    } else {
                        const float4 e = sh.bsc[(p >> a.log2_bs) - blk0];
                        sk[k] = e.x;
                        vf[k] = e.y;
                        rvf[k] = e.z;
                    }
                }
            }
            f32x4_t S[NQT][2];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) s4 = mfma(k_operand(tr, tt, ks), qb[qt][ks], s4);
                    S[qt][tt] = s4;
                }
            }
            after_qk();
            // Stage V into this wavefront's LDS area.
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 4 * u + G;
                *reinterpret_cast<uint4*>(vst + r * kVRowBytes + ((col ^ vswz(r)) << 4)) = v_row(tr, u);
            }
            after_stage();
            // Online softmax; P as the B operand of the PV product (with
            // per-block scales pbv = P times the V scales; pb stays P).
            uint4 pb[NQT];
            uint4 pbv[kBS ? NQT : 1];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                float sv[8];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int p = t0 + 16 * tt + 4 * G + v;
                        const float x = S[qt][tt][v] * sk[4 * tt + v];
                        const bool vis = GEN ? (p < w1 && (unsigned)(lim[qt] - 1 - p) < wlen) : p < w1;
                        sv[4 * tt + v] = vis ? x : kNegInf;
                    }
                }
                float mt = sv[0];
#pragma unroll
                for (int k = 1; k < 8; ++k) mt = fmaxf(mt, sv[k]);
                mt = fmaxf(mt, shfl_xor_f(mt, 16));
                mt = fmaxf(mt, shfl_xor_f(mt, 32));
                // The reference mrun moves (and the running sums are
                // rescaled) only when some lane's tile maximum passes it by
                // more than kLazyRescale; otherwise P = 2^(s - mrun) stays
                // below 2^kLazyRescale.  out = acc / l and lse = mrun +
                // log2 l do not depend on which reference the sums use.
                if (__any(mt > mrun[qt] + kLazyRescale)) {  // uniform branch
                    const float mnew = fmaxf(mrun[qt], mt);
                    const float r = (mnew == kNegInf) ? 0.0f : mnew;
                    const float alpha = fast_exp2(mrun[qt] - r);  // 0 while nothing was seen
                    mrun[qt] = mnew;
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) acc[qt][nt] *= alpha;
                    lacc[qt] *= alpha;
                    lex[qt] *= alpha;
                    if constexpr (kBS) lw[qt] *= alpha;
                }
                const float ref = (mrun[qt] == kNegInf) ? 0.0f : mrun[qt];
                float pv[8];
                float psum = 0.0f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    pv[k] = fast_exp2(sv[k] - ref);
                    psum += pv[k];
                }
                lex[qt] += psum;
                pb[qt] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                    pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
                if constexpr (kBS) {
                    pbv[qt] = make_uint4(pack_bf16x2(pv[0] * vf[0], pv[1] * vf[1]),
                                         pack_bf16x2(pv[2] * vf[2], pv[3] * vf[3]),
                                         pack_bf16x2(pv[4] * vf[4], pv[5] * vf[5]),
                                         pack_bf16x2(pv[6] * vf[6], pv[7] * vf[7]));
                    const uint4 w = pbv[qt];
                    lw[qt] += bf16_lo(w.x) * rvf[0] + bf16_hi(w.x) * rvf[1] + bf16_lo(w.y) * rvf[2] +
                              bf16_hi(w.y) * rvf[3] + bf16_lo(w.z) * rvf[4] + bf16_hi(w.z) * rvf[5] +
                              bf16_lo(w.w) * rvf[6] + bf16_hi(w.w) * rvf[7];
                }
            }

            wave_lds_sync();

            // PV: A operand = V^T rows (dims 16*nt + col) x positions
            // {4G + r} U {16 + 4G + r}, r = 0..3.  Lane 16G + 4r + qd reads 8
            // bytes of V row (16h + 4G + r) at dims 16*nt + 4*qd; the
            // transposing read hands lane 16G + i dim 16*nt + i of those rows.
            const int tr_r = (lane >> 2) & 3, tr_q = lane & 3;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int ch = 2 * nt + (tr_q >> 1);
                const int sub = (tr_q & 1) * 8;
                const int r0 = 4 * G + tr_r, r1 = 16 + 4 * G + tr_r;
                const uint2 lo = lds_read_tr16(vst + r0 * kVRowBytes + ((ch ^ vswz(r0)) << 4) + sub);
                const uint2 hi = lds_read_tr16(vst + r1 * kVRowBytes + ((ch ^ vswz(r1)) << 4) + sub);
                const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    if constexpr (kBS) acc[qt][nt] = mfma(av, pbv[qt], acc[qt][nt]);
                    else acc[qt][nt] = mfma(av, pb[qt], acc[qt][nt]);
                }
            }
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                if constexpr (!kBS) lacc[qt] = mfma(ones, pb[qt], lacc[qt]);  // (per-block: lw)

            wave_lds_sync();
        };

        // Windows of at most kMaxChunk positions, so that a window's slice of
        // the block table fits in shared memory.
        for (w0 = s; w0 < e_cache; w0 = w1) {
            w1 = min(e_cache, w0 + kMaxChunk);
            if (!PAGED) {
                long first = bj_base + w0;  // row of position w0
                if (GEN && a.ring) {
                    // a window never wraps around the ring: slot = p - wbase in it
                    const int wbase = w0 - w0 % a.t_cap;
                    w1 = min(w1, wbase + a.t_cap);
                    first -= wbase;
                }
                kwin = (const char*)a.k + first * kRowBytes;
                vwin = (const char*)a.v + first * kRowBytes;
            } else {
                blk0 = w0 >> a.log2_bs;
                const int nblk = ((w1 - 1) >> a.log2_bs) - blk0 + 1;
                for (int t = tid; t < nblk; t += 64 * W) {
                    int ph = a.block_table[(long)b * a.max_blocks + blk0 + t];
                    ph = ph < 0 ? 0 : (ph >= a.num_blocks ? a.num_blocks - 1 : ph);
                    sh.tbl[t] = ((uint32_t)ph * (uint32_t)a.g + (uint32_t)j) * (uint32_t)a.block_size;
                    if constexpr (kBS) {
                        const float vs_ = a.v_scale[(long)ph * a.g + j];
                        sh.bsc[t] = make_float4(a.scale_log2e * a.k_scale[(long)ph * a.g + j], vs_,
                                                __builtin_amdgcn_rcpf(vs_), 0.0f);
                    }
                }
                __syncthreads();
            }
            // A wavefront takes kStep positions per step while the next
            // step's loads are in flight.  FP8 tiles hold half the bytes: in
            // the 8-wavefront kernels (one work-group per unit) a wavefront
            // loads two 32-position tiles per step, which keeps as many bytes
            // in flight as with bf16 (measured faster there; slower with 4
            // wavefronts).
            constexpr bool kPair = KV8 && W >= 8 && !kSingleBuffer;
            constexpr int kStep = kPair ? 2 * kTileTokens : kTileTokens;
            const int stride = W * kStep;
            int t0 = w0 + wave * kStep;
            if constexpr (kSingleBuffer) {
                // One set of tile registers: the next tile's K is loaded as
                // soon as the product has consumed this tile's K, its V once
                // this tile's V is staged; the schedule barriers keep the
                // compiler from hoisting the loads (which would need a
                // second set of registers).  The first tile's loads keep the
                // same order, K then V (load_tile): issued the other way
                // round, the loop's first product would wait for them all,
                // and the compiler then waits for every load in flight at the
                // top of every step.
                TileRegs<kF8> tr;
                load_tile(t0, tr);
                for (; t0 < w1; t0 += stride) {
                    const int tn = t0 + stride;
                    compute_tile(t0, tr,
                                 [&] { __builtin_amdgcn_sched_barrier(0); load_k(tn, tr); __builtin_amdgcn_sched_barrier(0); },
                                 [&] { __builtin_amdgcn_sched_barrier(0); load_v(tn, tr); __builtin_amdgcn_sched_barrier(0); },
                                 false);
                }
            } else if constexpr (kPair) {
                TileRegs<kF8> a0, a1, b0, b1;
                load_tile(t0, a0);
                load_tile(t0 + kTileTokens, a1);
                for (;;) {
                    if (t0 >= w1) break;
                    load_tile(t0 + stride, b0);
                    load_tile(t0 + stride + kTileTokens, b1);
                    compute_tile(t0, a0, no_hook, no_hook, false);
                    if (t0 + kTileTokens < w1) compute_tile(t0 + kTileTokens, a1, no_hook, no_hook, false);
                    t0 += stride;
                    if (t0 >= w1) break;
                    load_tile(t0 + stride, a0);
                    load_tile(t0 + stride + kTileTokens, a1);
                    compute_tile(t0, b0, no_hook, no_hook, false);
                    if (t0 + kTileTokens < w1) compute_tile(t0 + kTileTokens, b1, no_hook, no_hook, false);
                    t0 += stride;
                }
            } else {
                TileRegs<kF8> tA, tB;
                load_tile(t0, tA);
                for (;;) {
                    if (t0 >= w1) break;
                    load_tile(t0 + stride, tB);
                    compute_tile(t0, tA, no_hook, no_hook, false);
                    t0 += stride;
                    if (t0 >= w1) break;
                    load_tile(t0 + stride, tA);
                    compute_tile(t0, tB, no_hook, no_hook, false);
                    t0 += stride;
                }
            }
            if (PAGED) __syncthreads();  // the next window rewrites the table slice
        }
        // The appended tokens (the last positions of the unit) are taken
        // last, tile i by wavefront (first + i) % W.
        if (new_wave) {
            w1 = e;
            if constexpr (kNewPair) {  // one new token: one tile
                TileRegs<kF8> tr;
                load_new_tile(fresh_lo, tr);
                compute_tile(fresh_lo, tr, no_hook, no_hook, true);
            } else {
                for (int t = fresh_lo + kTileTokens * new_i0; t < e; t += kTileTokens * W) {
                    TileRegs<kF8> tr;
                    load_new_tile(t, tr);
                    compute_tile(t, tr, no_hook, no_hook, true);
                }
            }
        }

        // lex holds this lane's positions only: sum the four row groups.
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            lex[qt] += shfl_xor_f(lex[qt], 16);
            lex[qt] += shfl_xor_f(lex[qt], 32);
            if constexpr (kBS) {
                lw[qt] += shfl_xor_f(lw[qt], 16);
                lw[qt] += shfl_xor_f(lw[qt], 32);
            }
        }

        // ---- every wavefront stores its state; then all threads combine
        // the W states of (query row, 4 dims) items and write them ----
        float* slots = reinterpret_cast<float*>(sh.lds);
        __syncthreads();  // every wavefront is done with its V staging area
        {
            float* slot = slots + wave * L::kSlotFloats;
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int qi = 16 * qt + col;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
                    *reinterpret_cast<f32x4_t*>(slot + qi * kOStride + 16 * nt + 4 * G) = acc[qt][nt];
                if (G == 0) {
                    slot[16 * NQT * kOStride + qi] = mrun[qt];
                    if constexpr (kBS) slot[16 * NQT * kOStride + 16 * NQT + qi] = lw[qt];
                    else slot[16 * NQT * kOStride + 16 * NQT + qi] = lacc[qt][0];
                    slot[16 * NQT * kOStride + 32 * NQT + qi] = lex[qt];
                }
            }
        }
        __syncthreads();
        constexpr int kQuads = kD / 4;
        for (int it = tid; it < m * kQuads; it += 64 * W) {
            const int qi = it / kQuads, d4 = it - qi * kQuads;
            float mx = kNegInf;
#pragma unroll
            for (int w = 0; w < W; ++w) mx = fmaxf(mx, slots[w * L::kSlotFloats + 16 * NQT * kOStride + qi]);
            const float ref = (mx == kNegInf) ? 0.0f : mx;
            float lr = 0.0f, l = 0.0f;
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float* slot = slots + w * L::kSlotFloats;
                const float f = fast_exp2(slot[16 * NQT * kOStride + qi] - ref);  // 0 for empty states
                lr += slot[16 * NQT * kOStride + 16 * NQT + qi] * f;
                l += slot[16 * NQT * kOStride + 32 * NQT + qi] * f;
                o += *reinterpret_cast<const f32x4_t*>(slot + qi * kOStride + 4 * d4) * f;
            }
            // out = sum of bf16(P) V / the sum of the same bf16(P); lse from
            // the fp32 sum; FP8: times the V head scale
            const float inv = lr > 0.0f ? v_sc / lr : 0.0f;
            *reinterpret_cast<f32x4_t*>(dst.o + (long)qi * dst.o_stride + 4 * d4) = o * inv;
            if (d4 == 0) {
                float v;
                if (dst.final_) v = l > 0.0f ? (mx + fast_log2(l)) * kLn2 : kNegInf;
                else v = l > 0.0f ? mx + fast_log2(l) : kNegInf;
                dst.lse[(long)qi * dst.lse_stride] = v;
            }
        }
    }
};

}  // namespace

// Resident wavefronts per SIMD the register allocator is asked to allow: two
// (256 registers; it fits them without spills: the 16-query variants with
// two sets of tile registers, the 32-query variant with one), three for the
// single-buffered 4-wavefront FP8 variant with per-head scales and no
// general features (168 registers; measured about 5 % faster on paged
// caches than two).
template <int NQT, int W, bool GEN, int KV8>
struct MfmaOccupancy { static constexpr int kWavesPerEu = (KV8 == 1 && W == 4 && NQT == 1 && !GEN) ? 3 : 2; };

template <int NQT, bool PAGED, int W, bool GEN, int KV8>
__global__ void __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(MfmaOccupancy<NQT, W, GEN, KV8>::kWavesPerEu)))
decode_mfma_chunked(DecodeArgs a) {
    using E = MfmaEngine<NQT, PAGED, W, GEN, KV8>;
    __shared__ typename E::Shared sh;
    int c = blockIdx.x, b = blockIdx.z;
    int j = blockIdx.y / a.slices, row0 = (blockIdx.y - j * a.slices) * 16 * NQT;
    if (a.slices > 1) {
        // The slices of one (chunk, KV head, sequence) read the same K/V.
        // Work-group ids go to the eight XCDs in turn, so the slices get ids
        // eight apart: they run on one XCD at about the same time and the
        // later reads find the lines in that XCD's L2.  Units go in groups
        // of eight (the last group may be narrower); within a group, slice
        // s of unit k has id s * width + k.
        const long L = blockIdx.x + (long)gridDim.x * (blockIdx.y + (long)gridDim.y * blockIdx.z);
        const long units = (long)a.num_chunks * a.g * a.B;
        const long grp = L / (8L * a.slices), rem = L - grp * 8L * a.slices;
        const long width = min(8L, units - grp * 8);
        const long u = grp * 8 + rem % width;
        row0 = (int)(rem / width) * 16 * NQT;
        c = (int)(u % a.num_chunks);
        j = (int)((u / a.num_chunks) % a.g);
        b = (int)(u / ((long)a.num_chunks * a.g));
    }
    // chunks cover [lo, hi); without the general features lo = 0
    const PosRange ur = GEN ? unit_range(a, a.seq_lens[b])
                            : PosRange{0, attended_len(a, a.seq_lens[b])};
    const int p0 = ur.lo + c * a.chunk_len;
    const int p1 = min(p0 + a.chunk_len, ur.hi);
    const bool single = a.num_chunks == 1;
    if (p0 >= ur.hi && !single) {  // past the end: a record of weight 0 for the merge
        mark_empty_rows(chunk_dst(a, b, j, c, row0), min(a.m - row0, 16 * NQT), threadIdx.x);
        return;
    }
    E::segment(a, sh, b, j, p0, p1, chunk_dst(a, b, j, c, row0), row0);
}

template <int NQT, bool PAGED, int W, bool GEN, int KV8>
__global__ void __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(MfmaOccupancy<NQT, W, GEN, KV8>::kWavesPerEu)))
decode_mfma_stream(DecodeArgs a) {
    using E = MfmaEngine<NQT, PAGED, W, GEN, KV8>;
    __shared__ typename E::Shared sh;
    __shared__ long long cum[kStreamMaxB + 1];
    stream_prefix(a, cum);
    stream_walk(a, cum, [&](int b, int j, int s, int e, bool complete, int slot) {
        const int lo = GEN ? unit_range(a, a.seq_lens[b]).lo : 0;  // walk offsets are relative to it
        E::segment(a, sh, b, j, lo + s, lo + e, complete ? final_dst(a, b, j) : stream_dst(a, slot));
    });
}

template <int NQT, bool PG, int WV, int KV>
static const void* mfma_pick_kv(bool stream, bool gen) {
    if (stream)
        return gen ? (const void*)decode_mfma_stream<NQT, PG, WV, true, KV>
                   : (const void*)decode_mfma_stream<NQT, PG, WV, false, KV>;
    return gen ? (const void*)decode_mfma_chunked<NQT, PG, WV, true, KV>
               : (const void*)decode_mfma_chunked<NQT, PG, WV, false, KV>;
}

// 8-wavefront kernels: chunked grids of contiguous caches only.
template <int NQT, int WV, int KV>
static const void* mfma_chunked_kv(bool gen) {
    return gen ? (const void*)decode_mfma_chunked<NQT, false, WV, true, KV>
               : (const void*)decode_mfma_chunked<NQT, false, WV, false, KV>;
}

template <int NQT, bool PG, int WV>
static const void* mfma_pick(bool stream, bool gen, int kv8) {
    if (kv8 == 2) {  // per-block scales: paged pools only; chunks only with two query tiles
        if constexpr (PG && NQT == 2) {
            if (stream) return nullptr;
            return gen ? (const void*)decode_mfma_chunked<NQT, PG, WV, true, 2>
                       : (const void*)decode_mfma_chunked<NQT, PG, WV, false, 2>;
        } else if constexpr (PG) {
            return mfma_pick_kv<NQT, PG, WV, 2>(stream, gen);
        } else {
            return nullptr;
        }
    }
    return kv8 ? mfma_pick_kv<NQT, PG, WV, 1>(stream, gen) : mfma_pick_kv<NQT, PG, WV, 0>(stream, gen);
}

// Kernel function for (m, layout, split mode, wavefronts per work-group,
// general features, cache kind: 0 bf16, 1 FP8 with per-head scales, 2 FP8
// with per-block scales); nullptr when that combination is not built.
// Every (m, layout, mode) has a 4-wavefront kernel; a contiguous cache also
// has 8-wavefront chunked kernels, for whole-unit work-groups and for chunk
// grids smaller than the device's slots.
const void* mfma_kernel(int m, bool paged, bool stream, int waves, bool gen, int kv8) {
    const bool two = m > 16;
    if (waves == 4) {
        if (two) return paged ? mfma_pick<2, true, 4>(stream, gen, kv8) : mfma_pick<2, false, 4>(stream, gen, kv8);
        return paged ? mfma_pick<1, true, 4>(stream, gen, kv8) : mfma_pick<1, false, 4>(stream, gen, kv8);
    }
    if (waves == 8 && !paged && !stream && kv8 != 2) {
        if (two) return kv8 ? mfma_chunked_kv<2, 8, 1>(gen) : mfma_chunked_kv<2, 8, 0>(gen);
        return kv8 ? mfma_chunked_kv<1, 8, 1>(gen) : mfma_chunked_kv<1, 8, 0>(gen);
    }
    return nullptr;
}

hipError_t launch_decode_mfma_bf16_d128(const DecodeArgs& a, hipStream_t s) {
    // more than 32 rows: slices of 32 (chunked mode only)
    if (a.slices < 1 || (a.m > 32 * a.slices) || (a.slices > 1 && (a.stream || a.m <= 32)))
        return hipErrorInvalidValue;
    const void* fn = mfma_kernel(min(a.m, 32), a.block_table != nullptr, a.stream != 0, a.waves,
                                 general_features(a), kv_mode(a));
    if (fn == nullptr) return hipErrorInvalidValue;
    const dim3 grid = a.stream ? dim3((unsigned)a.num_wgs)
                               : dim3((unsigned)a.num_chunks, (unsigned)(a.g * a.slices),
                                      (unsigned)a.B);
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    return hipLaunchKernel(fn, grid, dim3(64 * a.waves), args, 0, s);
}

}  // namespace kvc
