// kvc_api.hip -- the C ABI of libkvc (declared in include/kvc.h): argument
// validation, work-split planning and kernel selection.  Validation runs
// before any HIP call; every launch goes to the caller's stream.
#include "kvc.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "kvc_internal.h"

namespace kvc {

static long ceil_div(long a, long b) { return (a + b - 1) / b; }

Plan make_plan(int B, int g, int max_seq_len, int num_splits) {
    if (max_seq_len <= 0) return Plan{kTileTokens, 1};
    long C;
    if (num_splits > 0) {
        C = num_splits;
    } else {
        const long units = (long)B * g;
        C = ceil_div(kTargetWorkgroups, units > 0 ? units : 1);
        const long by_len = ceil_div(max_seq_len, kMinAutoChunk);
        if (C > by_len) C = by_len;
        if (C < 1) C = 1;
    }
    long chunk = ceil_div(max_seq_len, C);
    chunk = ceil_div(chunk, kTileTokens) * kTileTokens;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    if (chunk < kTileTokens) chunk = kTileTokens;
    return Plan{(int)chunk, (int)ceil_div(max_seq_len, chunk)};
}

// kv8: the cache kind (kv_mode): 0 bf16, 1 FP8 with a scale per KV head,
// 2 FP8 with a scale per (block, KV head).  bf16 or FP8 caches with head_dim
// 128: up to 3 rows per KV head on the vector ALUs, 4..32 on the matrix-core
// decode kernel, more on the multi-row kernel (per-block FP8 scales: as
// 32-row slices of the decode kernel).  bf16 caches and FP8 caches with
// per-head scales with head_dim 64, 80, 96 or 256: every row count on the
// multi-row kernel (one K/V read per KV head).  Everything else (fp32,
// other head dims, per-block FP8 scales with d != 128) takes the generic
// kernel.
KernelKind choose_kernel(int dtype, int d, int m, int kv8) {
    if (dtype == KVC_BF16 && d == 128) return m <= 3 ? kValu : (m <= 32 || kv8 == 2 ? kMfma : kPrefill);
    if (dtype == KVC_BF16 && kv8 != 2 && (d == 64 || d == 80 || d == 96 || d == 256)) return kPrefill;
    return kGeneric;
}

// Work-groups per unit that split its query rows on the decode kernel: it
// holds at most 32 rows, so more rows (FP8 caches only) take slices of 32,
// each reading the unit's K/V.
static int row_slices(KernelKind kind, int m) { return (kind == kMfma && m > 32) ? (m + 31) / 32 : 1; }

// Shape of the multi-row kernel for m rows per KV head: 16-row query tiles
// per wavefront, wavefronts per work-group, work-groups per unit.  Up to 64
// rows (HBM-bound: a few rows per K/V byte) 16 rows per wavefront and four
// wavefronts; up to 128, 32 rows per wavefront; beyond (bound by the matrix
// cores) 256 rows per work-group of eight wavefronts, so that each K/V tile
// staged in LDS serves 256 rows.  Head dimension 256 keeps 16 rows per
// wavefront (its accumulators take 64 registers per query tile): 128 rows
// per eight-wavefront work-group beyond 64.  Head dimensions 80 and 96 keep
// four wavefronts (eight would split a step's pieces unevenly): 128 rows
// per work-group beyond 64.
struct PrefillShape {
    int nqt, waves, row_blocks;
};
static PrefillShape prefill_shape(int m, int d) {
    if (m <= 64) return {1, 4, 1};
    if (d == 256) return {1, 8, (m + 127) / 128};
    if (d == 80 || d == 96) return {2, 4, (m + 127) / 128};  // four-wavefront work-groups only
    if (m <= 128) return {2, 4, 1};
    return {2, 8, (m + 255) / 256};
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A decode launch: the kernel family and how positions are split.
//   stream       persistent position-balanced grid (paged caches, or asked for)
//   auto_chunks  contiguous cache, automatic: as many chunks per (sequence, KV
//                head) as fill the resident work-group slots once; the count
//                is fixed at launch from the device (workspace sized for the
//                largest possible count)
//   otherwise    chunks from num_splits (or the generic kernel's heuristic)
struct Schedule {
    KernelKind kind;
    bool stream;
    bool auto_chunks;
    Plan plan;
};

// Largest automatic chunk over a paged pool (whose lengths are ragged) when
// it takes chunks: measured over the 64-sequence pool of 128-8192 positions
// with FP8 codes and 2 or 4 new tokens per sequence, 3 chunks of 2 688
// positions took 124 and 137 us per call against 146 and 151 us for 2 of
// 4 032 (per-block scales, 8 tokens: 189 against 206 us).
constexpr long kPagedChunk = 2816;

static long clamp_chunks(long C, int max_seq_len) {
    const long lo = ceil_div(max_seq_len, kMaxChunk);
    const long hi = ceil_div(max_seq_len, kTileTokens);
    if (C < lo) C = lo;
    if (C > hi) C = hi;
    return C < 1 ? 1 : C;
}

static Plan plan_for_chunks(int max_seq_len, long C) {
    if (max_seq_len <= 0) return Plan{kTileTokens, 1};
    long chunk = ceil_div(ceil_div(max_seq_len, C), kTileTokens) * kTileTokens;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    return Plan{(int)chunk, (int)ceil_div(max_seq_len, chunk)};
}

// Chunks per (sequence, KV head) that fill `slots` work-group slots once.
static long chunks_for_slots(long slots, int B, int g, int max_seq_len) {
    const long units = (long)B * g;
    return clamp_chunks(ceil_div(slots, units > 0 ? units : 1), max_seq_len);
}

// prefer_chunks: the call's position ranges suit chunks better than the
// stream grid even on a paged pool (sliding windows: ranges of at most
// W + n - 1 positions, nearly equal; FP8 caches with several new tokens per
// sequence: measured faster chunked).
static Schedule make_schedule(int B, int h, int g, int d, int dtype, int max_seq_len,
                              int num_splits, bool paged, bool prefer_chunks = false, int kv8 = 0) {
    Schedule sc;
    sc.kind = choose_kernel(dtype, d, h / g, kv8);
    // Stream mode keeps global positions in 64-bit products p * total with
    // p <= 1024: it is used only while B * g * max_seq_len < 2^40.
    const bool small_enough = (long double)B * g * max_seq_len < (long double)(1LL << 40);
    const int slices = row_slices(sc.kind, h / g);
    // the multi-row kernel streams over paged pools when a unit's rows fit
    // one 4-wavefront work-group
    const PrefillShape ps = prefill_shape(h / g, d);
    const bool prefill_streams = sc.kind == kPrefill && paged && ps.row_blocks == 1 && ps.waves == 4;
    // FP8 caches with per-block scales and two query tiles have no stream
    // kernel: its registers (tile scales on top of two query tiles) left one
    // wavefront per SIMD, half the grid the occupancy query sized it for.
    const bool fp8_two_tiles = kv8 != 0 && sc.kind == kMfma && h / g > 16;
    const bool can_stream = (sc.kind == kValu || sc.kind == kMfma || prefill_streams) && slices == 1 &&
                            B <= kStreamMaxB && small_enough && !(fp8_two_tiles && kv8 == 2);
    // automatic: paged caches stream (lengths vary) unless prefer_chunks.  The
    // multi-row kernel's walk pays a prologue per segment (query tiles, table
    // window, first step in flight): measured, it beats whole units over
    // ragged lengths only with bf16 rows of 256 dims and at most 16 rows per
    // KV head; elsewhere it streams only when asked to.  FP8 caches with two
    // query tiles (17-32 rows per KV head) on the decode kernel also chunk:
    // over the 64-sequence paged pool with 8 tokens per sequence, 3 chunks
    // per unit took 164 us (per-head scales) and 189 us (per-block scales)
    // against 241 us and 388 us streamed (the per-block-scale stream kernel
    // has since been dropped, above).
    const bool auto_stream = (sc.kind != kPrefill && !fp8_two_tiles) ||
                             (sc.kind == kPrefill && kv8 == 0 && d == 256 && h / g <= 16);
    sc.stream = can_stream && (num_splits == KVC_SPLITS_STREAM ||
                               (num_splits == 0 && paged && !prefer_chunks && auto_stream));
    sc.auto_chunks = !sc.stream && num_splits <= 0 && sc.kind != kGeneric;
    if (sc.auto_chunks) {
        // workspace bound: every slot of a 256-CU device, 4 work-groups
        // each (twice that chunk count for the VALU kernel, which may take
        // two rounds); plan_for_chunks grows with the count asked for
        long bound = chunks_for_slots((long)kStreamMaxCUs * kStreamMaxWgPerCu, B * slices, g, max_seq_len);
        if (sc.kind == kValu) bound = clamp_chunks(2 * bound, max_seq_len);
        if (paged) bound = clamp_chunks(std::max(bound, ceil_div(max_seq_len, kPagedChunk)), max_seq_len);
        sc.plan = plan_for_chunks(max_seq_len, bound);
    } else {
        sc.plan = make_plan(B, g, max_seq_len, num_splits > 0 ? num_splits : 0);
    }
    return sc;
}

// Workspace layout: partial O rows | partial lse rows.
static size_t workspace_rows(int B, int h, int g, const Schedule& sc) {
    if (sc.stream) return (size_t)kStreamMaxCUs * kStreamMaxWgPerCu * 2 * (size_t)(h / g);
    return sc.plan.num_chunks <= 1 ? 0 : (size_t)B * h * sc.plan.num_chunks;
}

static size_t workspace_for(int B, int h, int g, int d, const Schedule& sc) {
    const size_t rows = workspace_rows(B, h, g, sc);
    if (rows == 0) return 0;
    return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

// Workspace a call needs, the largest over the schedules one size query
// stands for: for automatic splits of a paged cache, both schedules it may
// take (stream, or chunks when the call prefers them), so that one query
// serves every call; and bf16 and FP8 caches alike (FP8 calls take q
// in bf16 and size with KVC_BF16 or KVC_FP8_E4M3), whose kernels may differ
// (bf16 head dims 64 and 256 run the multi-row kernel, FP8 ones the generic
// kernel, whose plans take more chunks).
static size_t required_workspace(int B, int h, int g, int d, int dtype, int max_len,
                                 int num_splits, bool paged) {
    size_t need = 0;
    for (int f8 = 0; f8 < (dtype == KVC_BF16 ? 3 : 1); ++f8) {
        for (int win = 0; win < (paged && num_splits == 0 ? 2 : 1); ++win) {
            const size_t w = workspace_for(
                B, h, g, d, make_schedule(B, h, g, d, dtype, max_len, num_splits, paged, win != 0, f8));
            if (w > need) need = w;
        }
    }
    return need;
}

// Compute units of the current device (cached per device).
// The per-process caches below may be filled from several host threads at
// once; one lock guards them (held only for a lookup or one HIP query).
static std::mutex g_cache_lock;

static int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kStreamMaxCUs;
    std::lock_guard<std::mutex> lock(g_cache_lock);
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = kStreamMaxCUs;
    if (dev < 64) cached[dev] = n;
    return n;
}

// Resident work-groups per compute unit for a kernel launched with `threads`
// threads per work-group (cached).
static int resident_wgs(const void* fn, int threads) {
    struct Entry { const void* fn; int n; };
    static Entry cache[64] = {};
    std::lock_guard<std::mutex> lock(g_cache_lock);
    for (auto& e : cache)
        if (e.fn == fn) return e.n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess || n < 0) n = 0;
    for (auto& e : cache)
        if (e.fn == nullptr) {
            e.fn = fn;
            e.n = n;
            break;
        }
    return n;
}

// Work-group slots of the current device for a kernel of `waves` wavefronts
// per work-group: CUs x resident work-groups, capped at 256 CUs x 4 (the
// workspace bound).  0 when the kernel cannot be resident at all.
static long device_slots(const void* fn, int waves) {
    int per_cu = resident_wgs(fn, 64 * waves);
    if (per_cu > kStreamMaxWgPerCu) per_cu = kStreamMaxWgPerCu;
    int cus = device_cus();
    if (cus > kStreamMaxCUs) cus = kStreamMaxCUs;
    return (long)cus * per_cu;
}

// kv8: the cache kind (kv_mode): 0 bf16, 1 FP8 per-head scales, 2 per-block
static const void* kernel_for(KernelKind kind, int m, bool paged, bool stream, int waves, bool gen,
                              int kv8) {
    return kind == kMfma ? mfma_kernel(m, paged, stream, waves, gen, kv8)
                         : valu_kernel(m, paged, stream, waves, gen, kv8);
}

// Fraction of the slot-rounds a grid of `wgs` equal work-groups keeps busy.
static double fill(long wgs, long slots) {
    const long rounds = ceil_div(wgs, slots);
    return (double)wgs / (double)(rounds * slots);
}

// Automatic chunking of a contiguous cache.  Two shapes compete:
//   whole units  one 8-wavefront work-group per (sequence, KV head), no
//                partial results and no merge pass;
//   chunks       4-wavefront work-groups, several chunks per unit, merged
//                afterwards.
// The matrix-core kernels with one query tile and one token per sequence
// (m <= 16): chunks of about kChunkTarget positions, at least one
// work-group per CU, and two per unit when each gets at least
// kMinSplitChunk positions; whole units on 8 wavefronts when they fill the
// device's slots (>= 7/8 of slot-rounds busy) and either stay one chunk or
// are bf16 with at least 512 positions per wavefront.  Measured over
// batches of 4 to 64 sequences of 1024 to 8192 positions (64 or 32 query
// heads, 8 KV heads): shorter chunks add partial results and merge work,
// longer ones, or filling every slot once, leave CUs to a tail of long
// work-groups (FP8 caches at 32 sequences of 4096 positions: 0.692 of
// 8 TB/s with two chunks per unit against 0.678 for whole units on 8
// wavefronts; bf16 at 8 sequences of 4096 positions: 0.602 with 4 chunks
// against 0.550 with the 8 that fill the slots).  Other kernels: whole
// units win when they keep at least as many tiles in flight per CU
// (resident wavefronts, counted twice for the 8-wavefront FP8 kernel, which
// loads two tiles per step) and the grid fills the slots nearly as well;
// chunks fill the slots once.
constexpr long kChunkTarget = 2560;
constexpr long kMinSplitChunk = 1024;

struct AutoShape {
    int waves;
    long chunks;
};

static AutoShape auto_shape(KernelKind kind, int m, int B, int g, int max_len, bool paged,
                            bool gen, int kv8) {
    const long units = (long)B * g;
    if (kind == kMfma && m <= 16 && !gen) {
        long C = ceil_div(max_len, kChunkTarget);
        const long per_cu = ceil_div(device_cus(), units > 0 ? units : 1);
        if (C < per_cu) C = per_cu;
        if (C < 2 && max_len >= 2 * kMinSplitChunk) C = 2;
        // within the workspace bound of automatic plans
        const long bound = chunks_for_slots((long)kStreamMaxCUs * kStreamMaxWgPerCu, B, g, max_len);
        if (C > bound) C = bound;
        C = clamp_chunks(C, max_len);
        const void* f8 = kernel_for(kind, m, paged, false, 8, gen, kv8);
        const long slots8 = f8 != nullptr ? device_slots(f8, 8) : 0;
        const bool wide = slots8 > 0 && units >= slots8 && fill(units, slots8) * 8.0 >= 7.0;
        if (wide && (C == 1 || (kv8 == 0 && max_len >= 8 * 512))) return AutoShape{8, 1};
        return AutoShape{4, C};
    }
    const void* f4 = kernel_for(kind, m, paged, false, 4, gen, kv8);
    const long slots4 = device_slots(f4, 4);
    AutoShape split{4, chunks_for_slots(slots4 > 0 ? slots4 : 1, B, g, max_len)};
    // A paged pool's lengths are ragged: chunks of at most kPagedChunk
    // positions, so that the long sequences' work spreads over more
    // work-groups.
    if (paged) split.chunks = clamp_chunks(std::max(split.chunks, ceil_div(max_len, kPagedChunk)), max_len);
    // bf16 VALU work-groups that fill the slots in one round with 2-8
    // chunks per unit: twice the chunks, two rounds.  The first work-group
    // dispatched to a CU runs ahead of the others there; with a second
    // round the dispatcher refills its slot instead of leaving the CU to its
    // last work-group (measured: 7B MHA 0.710 vs 0.695 of 8 TB/s at 6 vs 3
    // chunks; one chunk per unit doubled would add a merge, long contexts
    // with many chunks got slower, and the FP8 kernel, four work-groups per
    // CU, 0.549 vs 0.575 at 8 vs 4 chunks).
    if (kind == kValu && kv8 == 0 && split.chunks >= 2 && split.chunks <= 8)
        split.chunks = clamp_chunks(2 * split.chunks, max_len);
    const int wv = 8;
    const void* fn = kernel_for(kind, m, paged, false, wv, gen, kv8);
    const long slots = fn != nullptr ? device_slots(fn, wv) : 0;
    // resident tiles in flight: the 8-wavefront FP8 kernel loads two per step
    const long inflight = slots * wv * (kind == kMfma && kv8 != 0 ? 2 : 1);
    if (slots > 0 && units >= slots && inflight >= slots4 * 4 && fill(units, slots) * 8.0 >= 7.0)
        return AutoShape{wv, 1};
    return split;
}

// Alignment the kernels' vector accesses rely on: 16 bytes for tensors of
// elements (q, caches and pools, k_new / v_new, out, the workspace), 4 bytes
// for arrays of int32 or float32 values (seq_lens, block tables, lse,
// scales, pairs, parents).  A null pointer counts as aligned (the null
// checks are separate).
static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

static int ilog2_exact(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return (1 << l) == x ? l : -1;
}

static int check_common(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                        int B, int h, int g, int d, float scale, int dtype, int num_splits,
                        const float* out, const float* lse) {
    if (B < 0 || h <= 0 || g <= 0 || d <= 0 || num_splits < KVC_SPLITS_STREAM) return KVC_ERR_INVALID;
    if (h % g != 0) return KVC_ERR_INVALID;
    if (!isfinite(scale)) return KVC_ERR_INVALID;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    if (d > 256) return KVC_ERR_UNSUPPORTED;
    if (B > 0 && (!q || !k || !v || !seq_lens || !out || !lse)) return KVC_ERR_INVALID;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(out) || !al4(seq_lens) || !al4(lse))
        return KVC_ERR_INVALID;
    if (B > 65535 || g > 65535) return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
}

// Fix the launch on the current device: stream grid size, automatic chunk
// count and work-group width.  Needs a.B, a.g, a.m, a.cap_len.
static void resolve_launch(DecodeArgs& a, Schedule& sc, bool paged, int max_len) {
    a.stream = sc.stream ? 1 : 0;
    a.num_wgs = 0;
    a.waves = sc.kind == kGeneric ? generic_rows_per_wg(a.m) : 4;
    a.slices = row_slices(sc.kind, a.m);
    a.row_blocks = 1;
    a.nqt = 0;
    if (sc.kind == kPrefill) {
        const PrefillShape ps = prefill_shape(a.m, a.d);
        a.nqt = ps.nqt;
        a.waves = ps.waves;
        a.row_blocks = ps.row_blocks;
        if (sc.stream) {
            long P = device_slots(prefill_kernel(ps.nqt, ps.waves, paged, true, a.d, kv_mode(a)), ps.waves);
            const long pieces = ((long)a.B * a.g * max_len + 255) / 256;
            if (P > pieces) P = pieces;
            a.num_wgs = (int)(P < 1 ? 1 : P);
        } else if (sc.auto_chunks) {
            // chunks per unit that fill the device's slots once, counting
            // the row blocks; when the row blocks alone fill them, one chunk
            // per unit (the kernel walks a long chunk in table windows) and
            // no merge
            const long slots = device_slots(prefill_kernel(ps.nqt, ps.waves, paged, false, a.d, kv_mode(a)), ps.waves);
            const long groups = (long)a.B * ps.row_blocks * a.g;
            if (groups >= slots && paged && ps.row_blocks == 1 && kv_mode(a) == 0) {
                // a paged bf16 pool's ragged lengths: chunks of at most
                // kPagedChunk positions instead of whole units (64-sequence
                // pool: head dim 96 194 -> 174 us per call, 80: 195 -> 172
                // us, 32 tokens at head dim 128: 377 -> 358 us; FP8 codes
                // with 32 tokens measured 315 us whole, 333 us chunked)
                const long C = clamp_chunks(ceil_div(max_len, kPagedChunk), max_len);
                sc.plan = C == 1 ? Plan{(int)(ceil_div(max_len, kTileTokens) * kTileTokens), 1}
                                 : plan_for_chunks(max_len, C);
            } else if (groups >= slots) {
                sc.plan = Plan{(int)(ceil_div(max_len, kTileTokens) * kTileTokens), 1};
            } else {
                const long C = chunks_for_slots(slots, a.B * ps.row_blocks, a.g, max_len);
                sc.plan = C == 1 ? Plan{(int)(ceil_div(max_len, kTileTokens) * kTileTokens), 1}
                                 : plan_for_chunks(max_len, C);
            }
        }
        a.chunk_len = sc.plan.chunk_len;
        a.num_chunks = sc.plan.num_chunks;
        return;
    }
    if (sc.stream) {
        long P = device_slots(kernel_for(sc.kind, a.m, paged, true, 4, general_features(a), kv_mode(a)), 4);
        // No more work-groups than 256-position pieces of the largest possible batch.
        const long pieces = ((long)a.B * a.g * max_len + 255) / 256;
        if (P > pieces) P = pieces;
        a.num_wgs = (int)(P < 1 ? 1 : P);
    } else if (sc.auto_chunks) {
        const AutoShape sh = auto_shape(sc.kind, a.m < 32 ? a.m : 32, a.B * a.slices, a.g, max_len,
                                        paged, general_features(a), kv_mode(a));
        a.waves = sh.waves;
        // One chunk per unit may exceed kMaxChunk: the engines walk a chunk in
        // windows of at most kMaxChunk positions.
        sc.plan = sh.chunks == 1 ? Plan{(int)(ceil_div(max_len, kTileTokens) * kTileTokens), 1}
                                 : plan_for_chunks(max_len, sh.chunks);
    }
    a.chunk_len = sc.plan.chunk_len;
    a.num_chunks = sc.plan.num_chunks;
    if (!sc.stream && !sc.auto_chunks && sc.kind == kMfma && a.m > 16) {
        // Two query tiles per work-group: a fixed chunk grid that the device
        // holds at once with 8-wavefront work-groups runs twice the
        // wavefronts that way (with one tile, 4-wavefront work-groups keep
        // the tiling of the paged kernels).
        const void* f8 = kernel_for(sc.kind, a.m < 32 ? a.m : 32, paged, false, 8,
                                    general_features(a), kv_mode(a));
        const long wgs = (long)a.num_chunks * a.g * a.slices * a.B;
        if (f8 != nullptr && wgs <= device_slots(f8, 8)) a.waves = 8;
    }
}

// Scratch of kvc_append_decode_attention_noalloc: the split partials of one
// call live in this file-scope device array instead of a caller's
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: its device address comes from hipGetSymbolAddress,
// once per device (scratch_address), and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's `scratch` (nullptr if the query fails).
// The first call on a device makes the query with that device current.
static void* scratch_address() {
    static void* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_cache_lock);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// Marker for run_decode: take the split partials from `scratch`.
static char g_use_scratch;
static void* const kUseScratch = &g_use_scratch;

static int run_decode(DecodeArgs& a, int dtype, int max_len, int num_splits, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    const bool paged = a.block_table != nullptr;
    // Over a paged FP8 pool, several new tokens per sequence (the kernels'
    // general features) ran faster chunked than on the stream grid: 8 rows
    // per KV head (2 tokens) 130 vs 142 us, 16 rows 135 vs 167 us per call
    // at 3 chunks over the 64-sequence pool; bf16 pools stream (212 vs 218,
    // 221 vs 227 us).
    const bool prefer_chunks = a.window > 0 || (kv_mode(a) != 0 && a.n > 1);
    Schedule sc = make_schedule(a.B, a.h, a.g, a.d, dtype, max_len, num_splits, paged, prefer_chunks,
                                kv_mode(a));
    // (the workspace query knows no FP8 flag: it sizes for the bf16 kernels,
    // which bounds the FP8 ones)
    const size_t need = required_workspace(a.B, a.h, a.g, a.d, dtype, max_len, num_splits, paged);
    if (workspace == kUseScratch) {
        // every other argument has been validated by now
        if (need > kScratchBytes) return KVC_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0 && a.B > 0) {
            workspace = scratch_address();
            if (workspace == nullptr) return KVC_ERR_HIP;
            workspace_bytes = kScratchBytes;
        }
    }
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return KVC_ERR_WORKSPACE;
    if (!al16(workspace) || !al16(a.k_new) || !al16(a.v_new) || !al4(a.block_table) ||
        !al4(a.k_scale) || !al4(a.v_scale))
        return KVC_ERR_INVALID;
    if (a.B == 0) return KVC_OK;
    resolve_launch(a, sc, paged, max_len);
    // the launch's own partials must fit what was checked above
    if (workspace_for(a.B, a.h, a.g, a.d, sc) > (workspace != nullptr ? workspace_bytes : 0))
        return KVC_ERR_WORKSPACE;
    const size_t rows = workspace_rows(a.B, a.h, a.g, sc);
    if (rows > 0) {
        char* w = static_cast<char*>(workspace);
        a.part_o = reinterpret_cast<float*>(w);
        a.part_lse = reinterpret_cast<float*>(w + align256(rows * a.d * sizeof(float)));
    } else {
        a.part_o = nullptr;
        a.part_lse = nullptr;
    }
    hipError_t err;
    switch (sc.kind) {
        case kValu: err = launch_decode_valu_bf16_d128(a, stream); break;
        case kMfma: err = launch_decode_mfma_bf16_d128(a, stream); break;
        case kPrefill: err = launch_prefill_mfma(a, stream); break;
        default: err = launch_decode_generic(a, dtype, stream); break;
    }
    if (err != hipSuccess) return KVC_ERR_HIP;
    if (sc.stream) {
        if (launch_merge_stream(a, stream) != hipSuccess) return KVC_ERR_HIP;
    } else if (a.num_chunks > 1) {
        if (launch_merge(a, stream) != hipSuccess) return KVC_ERR_HIP;
    }
    return KVC_OK;
}

}  // namespace kvc

using namespace kvc;

extern "C" {

int kvc_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char* kvc_status_string(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_INVALID: return "invalid argument";
        case KVC_ERR_UNSUPPORTED: return "unsupported dtype or shape";
        case KVC_ERR_WORKSPACE: return "workspace missing or too small";
        case KVC_ERR_HIP: return "HIP launch error";
        case KVC_ERR_SCRATCH: return "the call needs more split scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

// Longest position range a unit can read: the capacity, or with a sliding
// window the window plus the other new tokens.  Chunk plans and workspaces
// are sized for it.
static int plan_len(int capacity, int window, int n) {
    if (window <= 0) return capacity;
    const long w = (long)window + n - 1;
    return w < capacity ? (int)w : capacity;
}

// The schedule a call with n query tokens per sequence and window W makes
// (n = 1, W = 0: the single-token call): h counts query rows (h * n).
static Schedule query_schedule(int B, int h, int g, int d, int dtype, int max_len, int num_splits,
                               bool paged, int n, int window, bool kv8) {
    const bool prefer_chunks = window > 0 || (kv8 && n > 1);
    return make_schedule(B, h, g, d, dtype, max_len, num_splits, paged, prefer_chunks, kv8 ? 1 : 0);
}

static int plan_query(int B, int h, int g, int d, int n, int window, int dtype, int max_seq_len,
                      int num_splits, int paged, int* mode, int* chunk_len, int* num_chunks) {
    if (B < 0 || h <= 0 || g <= 0 || d <= 0 || h % g != 0 || num_splits < KVC_SPLITS_STREAM ||
        max_seq_len < 0 || n <= 0 || window < 0)
        return KVC_ERR_INVALID;
    const bool kv8 = dtype == KVC_FP8_E4M3;  // bf16 q over an FP8 cache
    if (kv8) dtype = KVC_BF16;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    const Schedule sc = query_schedule(B, h, g, d, dtype, max_seq_len, num_splits, paged != 0, n,
                                       window, kv8);
    if (mode) *mode = sc.stream ? KVC_SPLIT_STREAM : (sc.auto_chunks ? KVC_SPLIT_AUTO_CHUNKS : KVC_SPLIT_CHUNKS);
    const bool fixed = !sc.stream && !sc.auto_chunks;
    if (chunk_len) *chunk_len = fixed ? sc.plan.chunk_len : 0;
    if (num_chunks) *num_chunks = fixed ? sc.plan.num_chunks : 0;
    return KVC_OK;
}

int kvc_decode_plan(int B, int h, int g, int d, int dtype, int max_seq_len, int num_splits,
                    int paged, int* mode, int* chunk_len, int* num_chunks) {
    return plan_query(B, h, g, d, 1, 0, dtype, max_seq_len, num_splits, paged, mode, chunk_len,
                      num_chunks);
}

int kvc_decode_plan_multi(int B, int h, int g, int d, int n, int window, int dtype, int capacity,
                          int num_splits, int paged, int* mode, int* chunk_len, int* num_chunks) {
    // h counts query heads: the head map needs h % g == 0 before the rows multiply by n
    if (n <= 0 || h <= 0 || g <= 0 || h % g != 0 || window < 0 || capacity < 0)
        return KVC_ERR_INVALID;
    if ((long)h * n > 65535) return KVC_ERR_UNSUPPORTED;
    return plan_query(B, h * n, g, d, n, window, dtype, plan_len(capacity, window, n), num_splits,
                      paged, mode, chunk_len, num_chunks);
}

static int launch_shape_query(int B, int h, int g, int d, int n, int window, int dtype,
                              int max_seq_len, int num_splits, int paged, int* waves, int* num_wgs,
                              int* chunk_len, int* num_chunks) {
    if (B <= 0 || h <= 0 || g <= 0 || d <= 0 || h % g != 0 || num_splits < KVC_SPLITS_STREAM ||
        max_seq_len <= 0 || n <= 0 || window < 0)
        return KVC_ERR_INVALID;
    const bool kv8 = dtype == KVC_FP8_E4M3;
    if (kv8) dtype = KVC_BF16;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    if (d > 256) return KVC_ERR_UNSUPPORTED;
    Schedule sc = query_schedule(B, h, g, d, dtype, max_seq_len, num_splits, paged != 0, n, window,
                                 kv8);
    DecodeArgs a{};
    a.B = B; a.h = h; a.g = g; a.d = d; a.m = h / g; a.n = n; a.window = window;
    a.cap_len = max_seq_len;
    a.kv8 = kv8 ? 1 : 0;
    resolve_launch(a, sc, paged != 0, max_seq_len);
    if (waves) *waves = a.waves;
    // the generic kernel: per KV head and block of up to 16 query rows (one
    // wavefront per row); the others: per unit and row slice
    const int per_chunk = sc.kind == kGeneric ? g * ((a.m + a.waves - 1) / a.waves)
                                              : g * a.slices * a.row_blocks;
    if (num_wgs) *num_wgs = a.stream ? a.num_wgs : a.num_chunks * per_chunk * B;
    if (chunk_len) *chunk_len = a.stream ? 0 : a.chunk_len;
    if (num_chunks) *num_chunks = a.stream ? 0 : a.num_chunks;
    return KVC_OK;
}

int kvc_decode_launch_shape(int B, int h, int g, int d, int dtype, int max_seq_len, int num_splits,
                            int paged, int* waves, int* num_wgs, int* chunk_len, int* num_chunks) {
    return launch_shape_query(B, h, g, d, 1, 0, dtype, max_seq_len, num_splits, paged, waves,
                              num_wgs, chunk_len, num_chunks);
}

int kvc_decode_launch_shape_multi(int B, int h, int g, int d, int n, int window, int dtype,
                                  int capacity, int num_splits, int paged, int* waves,
                                  int* num_wgs, int* chunk_len, int* num_chunks) {
    if (n <= 0 || h <= 0 || g <= 0 || h % g != 0 || window < 0 || capacity <= 0)
        return KVC_ERR_INVALID;
    if ((long)h * n > 65535) return KVC_ERR_UNSUPPORTED;
    return launch_shape_query(B, h * n, g, d, n, window, dtype, plan_len(capacity, window, n),
                              num_splits, paged, waves, num_wgs, chunk_len, num_chunks);
}

size_t kvc_decode_workspace_bytes(int B, int h, int g, int d, int dtype, int max_seq_len,
                                  int num_splits, int paged) {
    if (B <= 0 || h <= 0 || g <= 0 || d <= 0 || h % g != 0 || num_splits < KVC_SPLITS_STREAM ||
        max_seq_len < 0)
        return 0;
    if (dtype == KVC_FP8_E4M3) dtype = KVC_BF16;  // the same workspaces
    if (dtype != KVC_F32 && dtype != KVC_BF16) return 0;
    return required_workspace(B, h, g, d, dtype, max_seq_len, num_splits, paged != 0);
}

int kvc_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
               const int32_t* block_table, int max_blocks, int block_size,
               const int32_t* seq_lens_before, int B, int g, int d, int capacity, int dtype,
               hipStream_t stream) {
    if (B < 0 || g <= 0 || d <= 0 || capacity <= 0) return KVC_ERR_INVALID;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    if (B == 0) return KVC_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens_before) return KVC_ERR_INVALID;
    if (block_table != nullptr && (max_blocks <= 0 || block_size <= 0)) return KVC_ERR_INVALID;
    if (!al16(k_new) || !al16(v_new) || !al16(k_cache) || !al16(v_cache) || !al4(block_table) ||
        !al4(seq_lens_before))
        return KVC_ERR_INVALID;
    const int eb = dtype == KVC_F32 ? 4 : 2;
    if (launch_append(k_new, v_new, k_cache, v_cache, block_table, max_blocks, block_size,
                      seq_lens_before, B, g, 1, d, capacity, 0, eb, stream) != hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

// Shared body of the contiguous entry points.  n queries per sequence
// (q [B, h, n, d]); k_new != nullptr: the call also appends the n new tokens
// (k_new [B, g, n, d]) and seq_lens holds the lengths before the step.
static int decode_contiguous(const void* q, const void* k_new, const void* v_new,
                             const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                             int B, int h, int g, int d, int n, int t_cap, int window, int ring,
                             float scale, int dtype, int num_splits, void* workspace,
                             size_t workspace_bytes, float* out, float* lse, hipStream_t stream,
                             const float* k_scale = nullptr, const float* v_scale = nullptr) {
    int st = check_common(q, k_cache, v_cache, seq_lens, B, h, g, d, scale, dtype, num_splits,
                          out, lse);
    if (st != KVC_OK) return st;
    if (t_cap <= 0 || n <= 0 || window < 0) return KVC_ERR_INVALID;
    // a ring keeps every position a token can see: window + n - 1 <= t_cap
    if (ring && (window <= 0 || (long)window + n - 1 > t_cap)) return KVC_ERR_INVALID;
    if ((long)h * n > 65535) return KVC_ERR_UNSUPPORTED;
    DecodeArgs a{};
    a.q = q; a.k = k_cache; a.v = v_cache; a.seq_lens = seq_lens;
    a.block_table = nullptr; a.max_blocks = 0; a.block_size = 1; a.log2_bs = 0; a.num_blocks = 0;
    a.B = B; a.h = h * n; a.g = g; a.d = d; a.m = (h / g) * n; a.n = n;
    a.t_cap = t_cap; a.cap_len = ring ? 0x7fffffff : t_cap;
    a.window = window; a.ring = ring ? 1 : 0;
    a.kv8 = k_scale != nullptr ? 1 : 0; a.k_scale = k_scale; a.v_scale = v_scale;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.out = out; a.lse = lse;
    a.len_add = k_new != nullptr ? n : 0;
    a.k_new = k_new; a.v_new = v_new;
    return run_decode(a, dtype, plan_len(t_cap, window, n), num_splits, workspace, workspace_bytes,
                      stream);
}

static int decode_paged(const void* q, const void* k_new, const void* v_new, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, int max_blocks,
                        int block_size, int num_blocks, const int32_t* seq_lens, int B, int h,
                        int g, int d, int n, int window, float scale, int dtype, int num_splits,
                        void* workspace, size_t workspace_bytes, float* out, float* lse,
                        hipStream_t stream, const float* k_scale = nullptr,
                        const float* v_scale = nullptr, int block_scales = 0) {
    int st = check_common(q, k_pool, v_pool, seq_lens, B, h, g, d, scale, dtype, num_splits,
                          out, lse);
    if (st != KVC_OK) return st;
    if (max_blocks <= 0 || num_blocks <= 0 || n <= 0 || window < 0) return KVC_ERR_INVALID;
    if (B > 0 && block_table == nullptr) return KVC_ERR_INVALID;
    const int lg = ilog2_exact(block_size);
    if (block_size < 8 || block_size > 256 || lg < 0) return KVC_ERR_INVALID;
    const long cap = (long)max_blocks * block_size;
    if (cap > 0x7fffffffL) return KVC_ERR_UNSUPPORTED;
    if ((long)h * n > 65535) return KVC_ERR_UNSUPPORTED;
    // the kernels index pool rows (block, KV head, position) in 32 bits
    if ((long)num_blocks * g * block_size > 0xffffffffL) return KVC_ERR_UNSUPPORTED;
    DecodeArgs a{};
    a.q = q; a.k = k_pool; a.v = v_pool; a.seq_lens = seq_lens;
    a.block_table = block_table; a.max_blocks = max_blocks; a.block_size = block_size;
    a.log2_bs = lg; a.num_blocks = num_blocks;
    a.B = B; a.h = h * n; a.g = g; a.d = d; a.m = (h / g) * n; a.n = n;
    a.t_cap = 0; a.cap_len = (int)cap;
    a.window = window; a.ring = 0;
    a.kv8 = k_scale != nullptr ? 1 : 0; a.k_scale = k_scale; a.v_scale = v_scale;
    a.block_scales = block_scales;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.out = out; a.lse = lse;
    a.len_add = k_new != nullptr ? n : 0;
    a.k_new = k_new; a.v_new = v_new;
    return run_decode(a, dtype, plan_len((int)cap, window, n), num_splits, workspace,
                      workspace_bytes, stream);
}

int kvc_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, int B, int h, int g, int d, int t_cap,
                         float scale, int dtype, int num_splits, void* workspace,
                         size_t workspace_bytes, float* out, float* lse, hipStream_t stream) {
    return decode_contiguous(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h, g, d, 1, t_cap,
                             0, 0, scale, dtype, num_splits, workspace, workspace_bytes, out, lse,
                             stream);
}

int kvc_decode_attention_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, int max_blocks, int block_size,
                               int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                               int d, float scale, int dtype, int num_splits, void* workspace,
                               size_t workspace_bytes, float* out, float* lse,
                               hipStream_t stream) {
    return decode_paged(q, nullptr, nullptr, k_pool, v_pool, block_table, max_blocks, block_size,
                        num_blocks, seq_lens, B, h, g, d, 1, 0, scale, dtype, num_splits, workspace,
                        workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* seq_lens_before,
                                int B, int h, int g, int d, int t_cap, float scale, int dtype,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, 1, t_cap, 0, 0, scale, dtype, num_splits,
                             workspace, workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_noalloc(const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache,
                                        const int32_t* seq_lens_before, int B, int h, int g, int d,
                                        int t_cap, float scale, int dtype, int num_splits,
                                        float* out, float* lse, hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, 1, t_cap, 0, 0, scale, dtype, num_splits,
                             kUseScratch, 0, out, lse, stream);
}

size_t kvc_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kvc_append_decode_attention_paged(const void* q, const void* k_new, const void* v_new,
                                      void* k_pool, void* v_pool, const int32_t* block_table,
                                      int max_blocks, int block_size, int num_blocks,
                                      const int32_t* seq_lens_before, int B, int h, int g, int d,
                                      float scale, int dtype, int num_splits, void* workspace,
                                      size_t workspace_bytes, float* out, float* lse,
                                      hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table,
                        max_blocks, block_size, num_blocks, seq_lens_before, B, h, g, d, 1, 0,
                        scale, dtype, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int kvc_decode_attention_multi(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, int B, int h, int g, int d, int n,
                               int t_cap, float scale, int dtype, int num_splits, void* workspace,
                               size_t workspace_bytes, float* out, float* lse, hipStream_t stream) {
    return decode_contiguous(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h, g, d, n, t_cap,
                             0, 0, scale, dtype, num_splits, workspace, workspace_bytes, out, lse,
                             stream);
}

int kvc_decode_attention_multi_paged(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                     int d, int n, float scale, int dtype, int num_splits,
                                     void* workspace, size_t workspace_bytes, float* out,
                                     float* lse, hipStream_t stream) {
    return decode_paged(q, nullptr, nullptr, k_pool, v_pool, block_table, max_blocks, block_size,
                        num_blocks, seq_lens, B, h, g, d, n, 0, scale, dtype, num_splits, workspace,
                        workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_multi(const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache,
                                      const int32_t* seq_lens_before, int B, int h, int g, int d,
                                      int n, int t_cap, float scale, int dtype, int num_splits,
                                      void* workspace, size_t workspace_bytes, float* out,
                                      float* lse, hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, n, t_cap, 0, 0, scale, dtype, num_splits,
                             workspace, workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_multi_paged(const void* q, const void* k_new, const void* v_new,
                                            void* k_pool, void* v_pool,
                                            const int32_t* block_table, int max_blocks,
                                            int block_size, int num_blocks,
                                            const int32_t* seq_lens_before, int B, int h, int g,
                                            int d, int n, float scale, int dtype, int num_splits,
                                            void* workspace, size_t workspace_bytes, float* out,
                                            float* lse, hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table,
                        max_blocks, block_size, num_blocks, seq_lens_before, B, h, g, d, n, 0,
                        scale, dtype, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int kvc_decode_attention_window(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                int t_cap, int window, int ring, float scale, int dtype,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream) {
    return decode_contiguous(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h, g, d, n, t_cap,
                             window, ring, scale, dtype, num_splits, workspace, workspace_bytes, out,
                             lse, stream);
}

int kvc_decode_attention_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, int max_blocks, int block_size,
                                      int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                      int d, int n, int window, float scale, int dtype,
                                      int num_splits, void* workspace, size_t workspace_bytes,
                                      float* out, float* lse, hipStream_t stream) {
    return decode_paged(q, nullptr, nullptr, k_pool, v_pool, block_table, max_blocks, block_size,
                        num_blocks, seq_lens, B, h, g, d, n, window, scale, dtype, num_splits,
                        workspace, workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_window(const void* q, const void* k_new, const void* v_new,
                                       void* k_cache, void* v_cache,
                                       const int32_t* seq_lens_before, int B, int h, int g, int d,
                                       int n, int t_cap, int window, int ring, float scale,
                                       int dtype, int num_splits, void* workspace,
                                       size_t workspace_bytes, float* out, float* lse,
                                       hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, n, t_cap, window, ring, scale, dtype,
                             num_splits, workspace, workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_window_paged(const void* q, const void* k_new, const void* v_new,
                                             void* k_pool, void* v_pool,
                                             const int32_t* block_table, int max_blocks,
                                             int block_size, int num_blocks,
                                             const int32_t* seq_lens_before, int B, int h, int g,
                                             int d, int n, int window, float scale, int dtype,
                                             int num_splits, void* workspace,
                                             size_t workspace_bytes, float* out, float* lse,
                                             hipStream_t stream) {
    if (B > 0 && (k_new == nullptr || v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table,
                        max_blocks, block_size, num_blocks, seq_lens_before, B, h, g, d, n, window,
                        scale, dtype, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int kvc_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                    int num_blocks, int g, int block_size, int d, int dtype, hipStream_t stream) {
    if (num_pairs < 0 || num_blocks <= 0 || g <= 0 || block_size <= 0 || d <= 0)
        return KVC_ERR_INVALID;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    if (num_pairs == 0) return KVC_OK;
    if (!k_pool || !v_pool || !pairs) return KVC_ERR_INVALID;
    if (!al16(k_pool) || !al16(v_pool) || !al4(pairs)) return KVC_ERR_INVALID;
    const long block_bytes = (long)g * block_size * d * (dtype == KVC_F32 ? 4 : 2);
    if (launch_copy_blocks(k_pool, v_pool, pairs, num_pairs, num_blocks, block_bytes, stream) !=
        hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

int kvc_fork_block_tables(const int32_t* block_table, const int32_t* seq_lens, int B_src,
                          int max_blocks, const int32_t* parent, int B, int32_t* block_table_out,
                          int32_t* seq_lens_out, hipStream_t stream) {
    if (B < 0 || B_src <= 0 || max_blocks <= 0) return KVC_ERR_INVALID;
    if (B == 0) return KVC_OK;
    if (!block_table || !seq_lens || !parent || !block_table_out || !seq_lens_out)
        return KVC_ERR_INVALID;
    if (block_table_out == block_table || seq_lens_out == seq_lens) return KVC_ERR_INVALID;
    if (!al4(block_table) || !al4(seq_lens) || !al4(parent) || !al4(block_table_out) ||
        !al4(seq_lens_out))
        return KVC_ERR_INVALID;
    if (launch_fork_tables(block_table, seq_lens, B_src, max_blocks, parent, B, block_table_out,
                           seq_lens_out, stream) != hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

int kvc_gather_cache(const void* k_src, const void* v_src, const int32_t* seq_lens, int B_src,
                     const int32_t* parent, int B, void* k_dst, void* v_dst, int g, int t_cap,
                     int d, int dtype, hipStream_t stream) {
    if (B < 0 || B_src <= 0 || g <= 0 || t_cap <= 0 || d <= 0) return KVC_ERR_INVALID;
    if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
    if (B == 0) return KVC_OK;
    if (!k_src || !v_src || !seq_lens || !parent || !k_dst || !v_dst) return KVC_ERR_INVALID;
    if (k_dst == k_src || v_dst == v_src || k_dst == v_src || v_dst == k_src || k_dst == v_dst)
        return KVC_ERR_INVALID;
    if (!al16(k_src) || !al16(v_src) || !al16(k_dst) || !al16(v_dst) || !al4(seq_lens) ||
        !al4(parent))
        return KVC_ERR_INVALID;
    if ((long)B * g > 0x7fffffffL || ceil_div(t_cap, 64) > 65535) return KVC_ERR_UNSUPPORTED;
    const long row_bytes = (long)d * (dtype == KVC_F32 ? 4 : 2);
    if (launch_gather_cache(k_src, v_src, k_dst, v_dst, seq_lens, B_src, parent, B, g, t_cap,
                            row_bytes, stream) != hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

int kvc_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int max_blocks, int block_size, const int32_t* seq_lens_before, int B, int g,
                   int d, int capacity, hipStream_t stream) {
    if (B < 0 || g <= 0 || d <= 0 || capacity <= 0) return KVC_ERR_INVALID;
    if (B == 0) return KVC_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !seq_lens_before)
        return KVC_ERR_INVALID;
    if (block_table != nullptr && (max_blocks <= 0 || block_size <= 0)) return KVC_ERR_INVALID;
    if (!al16(k_new) || !al16(v_new) || !al16(k_cache) || !al16(v_cache) || !al4(k_scale) ||
        !al4(v_scale) || !al4(block_table) || !al4(seq_lens_before))
        return KVC_ERR_INVALID;
    if (launch_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                          max_blocks, block_size, seq_lens_before, B, g, 1, d, capacity, 0, 0,
                          stream) != hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

int kvc_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int B, int h, int g, int d, int t_cap, float scale, int num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             hipStream_t stream) {
    if (B > 0 && (!k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_contiguous(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h, g, d, 1, t_cap,
                             0, 0, scale, KVC_BF16, num_splits, workspace, workspace_bytes, out,
                             lse, stream, k_scale, v_scale);
}

int kvc_decode_attention_fp8_paged(const void* q, const void* k_pool, const void* v_pool,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, int max_blocks, int block_size,
                                   int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                   int d, float scale, int num_splits, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream) {
    if (B > 0 && (!k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_paged(q, nullptr, nullptr, k_pool, v_pool, block_table, max_blocks, block_size,
                        num_blocks, seq_lens, B, h, g, d, 1, 0, scale, KVC_BF16, num_splits,
                        workspace, workspace_bytes, out, lse, stream, k_scale, v_scale);
}

int kvc_append_decode_attention_fp8(const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* seq_lens_before, int B,
                                    int h, int g, int d, int t_cap, float scale, int num_splits,
                                    void* workspace, size_t workspace_bytes, float* out,
                                    float* lse, hipStream_t stream) {
    if (B > 0 && (!k_new || !v_new || !k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, 1, t_cap, 0, 0, scale, KVC_BF16,
                             num_splits, workspace, workspace_bytes, out, lse, stream, k_scale,
                             v_scale);
}

int kvc_append_decode_attention_fp8_paged(const void* q, const void* k_new, const void* v_new,
                                          void* k_pool, void* v_pool, const float* k_scale,
                                          const float* v_scale, const int32_t* block_table,
                                          int max_blocks, int block_size, int num_blocks,
                                          const int32_t* seq_lens_before, int B, int h, int g,
                                          int d, float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream) {
    if (B > 0 && (!k_new || !v_new || !k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table,
                        max_blocks, block_size, num_blocks, seq_lens_before, B, h, g, d, 1, 0,
                        scale, KVC_BF16, num_splits, workspace, workspace_bytes, out, lse, stream,
                        k_scale, v_scale);
}

// FP8 caches with several new tokens per sequence and / or a sliding window
// (window 0 = none; the _multi calls are the _window calls without one).
int kvc_decode_attention_fp8_window(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                    int t_cap, int window, int ring, float scale, int num_splits,
                                    void* workspace, size_t workspace_bytes, float* out, float* lse,
                                    hipStream_t stream) {
    if (B > 0 && (!k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_contiguous(q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, h, g, d, n, t_cap,
                             window, ring, scale, KVC_BF16, num_splits, workspace, workspace_bytes,
                             out, lse, stream, k_scale, v_scale);
}

int kvc_decode_attention_fp8_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                          const float* k_scale, const float* v_scale,
                                          const int32_t* block_table, int max_blocks,
                                          int block_size, int num_blocks, const int32_t* seq_lens,
                                          int B, int h, int g, int d, int n, int window,
                                          float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream) {
    if (B > 0 && (!k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_paged(q, nullptr, nullptr, k_pool, v_pool, block_table, max_blocks, block_size,
                        num_blocks, seq_lens, B, h, g, d, n, window, scale, KVC_BF16, num_splits,
                        workspace, workspace_bytes, out, lse, stream, k_scale, v_scale);
}

int kvc_append_decode_attention_fp8_window(const void* q, const void* k_new, const void* v_new,
                                           void* k_cache, void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* seq_lens_before,
                                           int B, int h, int g, int d, int n, int t_cap,
                                           int window, int ring, float scale, int num_splits,
                                           void* workspace, size_t workspace_bytes, float* out,
                                           float* lse, hipStream_t stream) {
    if (B > 0 && (!k_new || !v_new || !k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_contiguous(q, B > 0 ? k_new : nullptr, v_new, k_cache, v_cache,
                             seq_lens_before, B, h, g, d, n, t_cap, window, ring, scale, KVC_BF16,
                             num_splits, workspace, workspace_bytes, out, lse, stream, k_scale,
                             v_scale);
}

int kvc_append_decode_attention_fp8_window_paged(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens_before, int B, int h, int g, int d,
    int n, int window, float scale, int num_splits, void* workspace, size_t workspace_bytes,
    float* out, float* lse, hipStream_t stream) {
    if (B > 0 && (!k_new || !v_new || !k_scale || !v_scale)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table,
                        max_blocks, block_size, num_blocks, seq_lens_before, B, h, g, d, n, window,
                        scale, KVC_BF16, num_splits, workspace, workspace_bytes, out, lse, stream,
                        k_scale, v_scale);
}

int kvc_decode_attention_fp8_multi(const void* q, const void* k_cache, const void* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                   int t_cap, float scale, int num_splits, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream) {
    return kvc_decode_attention_fp8_window(q, k_cache, v_cache, k_scale, v_scale, seq_lens, B, h,
                                           g, d, n, t_cap, 0, 0, scale, num_splits, workspace,
                                           workspace_bytes, out, lse, stream);
}

int kvc_decode_attention_fp8_multi_paged(const void* q, const void* k_pool, const void* v_pool,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_table, int max_blocks,
                                         int block_size, int num_blocks, const int32_t* seq_lens,
                                         int B, int h, int g, int d, int n, float scale,
                                         int num_splits, void* workspace, size_t workspace_bytes,
                                         float* out, float* lse, hipStream_t stream) {
    return kvc_decode_attention_fp8_window_paged(q, k_pool, v_pool, k_scale, v_scale, block_table,
                                                 max_blocks, block_size, num_blocks, seq_lens, B,
                                                 h, g, d, n, 0, scale, num_splits, workspace,
                                                 workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_fp8_multi(const void* q, const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache, const float* k_scale,
                                          const float* v_scale, const int32_t* seq_lens_before,
                                          int B, int h, int g, int d, int n, int t_cap,
                                          float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream) {
    return kvc_append_decode_attention_fp8_window(q, k_new, v_new, k_cache, v_cache, k_scale,
                                                  v_scale, seq_lens_before, B, h, g, d, n, t_cap,
                                                  0, 0, scale, num_splits, workspace,
                                                  workspace_bytes, out, lse, stream);
}

int kvc_append_decode_attention_fp8_multi_paged(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens_before, int B, int h, int g, int d,
    int n, float scale, int num_splits, void* workspace, size_t workspace_bytes, float* out,
    float* lse, hipStream_t stream) {
    return kvc_append_decode_attention_fp8_window_paged(
        q, k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks, block_size,
        num_blocks, seq_lens_before, B, h, g, d, n, 0, scale, num_splits, workspace,
        workspace_bytes, out, lse, stream);
}

// FP8 pools with a scale per (physical block, KV head).
int kvc_append_fp8_paged_block_scaled(const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int max_blocks, int block_size,
                                      int num_blocks, const int32_t* seq_lens_before, int B, int g,
                                      int d, int n, hipStream_t stream) {
    if (B < 0 || g <= 0 || d <= 0 || n <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        block_size <= 0)
        return KVC_ERR_INVALID;
    if (B == 0) return KVC_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_table ||
        !seq_lens_before)
        return KVC_ERR_INVALID;
    if (!al16(k_new) || !al16(v_new) || !al16(k_pool) || !al16(v_pool) || !al4(k_scale) ||
        !al4(v_scale) || !al4(block_table) || !al4(seq_lens_before))
        return KVC_ERR_INVALID;
    if (launch_append_fp8(k_new, v_new, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks,
                          block_size, seq_lens_before, B, g, n, d, num_blocks, 0, 1, stream) !=
        hipSuccess)
        return KVC_ERR_HIP;
    return KVC_OK;
}

int kvc_decode_attention_fp8_paged_block_scaled(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens, int B, int h, int g, int d, int n,
    int window, float scale, int num_splits, void* workspace, size_t workspace_bytes, float* out,
    float* lse, hipStream_t stream) {
    if (B > 0 && (!k_scale || !v_scale)) return KVC_ERR_INVALID;
    if ((k_new == nullptr) != (v_new == nullptr)) return KVC_ERR_INVALID;
    return decode_paged(q, B > 0 ? k_new : nullptr, v_new, k_pool, v_pool, block_table, max_blocks,
                        block_size, num_blocks, seq_lens, B, h, g, d, n, window, scale, KVC_BF16,
                        num_splits, workspace, workspace_bytes, out, lse, stream, k_scale, v_scale,
                        1);
}

}  // extern "C"
