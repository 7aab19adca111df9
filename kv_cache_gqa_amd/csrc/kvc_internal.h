// kvc_internal.h -- host-side declarations shared by the launch code of
// libkvc.  Not part of the public ABI (that is include/kvc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvc {

// Positions per sub-tile: the unit every decode kernel walks the cache in.
constexpr int kTileTokens = 32;
// Upper bound on one chunk: keeps a chunk's slice of the block table
// (chunk_len / block_size + 2 entries for block_size >= 8) inside LDS.
constexpr int kMaxChunk = 4096;
constexpr int kMaxTableSlice = kMaxChunk / 8 + 2;
// Auto split: aim for about this many work-groups per launch, but never
// chunks shorter than kMinAutoChunk positions.
constexpr int kTargetWorkgroups = 2048;
constexpr int kMinAutoChunk = 256;
// Stream mode (persistent, position-balanced) needs the prefix sums of all
// sequence lengths in shared memory: batches up to kStreamMaxB sequences.
constexpr int kStreamMaxB = 1024;
// Stream-mode partial records are sized for at most this many resident
// work-groups per compute unit on a 256-CU device.
constexpr int kStreamMaxWgPerCu = 4;
constexpr int kStreamMaxCUs = 256;

struct Plan {
    int chunk_len;   // positions per chunk (multiple of kTileTokens)
    int num_chunks;  // chunks over max_seq_len (>= 1)
};

Plan make_plan(int B, int g, int max_seq_len, int num_splits);

// Everything one decode launch needs.  Layout facts:
//   q [B,h,d]; contiguous K/V [B,g,t_cap,d]; paged pools [nblk,g,bs,d];
//   block_table [B,max_blocks]; out [B,h,d] f32; lse [B,h] f32;
//   partial O [B,h,C,d] f32 and partial lse2 [B,h,C] f32 in the workspace.
struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* seq_lens;
    const int32_t* block_table;  // nullptr => contiguous
    int max_blocks;
    int block_size;
    int log2_bs;
    int num_blocks;
    int B, h, g, d, m;
    int t_cap;        // contiguous capacity in positions
    int cap_len;      // clamp bound for seq_lens: t_cap or max_blocks*block_size
    float scale_log2e;  // scale * log2(e): scores are kept in base 2
    int chunk_len;    // chunked mode
    int num_chunks;
    int stream;       // 1: persistent position-balanced grid of num_wgs work-groups
    int num_wgs;
    int waves;        // wavefronts per work-group (4 or 8)
    // Fused append: seq_lens holds the lengths before the step, the attended
    // length is seq_lens[b] + len_add, and when k_new is set the kernel reads
    // the new token (position seq_lens[b]) from k_new / v_new and writes it
    // into its cache slot.
    int len_add;
    const void* k_new;
    const void* v_new;
    // Queries per sequence (new tokens attending at once).  The kernels see
    // h = heads * n query rows per sequence and m = (heads / g) * n rows per
    // unit; row i is head i / n, token i % n, and token t sees
    // raw + len_add - (n - 1 - t) positions (clamped).
    int n;
    // Query-row slices per unit (chunked mode): more than 32 rows per KV head
    // are served by ceil(m / 32) work-groups of 32 rows each, blockIdx.y =
    // j * slices + slice.
    int slices;
    // Multi-row kernel (more than 32 rows per KV head, bf16): work-groups
    // per unit over its rows, and 16-row query tiles per wavefront.
    int row_blocks;
    int nqt;
    // Sliding window: 0 = none; W > 0: a token at position x sees positions
    // max(0, x + 1 - W) .. x.  ring (contiguous only): position p lives in
    // slot p mod t_cap (positions are not clamped to the capacity).
    int window;
    int ring;
    // FP8 E4M3 cache (q, k_new, v_new stay bf16): float32 scales, one per
    // KV head ([g]), or with block_scales (paged pools only) one per
    // physical block and KV head ([num_blocks, g]).
    int kv8;
    int block_scales;
    const float* k_scale;
    const float* v_scale;
    // Chunked mode (C > 1): partial O [B,h,C,d], partial base-2 lse [B,h,C].
    // Stream mode: records [num_wgs][2][m][d] and [num_wgs][2][m].
    float* part_o;
    float* part_lse;
    float* out;
    float* lse;
};

// Kernel families.  Each returns hipGetLastError() after its launch.
hipError_t launch_decode_generic(const DecodeArgs& a, int dtype, hipStream_t s);
// Query rows (one wavefront each) per work-group of the generic kernel.
int generic_rows_per_wg(int m);
hipError_t launch_decode_valu_bf16_d128(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_mfma_bf16_d128(const DecodeArgs& a, hipStream_t s);
hipError_t launch_prefill_mfma(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge_stream(const DecodeArgs& a, hipStream_t s);
// Kernel function for (m, layout, split mode, wavefronts per work-group,
// general features, FP8 cache), for launches and occupancy queries; nullptr
// when that combination is not built.  MFMA: waves in {4, 8}; VALU: 4.
// kv8: 0 = bf16 cache, 1 = FP8 with per-KV-head scales, 2 = FP8 with
// per-block scales (paged only).
const void* mfma_kernel(int m, bool paged, bool stream, int waves, bool gen, int kv8);
const void* valu_kernel(int m, bool paged, bool stream, int waves, bool gen, int kv8);
// Multi-row kernel for (16-row query tiles per wavefront, wavefronts per
// work-group, layout, grid: chunks or the stream grid (paged pools with one
// row block per unit), head dim, cache kind); nullptr when not built.
const void* prefill_kernel(int nqt, int waves, bool paged, bool stream, int d, int kv8);
// Whether a call needs the kernels' general features: several query tokens
// per sequence, a sliding window or a ring cache.
inline bool general_features(const DecodeArgs& a) { return a.n > 1 || a.window > 0 || a.ring != 0; }
// Cache kind of a call for kernel selection: 0 bf16, 1 FP8 with per-KV-head
// scales, 2 FP8 with per-block scales.
inline int kv_mode(const DecodeArgs& a) { return a.kv8 ? (a.block_scales ? 2 : 1) : 0; }
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int n_pairs,
                              int num_blocks, long block_bytes, hipStream_t s);
hipError_t launch_fork_tables(const int32_t* tables, const int32_t* lens, int B_src, int max_blocks,
                              const int32_t* parent, int B, int32_t* tables_out, int32_t* lens_out,
                              hipStream_t s);
hipError_t launch_gather_cache(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                               const int32_t* lens, int B_src, const int32_t* parent, int B, int g,
                               int t_cap, long row_bytes, hipStream_t s);
hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int max_blocks, int block_size,
                             const int32_t* seq_lens_before, int B, int g, int n, int d,
                             int capacity, int ring, int block_scales, hipStream_t s);
hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* block_table, int max_blocks, int block_size,
                         const int32_t* seq_lens_before, int B, int g, int n, int d, int capacity,
                         int ring, int elem_bytes, hipStream_t s);

// Which decode kernel a configuration uses (exposed for tests and tools).
enum KernelKind { kGeneric = 0, kValu = 1, kMfma = 2, kPrefill = 3 };
KernelKind choose_kernel(int dtype, int d, int m, int kv8 = 0);

}  // namespace kvc
