// blocks.hip -- block operations for shared and re-ranked caches.
//
// "KV Cache 优化与注意力机制加速" (plumephp.com) section 4.3: requests that
// share a prompt fork its block table and point at the same physical
// blocks; before a request writes into a shared block the block is copied
// (copy-on-write) and the request's table is pointed at the copy.  The host
// keeps reference counts and allocates blocks; these kernels move the bytes
// and the table rows.  "KV Cache 的增量解码" (zwjcode.cn) section 11: after
// beams are re-ranked, each beam's cache must follow its chosen parent.
//
// All copies are bit-exact 16-, 4- or 2-byte vector moves.
#include "kvc_device.h"

namespace kvc {

// Copy physical block src -> dst of the K pool (blockIdx.y = 0) or the V
// pool (1) for pair blockIdx.x.  Pairs naming a block outside [0, NB), and
// src == dst, are skipped.
template <typename V>
__global__ void __launch_bounds__(256) copy_blocks_kernel(V* k_pool, V* v_pool, const int32_t* pairs,
                                                          long vec_per_block, int num_blocks) {
    const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    V* pool = blockIdx.y == 0 ? k_pool : v_pool;
    const V* from = pool + (long)src * vec_per_block;
    V* to = pool + (long)dst * vec_per_block;
    // (Unrolling to keep 2, 4 or 8 loads in flight per thread measured no
    // faster on MI355X: scattered 32 KB copies run at about 4.85 TB/s.)
    for (long i = threadIdx.x; i < vec_per_block; i += blockDim.x) to[i] = from[i];
}

// Row b of the forked tables is row parent[b] of the source tables, and
// its length the parent's; a parent outside [0, B_src) gives a row of -1
// and length 0.  One thread per table entry; column 0's thread also moves
// the length.
__global__ void __launch_bounds__(256) fork_tables_kernel(const int32_t* tables, const int32_t* lens,
                                                          int B_src, int max_blocks,
                                                          const int32_t* parent, int B,
                                                          int32_t* tables_out, int32_t* lens_out) {
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long)B * max_blocks) return;
    const int b = (int)(t / max_blocks), i = (int)(t % max_blocks);
    const int pb = parent[b];
    const bool ok = pb >= 0 && pb < B_src;
    tables_out[t] = ok ? tables[(long)pb * max_blocks + i] : -1;
    if (i == 0) lens_out[b] = ok ? lens[pb] : 0;
}

// Contiguous caches re-ranked by parent: positions p < seq_lens[parent[b]]
// (clamped to [0, t_cap]) of every KV head of sequence b are copied from
// sequence parent[b]; other positions of the destination are not written.
// blockIdx.x = b * g + j, blockIdx.y = group of kGatherPositions positions.
constexpr int kGatherPositions = 64;

template <typename V>
__global__ void __launch_bounds__(256) gather_cache_kernel(const V* k_src, const V* v_src, V* k_dst,
                                                           V* v_dst, const int32_t* lens, int B_src,
                                                           const int32_t* parent, int g, int t_cap,
                                                           int vec_per_row) {
    const int b = blockIdx.x / g, j = blockIdx.x % g;
    const int pb = parent[b];
    if (pb < 0 || pb >= B_src) return;
    const int L = clamp_len(lens[pb], t_cap);
    const int p0 = blockIdx.y * kGatherPositions;
    const int p1 = min(p0 + kGatherPositions, L);
    if (p0 >= p1) return;
    const long src_row = ((long)pb * g + j) * t_cap;
    const long dst_row = ((long)b * g + j) * t_cap;
    const long n = (long)(p1 - p0) * vec_per_row;
    for (long i = threadIdx.x; i < n; i += blockDim.x) {
        const long off = (long)p0 * vec_per_row + i;
        k_dst[dst_row * vec_per_row + off] = k_src[src_row * vec_per_row + off];
        v_dst[dst_row * vec_per_row + off] = v_src[src_row * vec_per_row + off];
    }
}

template <typename V>
static void copy_blocks_t(void* k, void* v, const int32_t* pairs, int n_pairs, long bytes,
                          int num_blocks, hipStream_t s) {
    copy_blocks_kernel<V><<<dim3((unsigned)n_pairs, 2), dim3(256), 0, s>>>(
        (V*)k, (V*)v, pairs, bytes / (long)sizeof(V), num_blocks);
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int n_pairs,
                              int num_blocks, long block_bytes, hipStream_t s) {
    if (block_bytes % 16 == 0) copy_blocks_t<uint4>(k_pool, v_pool, pairs, n_pairs, block_bytes, num_blocks, s);
    else if (block_bytes % 4 == 0) copy_blocks_t<uint32_t>(k_pool, v_pool, pairs, n_pairs, block_bytes, num_blocks, s);
    else copy_blocks_t<uint16_t>(k_pool, v_pool, pairs, n_pairs, block_bytes, num_blocks, s);
    return hipGetLastError();
}

hipError_t launch_fork_tables(const int32_t* tables, const int32_t* lens, int B_src, int max_blocks,
                              const int32_t* parent, int B, int32_t* tables_out, int32_t* lens_out,
                              hipStream_t s) {
    const long n = (long)B * max_blocks;
    fork_tables_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
        tables, lens, B_src, max_blocks, parent, B, tables_out, lens_out);
    return hipGetLastError();
}

template <typename V>
static void gather_t(const void* ks, const void* vs, void* kd, void* vd, const int32_t* lens,
                     int B_src, const int32_t* parent, int B, int g, int t_cap, long row_bytes,
                     hipStream_t s) {
    const dim3 grid((unsigned)(B * g), (unsigned)((t_cap + kGatherPositions - 1) / kGatherPositions));
    gather_cache_kernel<V><<<grid, dim3(256), 0, s>>>((const V*)ks, (const V*)vs, (V*)kd, (V*)vd,
                                                      lens, B_src, parent, g, t_cap,
                                                      (int)(row_bytes / (long)sizeof(V)));
}

hipError_t launch_gather_cache(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                               const int32_t* lens, int B_src, const int32_t* parent, int B, int g,
                               int t_cap, long row_bytes, hipStream_t s) {
    if (row_bytes % 16 == 0) gather_t<uint4>(k_src, v_src, k_dst, v_dst, lens, B_src, parent, B, g, t_cap, row_bytes, s);
    else if (row_bytes % 4 == 0) gather_t<uint32_t>(k_src, v_src, k_dst, v_dst, lens, B_src, parent, B, g, t_cap, row_bytes, s);
    else gather_t<uint16_t>(k_src, v_src, k_dst, v_dst, lens, B_src, parent, B, g, t_cap, row_bytes, s);
    return hipGetLastError();
}

}  // namespace kvc
