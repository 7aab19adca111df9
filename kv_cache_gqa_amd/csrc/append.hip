// append.hip -- write the new token's K/V into the cache.
//
// Follows "大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com) section
// 四 4.1 (the new K/V go after the past cache along the sequence axis) and
// "KV Cache 的增量解码" (zwjcode.cn) section 08 (the new position equals the
// current cache length) and section 10 (preallocated cache written in place).
// Paged placement follows "KV Cache 优化与注意力机制加速" (plumephp.com)
// section 4.3: physical block = table[b, pos / block_size], offset
// pos % block_size.
//
// One thread moves one vector of W bytes (16, 4 or 2 depending on the row
// size) of one (tensor, sequence, KV head, new token); the copy is
// bit-exact.  New token k of sequence b goes to position seq_lens[b] + k.
#include "kvc_device.h"

namespace kvc {

template <typename V>
__global__ void __launch_bounds__(256) append_kernel(
    const V* __restrict__ k_new, const V* __restrict__ v_new, V* __restrict__ k_cache,
    V* __restrict__ v_cache, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, const int32_t* __restrict__ seq_lens, int B, int g, int n, int vec_per_row,
    int capacity, int ring) {
    const long total = (long)B * g * n * vec_per_row;
    long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool is_v = t >= total;
    if (is_v) t -= total;
    if (t >= total) return;
    const int vec = (int)(t % vec_per_row);
    const long tok = t / vec_per_row;       // (b * g + j) * n + token
    const int k = (int)(tok % n);
    const long bj = tok / n;
    const int b = (int)(bj / g);
    const int j = (int)(bj % g);
    const long pos_l = (long)seq_lens[b] + k;
    if (pos_l < 0 || pos_l > 0x7fffffffL) return;
    const int pos = (int)pos_l;
    long row;
    if (block_table == nullptr) {
        if (ring) {
            row = bj * (long)capacity + pos % capacity;  // ring cache: slot pos mod capacity
        } else {
            if (pos >= capacity) return;
            row = bj * (long)capacity + pos;
        }
    } else {
        const int logical = pos / block_size;
        if (logical >= max_blocks) return;
        const int phys = block_table[(long)b * max_blocks + logical];
        if (phys < 0 || phys >= capacity) return;
        row = ((long)phys * g + j) * block_size + (pos % block_size);
    }
    const V* src = is_v ? v_new : k_new;
    V* dst = is_v ? v_cache : k_cache;
    dst[row * vec_per_row + vec] = src[tok * vec_per_row + vec];
}

template <typename V>
static void launch_append_t(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* block_table, int max_blocks, int block_size,
                            const int32_t* seq_lens_before, int B, int g, int n, int vpr,
                            int capacity, int ring, hipStream_t s) {
    const int threads = 256;
    const long total = 2L * B * g * n * vpr;
    append_kernel<V><<<dim3((unsigned)((total + threads - 1) / threads)), dim3(threads), 0, s>>>(
        (const V*)k_new, (const V*)v_new, (V*)k_cache, (V*)v_cache, block_table, max_blocks,
        block_size, seq_lens_before, B, g, n, vpr, capacity, ring);
}

hipError_t launch_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int32_t* block_table, int max_blocks, int block_size,
                         const int32_t* seq_lens_before, int B, int g, int n, int d, int capacity,
                         int ring, int elem_bytes, hipStream_t s) {
    const long row_bytes = (long)d * elem_bytes;
    if (row_bytes % 16 == 0)
        launch_append_t<uint4>(k_new, v_new, k_cache, v_cache, block_table, max_blocks, block_size,
                               seq_lens_before, B, g, n, (int)(row_bytes / 16), capacity, ring, s);
    else if (row_bytes % 4 == 0)
        launch_append_t<uint32_t>(k_new, v_new, k_cache, v_cache, block_table, max_blocks,
                                  block_size, seq_lens_before, B, g, n, (int)(row_bytes / 4),
                                  capacity, ring, s);
    else
        launch_append_t<uint16_t>(k_new, v_new, k_cache, v_cache, block_table, max_blocks,
                                  block_size, seq_lens_before, B, g, n, (int)(row_bytes / 2),
                                  capacity, ring, s);
    return hipGetLastError();
}

// FP8 E4M3 cache: new token k of sequence b, KV head j, element e: the
// bf16 value divided by the float32 scale (the KV head's, or with
// block_scales that of the (target block, KV head)), encoded (nearest code,
// ties to even, saturating at 448), written at position seq_lens[b] + k.
// One thread per (tensor, sequence, KV head, token, element).
__global__ void __launch_bounds__(256) append_fp8_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ block_table, int max_blocks,
    int block_size, const int32_t* __restrict__ seq_lens, int B, int g, int n, int d, int capacity,
    int ring, int block_scales) {
    const long total = (long)B * g * n * d;
    long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const bool is_v = t >= total;
    if (is_v) t -= total;
    if (t >= total) return;
    const int e = (int)(t % d);
    const long tok = t / d;  // (b * g + j) * n + token
    const int k = (int)(tok % n);
    const long bj = tok / n;
    const int b = (int)(bj / g);
    const int j = (int)(bj % g);
    const long pos_l = (long)seq_lens[b] + k;
    if (pos_l < 0 || pos_l > 0x7fffffffL) return;
    const int pos = (int)pos_l;
    long row;
    long sidx = j;  // the scale: per KV head, or per (block, KV head)
    if (block_table == nullptr) {
        if (ring) {
            row = bj * (long)capacity + pos % capacity;
        } else {
            if (pos >= capacity) return;
            row = bj * (long)capacity + pos;
        }
    } else {
        const int logical = pos / block_size;
        if (logical >= max_blocks) return;
        const int phys = block_table[(long)b * max_blocks + logical];
        if (phys < 0 || phys >= capacity) return;
        row = ((long)phys * g + j) * block_size + (pos % block_size);
        if (block_scales) sidx = (long)phys * g + j;
    }
    const float x = __uint_as_float((uint32_t)(is_v ? v_new : k_new)[tok * d + e] << 16);
    const float sc = is_v ? v_scale[sidx] : k_scale[sidx];
    (is_v ? v_cache : k_cache)[row * d + e] = (uint8_t)e4m3_encode(x / sc);
}

hipError_t launch_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int max_blocks, int block_size,
                             const int32_t* seq_lens_before, int B, int g, int n, int d,
                             int capacity, int ring, int block_scales, hipStream_t s) {
    const long total = 2L * B * g * n * d;
    append_fp8_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
        (const uint16_t*)k_new, (const uint16_t*)v_new, (uint8_t*)k_cache, (uint8_t*)v_cache,
        k_scale, v_scale, block_table, max_blocks, block_size, seq_lens_before, B, g, n, d,
        capacity, ring, block_scales);
    return hipGetLastError();
}

}  // namespace kvc
