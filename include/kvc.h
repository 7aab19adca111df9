/*
 * kvc.h -- C ABI of libkvc: single-token decode attention over a KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * One decode step of causal self-attention for a batch of sequences:
 *   1. kvc_append writes the new token's K and V of every (sequence, KV head)
 *      into the cache at position seq_lens_before[b];
 *   2. kvc_decode_attention / kvc_decode_attention_paged compute, for every
 *      sequence b and query head i, with KV head j = floor(i * g / h),
 *        out[b,i,:] = softmax(scale * q[b,i,:] . K[b,j,p,:]) V[b,j,p,:]
 *      over positions p < seq_lens[b], and lse[b,i] = ln sum_p exp(score_p).
 *
 * Pages that define the operations (cited by title and section):
 *   [P1] "大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com): section 二
 *        (cache K_t, V_t and append them each step), section 三 3.1-3.3 (MHA,
 *        MQA, GQA; head map j = floor(i/m) = floor(i*g/h) with m = h/g
 *        consecutive query heads per group), section 四 4.1 (concatenate the
 *        new K/V after the past cache along the sequence axis, then scaled
 *        dot-product attention; h must be divisible by g).
 *   [P2] "从KV cache共享到批量调度：注意力机制下的隔离问题与口令实验"
 *        (0539edu.com): section 2.1 (scale 1/sqrt(d_k)), section 3.1 (paged
 *        blocks; the block table lives on the GPU and the kernel computes
 *        addresses itself), section 3.3 (variable lengths; a length-0 entry
 *        must not corrupt the batch).
 *   [P3] "每生成一个词为何又重算全文？KV Cache 的增量解码" (zwjcode.cn):
 *        section 02 (per-step shapes q [N,H,1,d], cache [N,H,t,d]), section
 *        08 (the new token's position is the current cache length), section
 *        10 (preallocated static cache; unwritten slots are invisible).
 *   [P4] "KV Cache 优化与注意力机制加速：FlashAttention / PagedAttention"
 *        (plumephp.com): section 2.2-2.3 (online softmax statistics m, l and
 *        the log-sum-exp L = m + log l returned with O), section 2.5
 *        (parallelism over the sequence dimension), section 4.2-4.3 (block
 *        of 16 tokens, block table, logical block = pos / block_size,
 *        offset = pos % block_size).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and keeps no state besides cached answers to
 *     device queries (compute-unit count, resident work-groups per kernel),
 *     guarded by a lock: entry points may be called from several host
 *     threads.  The current HIP device must be the one holding the data.
 *     Outputs must not alias inputs.
 *   - Every launch is asynchronous on the caller's `stream`; no entry point
 *     synchronises the host.  Validation of the host-side arguments happens
 *     before any HIP call and needs no GPU.
 *   - dtype: KVC_F32 or KVC_BF16, shared by q, the caches and k/v_new.
 *     out and lse are always float32.
 *   - Alignment: tensors of elements (q, caches and pools, k_new / v_new,
 *     out, the workspace) must start on a 16-byte boundary, because the
 *     kernels move them in 16-byte vectors; arrays of int32 or float32
 *     values (seq_lens, block tables, lse, scales, pairs, parents) on a
 *     4-byte boundary.  Any other pointer gives KVC_ERR_INVALID before any
 *     HIP call.  Allocations from hipMalloc or PyTorch's allocator satisfy
 *     both; a view at an element offset may not.
 *   - Device-side integers (seq_lens, block_table) are trusted.  They are
 *     clamped inside the kernels so that a bad value cannot fault the GPU:
 *     lengths to [0, capacity], physical block ids to [0, num_blocks).  A
 *     clamped value gives unspecified (but in-bounds) results.
 *   - Return value: a kvc_status.  No C++ exception crosses the ABI.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_INVALID = 1,      /* null pointer, non-positive size, h % g != 0, bad block size,
                                 num_splits < -1 */
    KVC_ERR_UNSUPPORTED = 2,  /* dtype or head_dim not built (head_dim must be 1..256) */
    KVC_ERR_WORKSPACE = 3,    /* workspace missing or smaller than kvc_decode_workspace_bytes */
    KVC_ERR_HIP = 4,          /* a HIP launch reported an error */
    KVC_ERR_SCRATCH = 5       /* kvc_append_decode_attention_noalloc: the split needs more
                                 than kvc_noalloc_scratch_bytes() of scratch */
} kvc_status;

/* KVC_FP8_E4M3 is for the planning queries only (kvc_decode_plan,
 * kvc_decode_workspace_bytes, kvc_decode_launch_shape): bf16 queries over an
 * FP8 E4M3 cache, the *_fp8 entry points.  Plans and workspaces are those of
 * KVC_BF16; the launch shape is the FP8 kernels' own. */
typedef enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1, KVC_FP8_E4M3 = 2 } kvc_dtype;

/* Library version, (major << 16) | (minor << 8) | patch. */
int kvc_version(void);

/* Human-readable text of a kvc_status value (static string). */
const char* kvc_status_string(int status);

/*
 * kvc_append -- write the new token's K/V into the cache ([P1] 二 and 四 4.1
 * concat; [P3] section 08 position = current length; [P4] 4.3 block lookup).
 *
 *   k_new, v_new      [B, g, d] of dtype
 *   k_cache, v_cache  contiguous [B, g, capacity, d] when block_table == NULL;
 *                     else pools [capacity, g, block_size, d] (capacity = number
 *                     of physical blocks)
 *   block_table       NULL, or device int32 [B, max_blocks]: physical block id
 *                     of each logical block of each sequence
 *   seq_lens_before   device int32 [B]: cache length before this step = the
 *                     slot written.  Not modified.
 *   For every b < B and j < g: with pos = seq_lens_before[b], the d elements
 *   of k_new[b,j,:] are copied byte-exactly to K[b, j, pos, :] (contiguous), or
 *   to pool[block_table[b, pos / block_size], j, pos % block_size, :] (paged),
 *   and likewise for V.  Nothing else is written.  Positions outside the
 *   capacity (pos < 0, pos >= capacity, logical block >= max_blocks, or a
 *   negative / out-of-range physical id) are skipped.
 *   The caller makes sure that the target block is allocated and private to
 *   the sequence (copy-on-write is the caller's policy).
 */
int kvc_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
               const int32_t* block_table, int max_blocks, int block_size,
               const int32_t* seq_lens_before, int B, int g, int d, int capacity,
               int dtype, hipStream_t stream);

/*
 * Work split.  The attention of one (sequence, KV head) over positions
 * [0, L) may be cut into position ranges whose partial (O, lse) results
 * combine exactly by log-sum-exp ([P4] 2.2-2.5).  Every work-group serves
 * all m = h/g query heads of its KV head, so every K/V byte is read once.
 * num_splits selects the split:
 *
 *   0 (automatic)
 *     contiguous cache: chunks (KVC_SPLIT_AUTO_CHUNKS) chosen at launch from
 *       the device's resident work-group slots (compute units x work-groups
 *       per CU that the kernel's registers and LDS allow).  For the MFMA
 *       kernel with 4 <= h/g <= 16, when there are at least as many
 *       (sequence, KV head) units as slots of an 8-wavefront work-group
 *       (and they fill at least 7/8 of the slot rounds), each unit is one
 *       8-wavefront work-group: one chunk, no merge.  Otherwise
 *       4-wavefront work-groups take ceil(slots / units) chunks per unit,
 *       so that they fill the slots once.
 *     paged cache: stream mode (KVC_SPLIT_STREAM, below), which stays
 *       balanced whatever the mix of sequence lengths, for the head_dim-128
 *       decode kernels (up to 32 query rows per KV head; FP8 caches up to
 *       16) and for the multi-row kernel with bf16 rows of 256 dims and at
 *       most 16 rows per KV head; other shapes take chunks as on a
 *       contiguous cache (the multi-row kernel's walk pays a prologue per
 *       segment, which only wide rows repay; the FP8 decode kernel with two
 *       query tiles measured faster chunked).
 *   KVC_SPLITS_STREAM (-1): stream mode.  A persistent grid of as many
 *     work-groups as the device keeps resident; all (sequence, KV head)
 *     ranges are laid end to end and every work-group takes an equal share
 *     of the positions.  The head_dim-128 decode kernels take it on any
 *     layout (FP8 pools with per-block scales up to 16 query rows per KV
 *     head; with more they take chunks); the multi-row kernel on paged
 *     pools when the rows of a KV head fit one 4-wavefront work-group (64
 *     rows; 128 below head_dim 256).
 *   n > 0: chunks of chunk_len positions (a multiple of 32) so that about n
 *     chunks cover max_seq_len (KVC_SPLIT_CHUNKS); each (chunk, sequence, KV
 *     head) is one work-group.
 * Stream mode also needs B <= 1024 and B * g * max_seq_len < 2^40;
 * otherwise the automatic choice is chunks.
 * When results are split, partials go to the workspace and a second kernel
 * merges them.
 *
 * kvc_decode_plan reports the mode and, for KVC_SPLIT_CHUNKS, chunk_len and
 * the chunk count (0 for the other modes).  kvc_decode_workspace_bytes
 * returns the workspace the decode call needs for the same arguments (0 if
 * none); for the automatic chunk count it covers the largest count any
 * device can select, and for automatic splits of a paged cache both the
 * stream schedule and the chunks a sliding window uses.  max_seq_len is t_cap for the contiguous entry point
 * and max_blocks * block_size for the paged one; paged is 0 or 1.  Both are
 * pure host arithmetic.
 */
enum { KVC_SPLITS_STREAM = -1 };
enum { KVC_SPLIT_CHUNKS = 0, KVC_SPLIT_STREAM = 1, KVC_SPLIT_AUTO_CHUNKS = 2 };
int kvc_decode_plan(int B, int h, int g, int d, int dtype, int max_seq_len, int num_splits,
                    int paged, int* mode, int* chunk_len, int* num_chunks);
size_t kvc_decode_workspace_bytes(int B, int h, int g, int d, int dtype, int max_seq_len,
                                  int num_splits, int paged);
/*
 * The launch kvc_decode_attention (paged = 0, max_seq_len = t_cap) or
 * kvc_decode_attention_paged (paged = 1, max_seq_len = max_blocks *
 * block_size) makes on the current device for these arguments: wavefronts
 * per work-group, work-groups of the decode kernel, and for the chunked
 * modes the chunk length and chunk count per (sequence, KV head) (0 in stream
 * mode).  Resolves the automatic choices, which query the device's
 * occupancy, so it needs a current HIP device.  Returns KVC_OK, or the
 * validation status the decode call would return.
 */
int kvc_decode_launch_shape(int B, int h, int g, int d, int dtype, int max_seq_len,
                            int num_splits, int paged, int* waves, int* num_wgs,
                            int* chunk_len, int* num_chunks);
/*
 * The same two queries for the calls with n query tokens per sequence and a
 * sliding window W (0 = none): the _multi, _window and FP8 _fp8_multi /
 * _fp8_window calls, whose plans can differ from the single-token call's
 * (their kernels' registers, and an automatic split of a paged FP8 pool with
 * n > 1 takes chunks).  h is query heads (not h * n); capacity is t_cap
 * (contiguous; ring caches too) or max_blocks * block_size (paged); the
 * plan covers min(capacity, W + n - 1) positions with a window, as the
 * calls do.  dtype KVC_FP8_E4M3 stands for FP8 caches with a scale per KV
 * head.  n = 1 and W = 0 give kvc_decode_plan / kvc_decode_launch_shape
 * with max_seq_len = capacity.  Returns KVC_OK, KVC_ERR_INVALID (n <= 0,
 * W < 0, a negative capacity, or as the single-token queries) or
 * KVC_ERR_UNSUPPORTED (h * n > 65535, or as the single-token queries).
 */
int kvc_decode_plan_multi(int B, int h, int g, int d, int n, int window, int dtype, int capacity,
                          int num_splits, int paged, int* mode, int* chunk_len, int* num_chunks);
int kvc_decode_launch_shape_multi(int B, int h, int g, int d, int n, int window, int dtype,
                                  int capacity, int num_splits, int paged, int* waves,
                                  int* num_wgs, int* chunk_len, int* num_chunks);

/*
 * kvc_decode_attention -- decode attention over a contiguous cache.
 *
 *   q            [B, h, d] of dtype: one query per sequence and head
 *   k_cache      [B, g, t_cap, d] of dtype
 *   v_cache      [B, g, t_cap, d] of dtype
 *   seq_lens     device int32 [B]: number of attended positions (after the
 *                append), 0..t_cap.  Positions >= seq_lens[b] are never read.
 *   B, h, g, d   batch, query heads, KV heads (h % g == 0), head dim
 *   scale        multiplies every q.k (usually 1/sqrt(d))
 *   num_splits   see "Work split"
 *   workspace    device buffer of at least kvc_decode_workspace_bytes(B, h, g,
 *                d, dtype, t_cap, num_splits, 0) bytes (may be NULL when that
 *                is 0); no initialisation needed.  Calls that share a
 *                workspace must not overlap in time (same stream, or
 *                synchronised).
 *   out          [B, h, d] float32; lse [B, h] float32 (natural log).
 *   A sequence of length 0 gets out = 0 and lse = -inf.
 */
int kvc_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, int B, int h, int g, int d, int t_cap,
                         float scale, int dtype, int num_splits,
                         void* workspace, size_t workspace_bytes,
                         float* out, float* lse, hipStream_t stream);

/*
 * kvc_decode_attention_paged -- decode attention over a paged cache.
 *
 *   k_pool, v_pool  [num_blocks, g, block_size, d] of dtype: physical blocks
 *   block_table     device int32 [B, max_blocks]; entry (b, n) is the
 *                   physical block holding positions [n*block_size,
 *                   (n+1)*block_size) of sequence b.  Entries past the last
 *                   block a sequence uses are never read.
 *   block_size      power of two, 8..256
 *   num_blocks      blocks in each pool; num_blocks * g * block_size must
 *                   not exceed 2^32 - 1 (KVC_ERR_UNSUPPORTED otherwise)
 *   seq_lens        device int32 [B], 0..max_blocks*block_size
 *   other arguments as kvc_decode_attention; the workspace size uses
 *   max_seq_len = max_blocks * block_size and paged = 1.
 */
int kvc_decode_attention_paged(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, int max_blocks, int block_size,
                               int num_blocks, const int32_t* seq_lens,
                               int B, int h, int g, int d, float scale, int dtype,
                               int num_splits, void* workspace, size_t workspace_bytes,
                               float* out, float* lse, hipStream_t stream);

/*
 * kvc_append_decode_attention / kvc_append_decode_attention_paged -- the
 * whole decode step in one call: the same result as kvc_append(k_new, v_new,
 * ..., seq_lens_before, ...) followed by kvc_decode_attention[_paged] with
 * seq_lens = seq_lens_before + 1 (each sequence attends to the positions it
 * had and to the new token, which it sees last: [P1] 4.1, [P3] 04 and 08).
 *
 *   q, caches, block table, B, h, g, d, t_cap, scale, dtype, num_splits,
 *   workspace, out, lse, stream: as for the decode entry points; the
 *     workspace size is kvc_decode_workspace_bytes of the same shapes.
 *   k_new, v_new      [B, g, d] of dtype: the new token's K and V.
 *   seq_lens_before   device int32 [B]: cache length before the step; not
 *                     modified.  The new token goes to that position.
 *
 * The decode kernels read the new token from k_new / v_new and write it into
 * its cache slot themselves (one launch, plus the merge when results are
 * split).  Out-of-range positions are skipped as kvc_append skips them (a
 * length at or past the capacity attends to the capacity and appends
 * nothing).  One difference from the two-call sequence: when the paged
 * table entry of the new position is not a valid block, kvc_append writes
 * nothing and a following decode reads whatever block the clamped entry
 * names; the fused call also writes nothing but attends to the new token's
 * true K/V.  k_new, v_new must not alias the caches.  Same status codes as
 * the decode entry points.
 */
int kvc_append_decode_attention(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* seq_lens_before,
                                int B, int h, int g, int d, int t_cap, float scale, int dtype,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream);
int kvc_append_decode_attention_paged(const void* q, const void* k_new, const void* v_new,
                                      void* k_pool, void* v_pool, const int32_t* block_table,
                                      int max_blocks, int block_size, int num_blocks,
                                      const int32_t* seq_lens_before, int B, int h, int g, int d,
                                      float scale, int dtype, int num_splits, void* workspace,
                                      size_t workspace_bytes, float* out, float* lse,
                                      hipStream_t stream);

/*
 * kvc_append_decode_attention_noalloc -- for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): kvc_append_decode_attention with no
 * workspace argument.  Same arguments otherwise, same kernels, same results.
 *
 * When the call's plan splits positions, the partial results go to a
 * static device buffer of the library (kvc_noalloc_scratch_bytes() = 16 MiB,
 * one per GPU, held from the first use of the library on that GPU until the
 * process ends) instead of a workspace; nothing is allocated, and the
 * buffer needs no clearing (every call writes the partials it reads).  A
 * call whose plan needs more (kvc_decode_workspace_bytes(B, h, g, d, dtype,
 * t_cap, num_splits, 0) > 16 MiB) returns KVC_ERR_SCRATCH before any HIP
 * call; choose fewer splits, or call kvc_append_decode_attention with a
 * workspace.  All calls on one GPU share the buffer: calls that may overlap
 * in time on one GPU (different streams, or several host threads) race on
 * it and must be serialised by the caller.  The first call on a device
 * queries the buffer's device address (hipGetSymbolAddress) with that
 * device current.
 */
int kvc_append_decode_attention_noalloc(const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache,
                                        const int32_t* seq_lens_before, int B, int h, int g, int d,
                                        int t_cap, float scale, int dtype, int num_splits,
                                        float* out, float* lse, hipStream_t stream);
size_t kvc_noalloc_scratch_bytes(void);

/*
 * Several new tokens per sequence at once: kvc_decode_attention_multi[_paged]
 * and kvc_append_decode_attention_multi[_paged] (a prefill of new tokens
 * after a cached prefix, [P1] 5.2; draft tokens checked in one pass, [P4]
 * 5.3).  Query token t of sequence b sits at position P_b + t, where P_b is
 * the number of positions cached before the n new tokens, and attends to
 * positions 0 .. P_b + t: the causal mask of the whole sequence aligned to
 * its bottom-right corner ([P3] 13 warns that a non-square is_causal mask is
 * aligned otherwise).
 *
 *   q      [B, h, n, d] of dtype: token t of head i at q[b, i, t, :]
 *   out    [B, h, n, d] fp32;  lse [B, h, n] fp32
 *   n      new tokens per sequence, >= 1; h * n <= 65535
 *   kvc_decode_attention_multi[_paged]: the n tokens are already in the
 *     cache and seq_lens[b] = P_b + n (the length after them).
 *   kvc_append_decode_attention_multi[_paged]: k_new, v_new [B, g, n, d];
 *     seq_lens_before[b] = P_b (not modified).  Token t is written at
 *     position P_b + t (skipped outside the capacity, as kvc_append skips),
 *     and the tokens attend as above, in one launch plus the merge when the
 *     results are split.
 *   Token t sees min(P_b + t + 1, capacity) positions (0 if negative).
 * Everything else is as for the single-token calls, which are the case
 * n = 1.  The workspace is kvc_decode_workspace_bytes(B, h * n, g, d, ...);
 * kvc_decode_plan_multi and kvc_decode_launch_shape_multi give these calls'
 * plans (kvc_decode_plan and kvc_decode_launch_shape, taking h * n as h,
 * describe a single-token call with as many rows).
 * Kernels by rows per KV head, r = (h / g) * n, for bf16 with d = 128: r <= 3
 * the VALU kernel; 4 <= r <= 32 the matrix-core decode kernel; r > 32 the
 * multi-row matrix-core kernel, which stages each K/V tile in LDS once for
 * up to 256 rows (ceil(r / 256) work-groups per unit, 128 at d = 80, 96 and
 * 256).  bf16 with d = 64, 80, 96 or 256: the multi-row kernel for any r.
 * fp32 or other head dims take the generic kernel for any r.
 */
int kvc_decode_attention_multi(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, int B, int h, int g, int d, int n,
                               int t_cap, float scale, int dtype, int num_splits, void* workspace,
                               size_t workspace_bytes, float* out, float* lse, hipStream_t stream);
int kvc_decode_attention_multi_paged(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                     int d, int n, float scale, int dtype, int num_splits,
                                     void* workspace, size_t workspace_bytes, float* out,
                                     float* lse, hipStream_t stream);
int kvc_append_decode_attention_multi(const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache,
                                      const int32_t* seq_lens_before, int B, int h, int g, int d,
                                      int n, int t_cap, float scale, int dtype, int num_splits,
                                      void* workspace, size_t workspace_bytes, float* out,
                                      float* lse, hipStream_t stream);
int kvc_append_decode_attention_multi_paged(const void* q, const void* k_new, const void* v_new,
                                            void* k_pool, void* v_pool,
                                            const int32_t* block_table, int max_blocks,
                                            int block_size, int num_blocks,
                                            const int32_t* seq_lens_before, int B, int h, int g,
                                            int d, int n, float scale, int dtype, int num_splits,
                                            void* workspace, size_t workspace_bytes, float* out,
                                            float* lse, hipStream_t stream);

/*
 * Sliding window: kvc_decode_attention_window[_paged] and
 * kvc_append_decode_attention_window[_paged].  As the _multi calls (n new
 * tokens per sequence; n = 1 is single-token decode), with a window W >= 1:
 * the token at position x attends only to positions max(0, x + 1 - W) .. x,
 * the last W including itself ([P4] 5.2: attention within a local window to
 * the left; [P3] 10: a window cache keeps only the most recent W positions,
 * so its memory is bounded).  W = 0 means no window (the _multi calls).
 * Only the positions some token sees are read: a paged table may hold -1 for
 * blocks wholly before every window.  With num_splits = 0 a windowed paged
 * call splits into chunks (its ranges are nearly equal), not stream mode.
 *
 *   ring (contiguous calls only): 1 = the cache is a ring of t_cap slots,
 *     position p in slot p mod t_cap, positions not limited by t_cap.
 *     Requires W >= 1 and W + n - 1 <= t_cap (so that writing the n new
 *     tokens never overwrites a position some token sees); KVC_ERR_INVALID
 *     otherwise.  0 = positions are slots, limited by t_cap as in the other
 *     calls.
 *   window  0 or W >= 1; negative is KVC_ERR_INVALID.
 * Workspace: kvc_decode_workspace_bytes(B, h * n, g, d, dtype, L, ...) with
 * L = min(W + n - 1, capacity) for W > 0, else the capacity; any larger L
 * gives a workspace that is also large enough.
 */
int kvc_decode_attention_window(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                int t_cap, int window, int ring, float scale, int dtype,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream);
int kvc_decode_attention_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, int max_blocks, int block_size,
                                      int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                      int d, int n, int window, float scale, int dtype,
                                      int num_splits, void* workspace, size_t workspace_bytes,
                                      float* out, float* lse, hipStream_t stream);
int kvc_append_decode_attention_window(const void* q, const void* k_new, const void* v_new,
                                       void* k_cache, void* v_cache,
                                       const int32_t* seq_lens_before, int B, int h, int g, int d,
                                       int n, int t_cap, int window, int ring, float scale,
                                       int dtype, int num_splits, void* workspace,
                                       size_t workspace_bytes, float* out, float* lse,
                                       hipStream_t stream);
int kvc_append_decode_attention_window_paged(const void* q, const void* k_new, const void* v_new,
                                             void* k_pool, void* v_pool,
                                             const int32_t* block_table, int max_blocks,
                                             int block_size, int num_blocks,
                                             const int32_t* seq_lens_before, int B, int h, int g,
                                             int d, int n, int window, float scale, int dtype,
                                             int num_splits, void* workspace,
                                             size_t workspace_bytes, float* out, float* lse,
                                             hipStream_t stream);

/*
 * FP8 caches ([P4] 2.5: FP8 attention; [P3] 14: low-bit K/V halve the
 * bytes a bandwidth-bound step reads, at a cost in error): kvc_append_fp8,
 * kvc_decode_attention_fp8[_paged] and kvc_append_decode_attention_fp8[_paged].
 *
 *   Caches hold OCP FP8 E4M3 codes, one byte per element, in the layouts of
 *   the bf16 calls ([B, g, t_cap, d] or pools [NB, g, bs, d]).
 *   k_scale, v_scale  device float32 [g]: one scale per KV head.
 *   q, k_new, v_new   bf16, as in the bf16 calls; out, lse float32.
 *   A new element x (bf16) is stored as the code of the float32 quotient
 *   x / scale: the nearest E4M3 value, ties to the even code, magnitudes
 *   above 448 saturating to 448, NaN to S.1111.111, the sign kept.
 *   Attention is computed over the dequantised values code * scale (codes
 *   are widened to bf16 exactly; the K scale is folded into the score scale
 *   and the V scale into the output).
 *   The one-call step attends to the new token's codes (what
 *   kvc_append_fp8 stores), so it gives what kvc_append_fp8 followed by
 *   kvc_decode_attention_fp8[_paged] gives; as with bf16, when the new
 *   position's paged table entry is not a valid block nothing is written
 *   but the token is still attended to.
 * Everything else (validation, splits, workspace from
 * kvc_decode_workspace_bytes with dtype KVC_BF16, positions, status codes)
 * is as in the bf16 single-token calls.  Kernels: at d = 128 as for bf16
 * (up to 3 rows per KV head the VALU kernel, 4-32 the matrix-core decode
 * kernel, more the multi-row kernel, which widens the codes to bf16 as it
 * stages each tile in LDS); at d = 64, 80, 96 and 256 the multi-row kernel
 * for any row count; other head dims the generic kernel.
 */
int kvc_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   int max_blocks, int block_size, const int32_t* seq_lens_before, int B, int g,
                   int d, int capacity, hipStream_t stream);
int kvc_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int B, int h, int g, int d, int t_cap, float scale, int num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             hipStream_t stream);
int kvc_decode_attention_fp8_paged(const void* q, const void* k_pool, const void* v_pool,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, int max_blocks, int block_size,
                                   int num_blocks, const int32_t* seq_lens, int B, int h, int g,
                                   int d, float scale, int num_splits, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream);
int kvc_append_decode_attention_fp8(const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* seq_lens_before, int B,
                                    int h, int g, int d, int t_cap, float scale, int num_splits,
                                    void* workspace, size_t workspace_bytes, float* out,
                                    float* lse, hipStream_t stream);
int kvc_append_decode_attention_fp8_paged(const void* q, const void* k_new, const void* v_new,
                                          void* k_pool, void* v_pool, const float* k_scale,
                                          const float* v_scale, const int32_t* block_table,
                                          int max_blocks, int block_size, int num_blocks,
                                          const int32_t* seq_lens_before, int B, int h, int g,
                                          int d, float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream);

/*
 * FP8 caches with several new tokens per sequence ([P1] 5.2, [P4] 5.3) and
 * sliding windows ([P4] 5.2, [P3] 10), the FP8 forms of the _multi and
 * _window calls: kvc_decode_attention_fp8_multi[_paged],
 * kvc_append_decode_attention_fp8_multi[_paged] and the _fp8_window
 * versions of both, which take a window W (0 = none, the same as _multi)
 * and, contiguous only, ring.
 *
 *   Shapes, positions, the bottom-right causal alignment, windows, ring
 *   slots, capacity clamping and workspaces as in the bf16 _multi / _window
 *   calls (q [B, h, n, d] and out [B, h, n, d], lse [B, h, n]; the workspace
 *   is kvc_decode_workspace_bytes(B, h * n, g, d, KVC_BF16, L, ...) with L as
 *   for the bf16 window calls).  Caches and scales as in the FP8 single-
 *   token calls: OCP E4M3 codes, k_scale / v_scale float32 [g], q, k_new,
 *   v_new bf16 [B, g, n, d].
 *   The appending calls write the n tokens' codes (each the code of the
 *   float32 quotient x / scale, as kvc_append_fp8 encodes) and attend to
 *   those codes' values, so they give what writing the codes and then the
 *   non-appending call gives.
 *   Attention is over the dequantised values code * scale.
 *   Splits: with n > 1 an automatic split (num_splits = 0) of a paged pool
 *   takes chunks, not the stream grid (measured faster there), as
 *   kvc_decode_plan_multi reports.
 */
int kvc_decode_attention_fp8_multi(const void* q, const void* k_cache, const void* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                   int t_cap, float scale, int num_splits, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream);
int kvc_decode_attention_fp8_multi_paged(const void* q, const void* k_pool, const void* v_pool,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_table, int max_blocks,
                                         int block_size, int num_blocks, const int32_t* seq_lens,
                                         int B, int h, int g, int d, int n, float scale,
                                         int num_splits, void* workspace, size_t workspace_bytes,
                                         float* out, float* lse, hipStream_t stream);
int kvc_append_decode_attention_fp8_multi(const void* q, const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache, const float* k_scale,
                                          const float* v_scale, const int32_t* seq_lens_before,
                                          int B, int h, int g, int d, int n, int t_cap,
                                          float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream);
int kvc_append_decode_attention_fp8_multi_paged(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens_before, int B, int h, int g, int d,
    int n, float scale, int num_splits, void* workspace, size_t workspace_bytes, float* out,
    float* lse, hipStream_t stream);
int kvc_decode_attention_fp8_window(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* seq_lens, int B, int h, int g, int d, int n,
                                    int t_cap, int window, int ring, float scale, int num_splits,
                                    void* workspace, size_t workspace_bytes, float* out, float* lse,
                                    hipStream_t stream);
int kvc_decode_attention_fp8_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                          const float* k_scale, const float* v_scale,
                                          const int32_t* block_table, int max_blocks,
                                          int block_size, int num_blocks, const int32_t* seq_lens,
                                          int B, int h, int g, int d, int n, int window,
                                          float scale, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* out, float* lse,
                                          hipStream_t stream);
int kvc_append_decode_attention_fp8_window(const void* q, const void* k_new, const void* v_new,
                                           void* k_cache, void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* seq_lens_before,
                                           int B, int h, int g, int d, int n, int t_cap,
                                           int window, int ring, float scale, int num_splits,
                                           void* workspace, size_t workspace_bytes, float* out,
                                           float* lse, hipStream_t stream);
int kvc_append_decode_attention_fp8_window_paged(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens_before, int B, int h, int g, int d,
    int n, int window, float scale, int num_splits, void* workspace, size_t workspace_bytes,
    float* out, float* lse, hipStream_t stream);

/*
 * FP8 paged pools with a scale per (physical block, KV head) ([P3] 14 and
 * [P4] 2.5: low-bit K/V; a scale per page lets each block follow the range
 * of the values it holds): k_scale, v_scale are device float32 [num_blocks,
 * g]; the value of a stored code in block blk, KV head j is code *
 * scale[blk, j].  Choosing a block's scale (calibration) is the caller's
 * business; it must be set before tokens are written into the block.
 *
 * kvc_append_fp8_paged_block_scaled -- n new tokens per sequence (k_new,
 *   v_new bf16 [B, g, n, d]): token t of sequence b is written at position
 *   seq_lens_before[b] + t as the codes of x / scale[blk, j] of its target
 *   block (nearest code, ties to even, saturating, as kvc_append_fp8).
 *   Positions outside the table or whose entry is not a valid block are
 *   skipped.
 * kvc_decode_attention_fp8_paged_block_scaled -- attention over such a
 *   pool for n query tokens per sequence (q bf16 [B, h, n, d], out
 *   [B, h, n, d], lse [B, h, n]), with an optional sliding window (window 0 =
 *   none), and with k_new, v_new (bf16 [B, g, n, d]) also the append (one
 *   launch; seq_lens are then the lengths before the step, else the lengths
 *   including the n tokens).  Both or neither of k_new, v_new.  Positions,
 *   masks, splits and the workspace (kvc_decode_workspace_bytes(B, h * n, g,
 *   d, KVC_BF16, L, num_splits, 1) with L = min(W + n - 1, max_blocks *
 *   block_size) for W > 0, else max_blocks * block_size) as in the bf16
 *   paged _multi / _window calls.  Attention is over the dequantised values:
 *   each score uses the K scale of its position's block, and each V row is
 *   weighted by its block's V scale; a new token whose table entry is not a
 *   valid block is attended with the scales of the clamped entry.  Kernels:
 *   at d = 128 up to 3 rows per KV head the VALU kernel, 4-32 the
 *   matrix-core decode kernel, more as 32-row slices of it (each reading
 *   the unit's K/V); other head dims the generic kernel.
 */
int kvc_append_fp8_paged_block_scaled(const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, int max_blocks, int block_size,
                                      int num_blocks, const int32_t* seq_lens_before, int B, int g,
                                      int d, int n, hipStream_t stream);
int kvc_decode_attention_fp8_paged_block_scaled(
    const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const float* k_scale, const float* v_scale, const int32_t* block_table, int max_blocks,
    int block_size, int num_blocks, const int32_t* seq_lens, int B, int h, int g, int d, int n,
    int window, float scale, int num_splits, void* workspace, size_t workspace_bytes, float* out,
    float* lse, hipStream_t stream);

/*
 * Block operations for shared and re-ranked caches ([P4] 4.3: requests that
 * share a prompt fork its block table and point at the same physical
 * blocks; before one of them writes into a shared block, the block is copied
 * and that request's table is pointed at the copy; [P2] 3.2: shared blocks
 * are read-only, copied on write; [P3] 11: after beams are re-ranked, each
 * beam's cache must follow its chosen parent).  The host keeps reference
 * counts and allocates blocks; these calls move bytes and table rows,
 * bit-exactly, asynchronously on `stream`.
 *
 * kvc_copy_blocks: for each of the num_pairs pairs (src, dst) of device
 *   int32 pairs[num_pairs][2], copy physical block src of both pools
 *   [num_blocks, g, block_size, d] (all KV heads) to block dst.  Pairs that
 *   name a block outside [0, num_blocks), and src == dst, are skipped.  No
 *   dst may appear twice or also be a src (the copies run concurrently).
 * kvc_fork_block_tables: block_table_out[b, :] = block_table[parent[b], :]
 *   and seq_lens_out[b] = seq_lens[parent[b]] for b < B (tables
 *   [B_src, max_blocks] -> [B, max_blocks]); a parent outside [0, B_src)
 *   gives a row of -1 and length 0.  Outputs must not alias the inputs.
 * kvc_gather_cache: contiguous caches [B_src, g, t_cap, d] -> [B, g, t_cap,
 *   d]: positions p < seq_lens[parent[b]] (clamped to [0, t_cap]) of
 *   sequence b are copied from sequence parent[b]; other positions of the
 *   destination are not written; nothing is written for a parent outside
 *   [0, B_src).  The two destinations must be distinct buffers, distinct
 *   from both sources.
 * Status: KVC_ERR_INVALID for bad sizes, null pointers or aliasing,
 *   KVC_ERR_UNSUPPORTED for other dtypes or t_cap > 4194240 (gather).
 */
int kvc_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                    int num_blocks, int g, int block_size, int d, int dtype, hipStream_t stream);
int kvc_fork_block_tables(const int32_t* block_table, const int32_t* seq_lens, int B_src,
                          int max_blocks, const int32_t* parent, int B, int32_t* block_table_out,
                          int32_t* seq_lens_out, hipStream_t stream);
int kvc_gather_cache(const void* k_src, const void* v_src, const int32_t* seq_lens, int B_src,
                     const int32_t* parent, int B, void* k_dst, void* v_dst, int g, int t_cap,
                     int d, int dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
