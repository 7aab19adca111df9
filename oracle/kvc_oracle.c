/*
 * kvc_oracle.c -- plain, slow, CPU fp64 reference for single-token decode
 * attention over a KV cache.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the CPU-baseline leg of the benchmark call it; the GPU library
 * never links, includes or calls anything in this directory, and this file
 * shares no code, header or table with the GPU library.
 *
 * Pages this file follows (cited by title and section):
 *   [P1] "大语言模型研究15——注意力机制优化之KV缓存" (limoncc.com)
 *        section 三 3.3 (GQA head map j = floor(i*g/h)), section 四 4.1
 *        (the GQAttentionWithCache listing: concat the new K/V after the past
 *        cache, then scaled dot-product softmax attention).
 *   [P3] "每生成一个词为何又重算全文？KV Cache 的增量解码" (zwjcode.cn)
 *        section 02 (per-step shapes: q [N,H,1,d], cache [N,H,t,d],
 *        scores [N,H,1,t]), section 04 (d=1 worked example), section 08
 *        (the new token's position equals the current cache length),
 *        section 10 (unwritten slots must be invisible to the query).
 *   [P4] "KV Cache 优化与注意力机制加速：FlashAttention / PagedAttention"
 *        (plumephp.com) section 2.2 (online-softmax statistics m and l),
 *        section 2.3 (log-sum-exp L = m + log l), section 2.5 (splitting
 *        the sequence dimension), section 4.2-4.3 (block table: logical
 *        block = pos / block_size, offset = pos % block_size).
 *
 * Every floating-point input is widened exactly to double; all arithmetic is
 * in double, in the plain order of the definition.  Nothing here is blocked,
 * fused or reordered beyond what the definition states.
 *
 * Parity pins (all in tests/test_oracle.py): the [P3] section 04 printed
 * values; fp64 torch scaled_dot_product_attention on the same inputs; GQA on
 * the cache equals MHA on the repeat_kv-expanded cache; paged equals
 * contiguous; incremental decode equals a full causal recompute ([P3]
 * section 07); split-and-merge equals unsplit; scale = 0 closed form; equal-V
 * and needle special cases; append changes only the target slots.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVO_F32 0
#define KVO_BF16 1
#define KVO_F64 2 /* values already widened (e.g. dequantised FP8 codes) */

/* Exact widening of one stored element to double.  A bf16 value is the top
 * 16 bits of an IEEE-754 binary32, so shifting its bits up by 16 gives the
 * float with the same value. */
static double load_elem(const void* base, size_t idx, int dtype) {
    if (dtype == KVO_F64) {
        return ((const double*)base)[idx];
    }
    if (dtype == KVO_F32) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t elem_bytes(int dtype) {
    return dtype == KVO_F64 ? 8u : (dtype == KVO_F32 ? 4u : 2u);
}

/* Row index (in units of d elements) of the K/V vector of sequence b, KV head
 * j, logical position p.
 *   contiguous cache [B, g, t_cap, d]:  ((b*g + j)*t_cap + p)
 *   paged pool [num_blocks, g, block_size, d]: the [P4] 4.3 get_kv rule,
 *     physical = block_table[b, p / block_size], offset = p % block_size,
 *     row = (physical*g + j)*block_size + offset. */
static size_t kv_row(const int32_t* block_table, int max_blocks, int block_size,
                     int b, int j, int p, int g, int t_cap) {
    if (block_table == NULL) {
        return ((size_t)b * g + j) * (size_t)t_cap + (size_t)p;
    }
    int logical = p / block_size;
    int offset = p % block_size;
    int physical = block_table[(size_t)b * max_blocks + logical];
    return ((size_t)physical * g + j) * (size_t)block_size + (size_t)offset;
}

/* Attention of one query head over positions [p0, p1) of one KV head.
 * Writes acc[d] = sum_p w_p V_p (unnormalised), *m_out = max_p s_p and
 * *l_out = sum_p w_p with w_p = exp(s_p - m).  An empty range gives
 * m = -inf, l = 0, acc = 0.  ([P1] 三 eq. softmax(Q_i K_j^T / sqrt(d_k)) V_j
 * with the caller's scale; [P4] 2.2 statistics m and l.) */
static void attend_range(const void* q, const void* kc, const void* vc, int dtype,
                         const int32_t* block_table, int max_blocks, int block_size,
                         int b, int i, int j, int p0, int p1,
                         int h, int g, int d, int t_cap, double scale,
                         double* s /* scratch, >= p1 - p0 */,
                         double* acc, double* m_out, double* l_out) {
    for (int k = 0; k < d; ++k) acc[k] = 0.0;
    if (p1 <= p0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    size_t qbase = ((size_t)b * h + i) * (size_t)d;
    /* scores s_p = scale * sum_k q[k] * K_p[k] */
    double m = -INFINITY;
    for (int p = p0; p < p1; ++p) {
        size_t row = kv_row(block_table, max_blocks, block_size, b, j, p, g, t_cap);
        double dot = 0.0;
        for (int k = 0; k < d; ++k) {
            dot += load_elem(q, qbase + k, dtype) * load_elem(kc, row * d + k, dtype);
        }
        s[p - p0] = scale * dot;
        if (s[p - p0] > m) m = s[p - p0];
    }
    /* w_p = exp(s_p - m), l = sum_p w_p, acc = sum_p w_p V_p */
    double l = 0.0;
    for (int p = p0; p < p1; ++p) {
        double w = exp(s[p - p0] - m);
        l += w;
        size_t row = kv_row(block_table, max_blocks, block_size, b, j, p, g, t_cap);
        for (int k = 0; k < d; ++k) acc[k] += w * load_elem(vc, row * d + k, dtype);
    }
    *m_out = m;
    *l_out = l;
}

/* Decode attention for every (sequence b, query head i).
 *   q            [B, h, d]                       (dtype)
 *   k, v         contiguous [B, g, t_cap, d] if block_table == NULL,
 *                else pools [num_blocks, g, block_size, d]       (dtype)
 *   block_table  [B, max_blocks] int32 or NULL
 *   seq_lens     [B] int32: number of attended positions (after append)
 *   out          [B, h, d] double;  lse [B, h] double
 * Query head i reads KV head j = (i*g)/h ([P1] 三 3.3).  Positions
 * >= seq_lens[b] are never read ([P3] section 10).  A sequence of length 0
 * gets out = 0 and lse = -inf.  out = acc / l, lse = m + ln l ([P4] 2.3). */
static void decode_rows(const void* q, const void* k, const void* v, int dtype,
                        const int32_t* block_table, int max_blocks, int block_size,
                        const int32_t* starts, const int32_t* seq_lens, int B, int h, int g,
                        int d, int t_cap, double scale, double* out, double* lse, int nthreads) {
    int max_len = 0;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > max_len) max_len = seq_lens[b];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long bi = 0; bi < (long)B * h; ++bi) {
            int b = (int)(bi / h), i = (int)(bi % h);
            int j = (int)(((long)i * g) / h);
            double m, l;
            attend_range(q, k, v, dtype, block_table, max_blocks, block_size, b, i, j,
                         starts ? starts[b] : 0, seq_lens[b], h, g, d, t_cap, scale, s, acc, &m, &l);
            double* o = out + (size_t)bi * d;
            if (l > 0.0) {
                for (int kk = 0; kk < d; ++kk) o[kk] = acc[kk] / l;
                lse[bi] = m + log(l);
            } else {
                for (int kk = 0; kk < d; ++kk) o[kk] = 0.0;
                lse[bi] = -INFINITY;
            }
        }
        free(s);
        free(acc);
    }
}

void kvo_decode(const void* q, const void* k, const void* v, int dtype,
                const int32_t* block_table, int max_blocks, int block_size,
                const int32_t* seq_lens, int B, int h, int g, int d, int t_cap,
                double scale, double* out, double* lse, int nthreads) {
    decode_rows(q, k, v, dtype, block_table, max_blocks, block_size, NULL, seq_lens, B, h, g, d,
                t_cap, scale, out, lse, nthreads);
}

/* Decode attention over positions [starts[b], seq_lens[b]) only: the last
 * positions a sliding window keeps ([P4] 5.2: each token attends within a
 * local window to its left; [P3] section 10: a window cache keeps only the
 * most recent W positions).  Otherwise as kvo_decode. */
void kvo_decode_range(const void* q, const void* k, const void* v, int dtype,
                      const int32_t* block_table, int max_blocks, int block_size,
                      const int32_t* starts, const int32_t* seq_lens, int B, int h, int g, int d,
                      int t_cap, double scale, double* out, double* lse, int nthreads) {
    decode_rows(q, k, v, dtype, block_table, max_blocks, block_size, starts, seq_lens, B, h, g, d,
                t_cap, scale, out, lse, nthreads);
}

/* Split reference: the context of every sequence is cut into chunks of
 * chunk_len positions; chunk c covers [c*chunk_len, min((c+1)*chunk_len, L)).
 * Each chunk yields (O_c = acc_c / l_c, lse_c = m_c + ln l_c), the partial
 * result of [P4] 2.5's sequence splitting, and the chunks are merged by
 * log-sum-exp ([P4] 2.2 rescaling identity):
 *   M = max_c lse_c,  w_c = exp(lse_c - M),
 *   out = sum_c w_c O_c / sum_c w_c,  lse = M + ln sum_c w_c.
 * Chunks with no positions have lse_c = -inf and weight 0. */
void kvo_decode_split(const void* q, const void* k, const void* v, int dtype,
                      const int32_t* block_table, int max_blocks, int block_size,
                      const int32_t* seq_lens, int B, int h, int g, int d, int t_cap,
                      double scale, int chunk_len, double* out, double* lse, int nthreads) {
    int max_len = 0;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > max_len) max_len = seq_lens[b];
    int max_chunks = (max_len + chunk_len - 1) / chunk_len;
    if (max_chunks < 1) max_chunks = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)chunk_len);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        double* po = (double*)malloc(sizeof(double) * (size_t)max_chunks * d);
        double* plse = (double*)malloc(sizeof(double) * (size_t)max_chunks);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long bi = 0; bi < (long)B * h; ++bi) {
            int b = (int)(bi / h), i = (int)(bi % h);
            int j = (int)(((long)i * g) / h);
            int L = seq_lens[b];
            int nc = (L + chunk_len - 1) / chunk_len;
            for (int c = 0; c < nc; ++c) {
                int p0 = c * chunk_len;
                int p1 = p0 + chunk_len < L ? p0 + chunk_len : L;
                double m, l;
                attend_range(q, k, v, dtype, block_table, max_blocks, block_size, b, i, j,
                             p0, p1, h, g, d, t_cap, scale, s, acc, &m, &l);
                for (int kk = 0; kk < d; ++kk) po[(size_t)c * d + kk] = acc[kk] / l;
                plse[c] = m + log(l);
            }
            double M = -INFINITY;
            for (int c = 0; c < nc; ++c)
                if (plse[c] > M) M = plse[c];
            double* o = out + (size_t)bi * d;
            for (int kk = 0; kk < d; ++kk) o[kk] = 0.0;
            if (nc == 0) {
                lse[bi] = -INFINITY;
                continue;
            }
            double wsum = 0.0;
            for (int c = 0; c < nc; ++c) {
                double w = exp(plse[c] - M);
                wsum += w;
                for (int kk = 0; kk < d; ++kk) o[kk] += w * po[(size_t)c * d + kk];
            }
            for (int kk = 0; kk < d; ++kk) o[kk] /= wsum;
            lse[bi] = M + log(wsum);
        }
        free(s);
        free(acc);
        free(po);
        free(plse);
    }
}

/* Append: write the new token's K and V of sequence b, KV head j into
 * position pos = seq_lens_before[b] (the current cache length, [P3] section
 * 08), the slot that [P1] 4.1's concat along the sequence axis creates.
 * Contiguous: cache row (b*g + j)*t_cap + pos.  Paged: the [P4] 4.3 rule
 * through block_table.  The copy is byte-exact; nothing else is written.
 *   k_new, v_new [B, g, d]; caches as for kvo_decode. */
void kvo_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                const int32_t* block_table, int max_blocks, int block_size,
                const int32_t* seq_lens_before, int B, int g, int d, int t_cap) {
    size_t eb = elem_bytes(dtype);
    size_t row_bytes = eb * (size_t)d;
    for (int b = 0; b < B; ++b) {
        int pos = seq_lens_before[b];
        for (int j = 0; j < g; ++j) {
            size_t row = kv_row(block_table, max_blocks, block_size, b, j, pos, g, t_cap);
            size_t src = ((size_t)b * g + j) * row_bytes;
            memcpy((char*)k_cache + row * row_bytes, (const char*)k_new + src, row_bytes);
            memcpy((char*)v_cache + row * row_bytes, (const char*)v_new + src, row_bytes);
        }
    }
}
