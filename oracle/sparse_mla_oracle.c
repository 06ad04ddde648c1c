/*
 * CPU oracle for sparse top-k MLA attention (prefill and paged decode).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The product path
 * never calls it; it shares no code with the HIP kernels.
 *
 * It is the plain definition of the operation, written out loop by loop in
 * double precision (every bf16 input widens exactly to double):
 *
 *   Validity of an index entry (FlashMLA PR #196, "Fix"): an entry is valid
 *   iff 0 <= idx < K, where K = s_kv for prefill.  For paged decode K is the
 *   request's cache length (reading: cache_seqlens[b], further limited to the
 *   tokens the block table can address, max_blocks_per_seq * page_size).
 *
 *   Row length L (FlashMLA PR #196, "Fix"; PR #216, "Summary"): with an
 *   explicit topk_length, L = that value clamped to [0, topk] (reading: the
 *   pages do not say what happens out of range); without it, L is one past the
 *   last valid position of the row, or 0 when the row has none.
 *
 *   Keys of a row (PR #216, "Summary": positions at or past L are never used
 *   for addressing; PR #196, "Correctness notes": invalid entries before L stay
 *   masked): the valid entries at positions j < L, in position order, each
 *   occurrence counted once.
 *
 *   Paged address (PR #216, 64-token page blocks with a block table): logical
 *   position p of request b lives in physical page block_table[b][p / page]
 *   at slot p % page.  Reading: a key whose page entry lies outside
 *   [0, num_blocks) is masked like an invalid index (the tail scan still sees
 *   only the index value).
 *
 *   Attention per (row, head) (PR #196, "Problem"/"Numbers": all h_q heads
 *   share one latent KV head; V is the first d_v columns of each KV row):
 *     s_j   = sm_scale * sum_d q[h][d] * kv[key_j][d]
 *     m     = max_j s_j                       -> max_logits
 *     Z     = sum_j exp(s_j - m)
 *     lse   = m + ln Z                        (natural log, sink-free; reading)
 *     denom = Z + exp(attn_sink[h] - m)       (PR #198, "Summary": the sink is
 *                                              a value-less virtual key folded
 *                                              into the softmax denominator)
 *     out[c]= sum_j exp(s_j - m) * kv[key_j][c] / denom,  c < d_v
 *   A row with no key (PR #196, "Correctness notes") gives out = 0,
 *   lse = +inf, max_logits = -inf, with or without a sink.
 *
 * Every output is double.  Rows are independent; OpenMP spreads them over the
 * host cores without changing any per-row arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int is_valid_index(int32_t idx, int64_t bound)
{
    return idx >= 0 && (int64_t)idx < bound;
}

/* Row length L of one index row (see header). */
static int32_t row_length(const int32_t *idx_row, int32_t topk, const int32_t *explicit_len,
                          int64_t bound)
{
    if (explicit_len != NULL) {
        int32_t L = *explicit_len;
        if (L < 0) L = 0;
        if (L > topk) L = topk;
        return L;
    }
    int32_t L = 0;
    for (int32_t j = 0; j < topk; ++j)
        if (is_valid_index(idx_row[j], bound)) L = j + 1;
    return L;
}

/* Masked softmax attention of one query row over an explicit key list.
 * q_row: [h_q][d_qk] bf16; keys[j]: pointer to a KV row of d_qk bf16. */
static void attend(const uint16_t *q_row, const uint16_t *const *keys, int64_t nkeys,
                   int32_t h_q, int32_t d_qk, int32_t d_v, double sm_scale, const float *attn_sink,
                   double *s, double *out_row, double *lse_row, double *ml_row)
{
    for (int32_t h = 0; h < h_q; ++h) {
        double *o = out_row + (int64_t)h * d_v;
        for (int32_t c = 0; c < d_v; ++c) o[c] = 0.0;
        if (nkeys == 0) {
            lse_row[h] = INFINITY;
            ml_row[h] = -INFINITY;
            continue;
        }
        const uint16_t *qh = q_row + (int64_t)h * d_qk;
        for (int64_t j = 0; j < nkeys; ++j) {
            double acc = 0.0;
            for (int32_t d = 0; d < d_qk; ++d)
                acc += bf16_to_double(qh[d]) * bf16_to_double(keys[j][d]);
            s[j] = sm_scale * acc;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < nkeys; ++j)
            if (s[j] > m) m = s[j];
        double Z = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) Z += exp(s[j] - m);
        double denom = Z;
        if (attn_sink != NULL) denom += exp((double)attn_sink[h] - m);
        for (int64_t j = 0; j < nkeys; ++j) {
            double p = exp(s[j] - m);
            for (int32_t c = 0; c < d_v; ++c) o[c] += p * bf16_to_double(keys[j][c]);
        }
        for (int32_t c = 0; c < d_v; ++c) o[c] /= denom;
        ml_row[h] = m;
        lse_row[h] = m + log(Z);
    }
}

static int oracle_threads(int requested)
{
#ifdef _OPENMP
    return requested > 0 ? requested : omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

/* Per-row lengths.  rows = B * rows_per_seq.  The validity bound of row r is
 * s_kv when cache_seqlens is NULL (prefill), else
 * min(cache_seqlens[r / rows_per_seq], addressable) (paged decode;
 * addressable = max_blocks_per_seq * page_size). */
int oracle_row_lengths(const int32_t *indices, const int32_t *topk_length,
                       const int32_t *cache_seqlens, int64_t rows, int64_t rows_per_seq,
                       int32_t topk, int64_t s_kv, int64_t addressable, int32_t *row_len)
{
    if (!indices || !row_len || topk <= 0 || rows < 0 || rows_per_seq <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t bound = s_kv;
        if (cache_seqlens) {
            bound = cache_seqlens[r / rows_per_seq];
            if (bound > addressable) bound = addressable;
        }
        row_len[r] = row_length(indices + r * topk, topk, topk_length ? topk_length + r : NULL,
                                bound);
    }
    return 0;
}

/* Prefill.  q [s_q][h_q][d_qk] bf16; kv [s_kv][d_qk] bf16 (h_kv = 1);
 * indices [s_q][topk]; topk_length [s_q] or NULL; attn_sink [h_q] or NULL.
 * rows_sel lists the rows to evaluate (NULL: all s_q rows, n_sel = s_q);
 * outputs are packed in rows_sel order: out [n_sel][h_q][d_v],
 * lse/max_logits [n_sel][h_q], row_len [n_sel] (may be NULL). */
int oracle_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *indices,
                          const int32_t *topk_length, const float *attn_sink, int64_t s_q,
                          int64_t s_kv, int32_t h_q, int32_t d_qk, int32_t d_v, int32_t topk,
                          double sm_scale, const int64_t *rows_sel, int64_t n_sel, double *out,
                          double *lse, double *max_logits, int32_t *row_len, int threads)
{
    if (!q || !kv || !indices || !out || !lse || !max_logits) return 1;
    if (h_q <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk || topk <= 0 || s_q < 0 || s_kv < 0)
        return 2;
    if (rows_sel == NULL) n_sel = s_q;
    int bad = 0;
#pragma omp parallel num_threads(oracle_threads(threads)) reduction(| : bad)
    {
        double *s = malloc(sizeof(double) * (size_t)topk);
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)topk);
        if (!s || !keys) bad = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_sel; ++n) {
            if (!s || !keys) continue;
            int64_t r = rows_sel ? rows_sel[n] : n;
            if (r < 0 || r >= s_q) { bad = 1; continue; }
            const int32_t *idx = indices + r * topk;
            int32_t L = row_length(idx, topk, topk_length ? topk_length + r : NULL, s_kv);
            int64_t nk = 0;
            for (int32_t j = 0; j < L; ++j)
                if (is_valid_index(idx[j], s_kv)) keys[nk++] = kv + (int64_t)idx[j] * d_qk;
            attend(q + r * (int64_t)h_q * d_qk, keys, nk, h_q, d_qk, d_v, sm_scale, attn_sink, s,
                   out + n * (int64_t)h_q * d_v, lse + n * h_q, max_logits + n * h_q);
            if (row_len) row_len[n] = L;
        }
        free(s);
        free(keys);
    }
    return bad ? 3 : 0;
}

/* Paged decode.  q [B][s_q][h_q][d_qk]; kv_cache [num_blocks][page_size][d_qk];
 * block_table [B][max_blocks_per_seq]; cache_seqlens [B];
 * indices [B][s_q][topk] (logical positions); topk_length [B][s_q] or NULL.
 * Rows are r = b * s_q + t; rows_sel / outputs as for prefill. */
int oracle_sparse_mla_decode_fwd(const uint16_t *q, const uint16_t *kv_cache,
                                 const int32_t *block_table, const int32_t *cache_seqlens,
                                 const int32_t *indices, const int32_t *topk_length,
                                 const float *attn_sink, int64_t B, int64_t s_q, int32_t h_q,
                                 int32_t d_qk, int32_t d_v, int32_t topk, int64_t num_blocks,
                                 int32_t page_size, int32_t max_blocks_per_seq, double sm_scale,
                                 const int64_t *rows_sel, int64_t n_sel, double *out, double *lse,
                                 double *max_logits, int32_t *row_len, int threads)
{
    if (!q || !kv_cache || !block_table || !cache_seqlens || !indices || !out || !lse ||
        !max_logits)
        return 1;
    if (h_q <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk || topk <= 0 || B < 0 || s_q <= 0 ||
        page_size <= 0 || max_blocks_per_seq <= 0)
        return 2;
    int64_t rows = B * s_q;
    if (rows_sel == NULL) n_sel = rows;
    int bad = 0;
#pragma omp parallel num_threads(oracle_threads(threads)) reduction(| : bad)
    {
        double *s = malloc(sizeof(double) * (size_t)topk);
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)topk);
        if (!s || !keys) bad = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_sel; ++n) {
            if (!s || !keys) continue;
            int64_t r = rows_sel ? rows_sel[n] : n;
            if (r < 0 || r >= rows) { bad = 1; continue; }
            int64_t b = r / s_q;
            int64_t bound = cache_seqlens[b];
            int64_t addressable = (int64_t)max_blocks_per_seq * page_size;
            if (bound > addressable) bound = addressable;
            const int32_t *idx = indices + r * topk;
            int32_t L = row_length(idx, topk, topk_length ? topk_length + r : NULL, bound);
            int64_t nk = 0;
            for (int32_t j = 0; j < L; ++j) {
                if (!is_valid_index(idx[j], bound)) continue;
                int64_t page = block_table[b * max_blocks_per_seq + idx[j] / page_size];
                if (page < 0 || page >= num_blocks) continue;
                keys[nk++] = kv_cache + (page * page_size + idx[j] % page_size) * (int64_t)d_qk;
            }
            attend(q + r * (int64_t)h_q * d_qk, keys, nk, h_q, d_qk, d_v, sm_scale, attn_sink, s,
                   out + n * (int64_t)h_q * d_v, lse + n * h_q, max_logits + n * h_q);
            if (row_len) row_len[n] = L;
        }
        free(s);
        free(keys);
    }
    return bad ? 3 : 0;
}
