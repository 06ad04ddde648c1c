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

/* Backward of the prefill operation (FlashMLA PR #198, "Summary", item 1: the
 * sparse MLA backward works from the forward's saved out and lse; the key and
 * value gradients of a row go to the KV row the index names, summed over every
 * query row, head and occurrence).  It is the gradient of the forward's
 * definition above, written out per (query row i, key occurrence j, head h):
 *
 *   lse'  = lse                          (natural log, as the forward returns)
 *         = lse * ln 2                   (lse_base2: the pages' bwd takes
 *                                          base-2 lse)
 *         = ln(exp(lse') + exp(sink[h])) (with attn_sink: the forward's lse
 *                                          leaves the sink out; the softmax
 *                                          denominator holds it)
 *   p     = exp(s_j - lse')              (the forward's softmax weight)
 *   delta = sum_c dout[c] * out[c]       (c < d_v; d out / d s_j = p (v_j - out))
 *   dp    = sum_c dout[c] * kv[key_j][c]
 *   ds    = p * (dp - delta)             (d loss / d s_j)
 *   dq[i][h][d]      += sm_scale * ds * kv[key_j][d]           d < d_qk
 *   dkv[key_j][d]    += sm_scale * ds * q[i][h][d]             d < d_qk
 *   dkv[key_j][c]    += p * dout[c]                            c < d_v
 *   d_sink[h]        -= exp(sink[h] - lse') * delta            (once per row)
 *
 * The keys of a row are the forward's (valid positions before the row's
 * length, each occurrence once).  A row whose lse' is +inf (no key) adds
 * nothing.  out and dout come in as doubles (the caller widens bf16 exactly).
 *
 * dq is evaluated for the rows rows_sel lists (all rows when NULL), dkv for
 * the KV rows kv_sel lists (all when NULL), each a sum over the occurrences
 * of that KV row in the query rows' key lists. */

/* Orders (KV row, query row) pairs. */
static int cmp_pair(const void *a, const void *b)
{
    const int64_t *x = a, *y = b;
    if (x[0] != y[0]) return x[0] < y[0] ? -1 : 1;
    return x[1] < y[1] ? -1 : (x[1] > y[1]);
}

/* lse' of (row, head), see above. */
static double effective_lse(double lse, int lse_base2, const float *attn_sink, int32_t h)
{
    double l = lse_base2 ? lse * log(2.0) : lse;
    if (attn_sink != NULL && !isinf(l)) {
        double s = (double)attn_sink[h];
        double m = l > s ? l : s;
        l = m + log(exp(l - m) + exp(s - m));
    }
    return l;
}

/* Gradient terms of one (row, key occurrence) over all heads.  dq_row
 * [h_q][d_qk] and dkv_row [d_qk] are added to when not NULL. */
static void key_grad(const uint16_t *q_row, const uint16_t *key, const double *dout_row,
                     const double *lse_eff, const double *delta, int32_t h_q, int32_t d_qk,
                     int32_t d_v, double sm_scale, double *dq_row, double *dkv_row)
{
    for (int32_t h = 0; h < h_q; ++h) {
        if (isinf(lse_eff[h])) continue;
        const uint16_t *qhd = q_row + (int64_t)h * d_qk;
        const double *doh = dout_row + (int64_t)h * d_v;
        double acc = 0.0;
        for (int32_t d = 0; d < d_qk; ++d) acc += bf16_to_double(qhd[d]) * bf16_to_double(key[d]);
        double p = exp(sm_scale * acc - lse_eff[h]);
        double dp = 0.0;
        for (int32_t c = 0; c < d_v; ++c) dp += doh[c] * bf16_to_double(key[c]);
        double ds = p * (dp - delta[h]);
        if (dq_row != NULL) {
            double *dqh = dq_row + (int64_t)h * d_qk;
            for (int32_t d = 0; d < d_qk; ++d) dqh[d] += sm_scale * ds * bf16_to_double(key[d]);
        }
        if (dkv_row != NULL) {
            for (int32_t d = 0; d < d_qk; ++d) dkv_row[d] += sm_scale * ds * bf16_to_double(qhd[d]);
            for (int32_t c = 0; c < d_v; ++c) dkv_row[c] += p * doh[c];
        }
    }
}

/* q [s_q][h_q][d_qk] bf16; kv [s_kv][d_qk] bf16; out, dout [s_q][h_q][d_v]
 * double; indices [s_q][topk]; topk_length [s_q] or NULL; lse [s_q][h_q];
 * attn_sink [h_q] or NULL.  Outputs: dq [n_sel][h_q][d_qk] (NULL: skipped),
 * dkv [n_kv_sel][d_qk] (NULL: skipped), d_sink [h_q] (NULL: skipped; needs
 * attn_sink). */
int oracle_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const double *out,
                          const double *dout, const int32_t *indices, const int32_t *topk_length,
                          const double *lse, const float *attn_sink, int64_t s_q, int64_t s_kv,
                          int32_t h_q, int32_t d_qk, int32_t d_v, int32_t topk, double sm_scale,
                          int lse_base2, const int64_t *rows_sel, int64_t n_sel,
                          const int64_t *kv_sel, int64_t n_kv_sel, double *dq, double *dkv,
                          double *d_sink, int threads)
{
    if (!q || !kv || !out || !dout || !indices || !lse) return 1;
    if (h_q <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk || topk <= 0 || s_q < 0 || s_kv < 0)
        return 2;
    if (d_sink != NULL && attn_sink == NULL) return 2;
    if (rows_sel == NULL) n_sel = s_q;
    if (kv_sel == NULL) n_kv_sel = s_kv;
    const int nt = oracle_threads(threads);

    /* Per row: length, lse' and delta of every head. */
    int32_t *len = malloc(sizeof(int32_t) * (size_t)(s_q > 0 ? s_q : 1));
    double *lse_eff = malloc(sizeof(double) * (size_t)(s_q * h_q > 0 ? s_q * h_q : 1));
    double *delta = malloc(sizeof(double) * (size_t)(s_q * h_q > 0 ? s_q * h_q : 1));
    if (!len || !lse_eff || !delta) { free(len); free(lse_eff); free(delta); return 3; }
    for (int64_t i = 0; i < s_q; ++i) {
        len[i] = row_length(indices + i * topk, topk, topk_length ? topk_length + i : NULL, s_kv);
        for (int32_t h = 0; h < h_q; ++h) {
            int64_t rh = i * h_q + h;
            lse_eff[rh] = effective_lse(lse[rh], lse_base2, attn_sink, h);
            double dl = 0.0;
            for (int32_t c = 0; c < d_v; ++c) dl += dout[rh * d_v + c] * out[rh * d_v + c];
            delta[rh] = dl;
        }
    }

    int bad = 0;
    if (dq != NULL) {
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(| : bad)
        for (int64_t n = 0; n < n_sel; ++n) {
            int64_t i = rows_sel ? rows_sel[n] : n;
            double *dq_row = dq + n * (int64_t)h_q * d_qk;
            for (int64_t e = 0; e < (int64_t)h_q * d_qk; ++e) dq_row[e] = 0.0;
            if (i < 0 || i >= s_q) { bad = 1; continue; }
            const int32_t *idx = indices + i * topk;
            for (int32_t j = 0; j < len[i]; ++j)
                if (is_valid_index(idx[j], s_kv))
                    key_grad(q + i * (int64_t)h_q * d_qk, kv + (int64_t)idx[j] * d_qk,
                             dout + i * (int64_t)h_q * d_v, lse_eff + i * h_q, delta + i * h_q,
                             h_q, d_qk, d_v, sm_scale, dq_row, NULL);
        }
    }

    if (dkv != NULL && !bad) {
        /* Occurrences as (KV row, query row) pairs sorted by KV row then query
         * row; the pairs of KV row k are found by binary search. */
        int64_t total = 0;
        for (int64_t i = 0; i < s_q; ++i)
            for (int32_t j = 0; j < len[i]; ++j)
                if (is_valid_index(indices[i * topk + j], s_kv)) ++total;
        int64_t *pairs = malloc(sizeof(int64_t) * 2 * (size_t)(total > 0 ? total : 1));
        if (!pairs) bad = 1;
        int64_t np = 0;
        for (int64_t i = 0; !bad && i < s_q; ++i)
            for (int32_t j = 0; j < len[i]; ++j) {
                int32_t k = indices[i * topk + j];
                if (is_valid_index(k, s_kv)) {
                    pairs[2 * np] = k;
                    pairs[2 * np + 1] = i;
                    ++np;
                }
            }
        if (!bad) qsort(pairs, (size_t)np, 2 * sizeof(int64_t), cmp_pair);
        if (!bad) {
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1) reduction(| : bad)
            for (int64_t n = 0; n < n_kv_sel; ++n) {
                int64_t k = kv_sel ? kv_sel[n] : n;
                double *dkv_row = dkv + n * (int64_t)d_qk;
                for (int32_t d = 0; d < d_qk; ++d) dkv_row[d] = 0.0;
                if (k < 0 || k >= s_kv) { bad = 1; continue; }
                int64_t lo = 0, hi = np;  /* first pair with KV row >= k */
                while (lo < hi) {
                    int64_t mid = lo + (hi - lo) / 2;
                    if (pairs[2 * mid] < k) lo = mid + 1; else hi = mid;
                }
                for (int64_t e = lo; e < np && pairs[2 * e] == k; ++e) {
                    int64_t i = pairs[2 * e + 1];
                    key_grad(q + i * (int64_t)h_q * d_qk, kv + k * (int64_t)d_qk,
                             dout + i * (int64_t)h_q * d_v, lse_eff + i * h_q, delta + i * h_q,
                             h_q, d_qk, d_v, sm_scale, NULL, dkv_row);
                }
            }
        }
        free(pairs);
    }

    if (d_sink != NULL && !bad) {
        for (int32_t h = 0; h < h_q; ++h) d_sink[h] = 0.0;
        for (int64_t i = 0; i < s_q; ++i)
            for (int32_t h = 0; h < h_q; ++h) {
                int64_t rh = i * h_q + h;
                if (isinf(lse_eff[rh])) continue;
                d_sink[h] -= exp((double)attn_sink[h] - lse_eff[rh]) * delta[rh];
            }
    }
    free(len);
    free(lse_eff);
    free(delta);
    return bad ? 3 : 0;
}

/* Block-sparse attention forward, non-absorbed MLA shape (FlashMLA PR #198,
 * "Summary", item 3: each query block attends only the key blocks it
 * selects; "Benchmarks": 192/128 heads).  One sequence of s tokens;
 * q [s][h_q][d_qk], k [s][h_kv][d_qk], v [s][h_kv][d_v] bf16; query head h
 * reads KV head h / (h_q / h_kv).  The selection of query block
 * qb = i / q_block is the list q2k_col_idx[q2k_row_ptr[qb] .. q2k_row_ptr[qb + 1]).
 *
 * Keys of row i (readings): every listed block b with 0 <= b < ceil(s / k_block)
 * contributes its keys b * k_block .. min((b + 1) * k_block, s) - 1, each
 * listing once (a block listed twice counts twice, like a repeated top-k
 * index); other block ids are ignored; with `causal`, keys j > i are left
 * out.  Attention per (row, head) is the forward's definition above (no
 * sink); a row without keys gives out = 0, lse = +inf.
 * rows_sel / n_sel select the rows (NULL: all); outputs are packed in that
 * order: out [n_sel][h_q][d_v], lse [n_sel][h_q] (natural log). */
int oracle_block_sparse_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const int32_t *q2k_row_ptr, const int32_t *q2k_col_idx, int64_t s,
                            int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t q_block,
                            int32_t k_block, int causal, double sm_scale, const int64_t *rows_sel,
                            int64_t n_sel, double *out, double *lse, int threads)
{
    if (!q || !k || !v || !q2k_row_ptr || !out || !lse) return 1;
    if (s < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 || d_qk <= 0 || d_v <= 0 ||
        q_block <= 0 || k_block <= 0)
        return 2;
    if (rows_sel == NULL) n_sel = s;
    const int64_t n_kblocks = (s + k_block - 1) / k_block;
    const int32_t group = h_q / h_kv;
    int bad = 0;
#pragma omp parallel num_threads(oracle_threads(threads)) reduction(| : bad)
    {
        int64_t cap = 0;
        int64_t *keys = NULL;
        double *sc = NULL;
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_sel; ++n) {
            int64_t i = rows_sel ? rows_sel[n] : n;
            if (i < 0 || i >= s) { bad = 1; continue; }
            int64_t qb = i / q_block;
            int64_t nk = 0;
            for (int32_t e = q2k_row_ptr[qb]; e < q2k_row_ptr[qb + 1]; ++e) {
                int64_t b = q2k_col_idx[e];
                if (b < 0 || b >= n_kblocks) continue;
                int64_t end = (b + 1) * k_block < s ? (b + 1) * k_block : s;
                for (int64_t j = b * k_block; j < end; ++j) {
                    if (causal && j > i) continue;
                    if (nk == cap) {
                        cap = cap ? 2 * cap : 1024;
                        keys = realloc(keys, sizeof(int64_t) * (size_t)cap);
                        sc = realloc(sc, sizeof(double) * (size_t)cap);
                        if (!keys || !sc) { bad = 1; cap = 0; nk = 0; break; }
                    }
                    keys[nk++] = j;
                }
            }
            for (int32_t h = 0; h < h_q; ++h) {
                double *o = out + (n * h_q + h) * (int64_t)d_v;
                for (int32_t c = 0; c < d_v; ++c) o[c] = 0.0;
                if (nk == 0) { lse[n * h_q + h] = INFINITY; continue; }
                const uint16_t *qh = q + (i * h_q + h) * (int64_t)d_qk;
                const int32_t kvh = h / group;
                double m = -INFINITY;
                for (int64_t t = 0; t < nk; ++t) {
                    const uint16_t *kr = k + (keys[t] * h_kv + kvh) * (int64_t)d_qk;
                    double acc = 0.0;
                    for (int32_t d = 0; d < d_qk; ++d) acc += bf16_to_double(qh[d]) * bf16_to_double(kr[d]);
                    sc[t] = sm_scale * acc;
                    if (sc[t] > m) m = sc[t];
                }
                double Z = 0.0;
                for (int64_t t = 0; t < nk; ++t) {
                    const double p = exp(sc[t] - m);
                    const uint16_t *vr = v + (keys[t] * h_kv + kvh) * (int64_t)d_v;
                    Z += p;
                    for (int32_t c = 0; c < d_v; ++c) o[c] += p * bf16_to_double(vr[c]);
                }
                for (int32_t c = 0; c < d_v; ++c) o[c] /= Z;
                lse[n * h_q + h] = m + log(Z);
            }
        }
        free(keys);
        free(sc);
    }
    return bad ? 3 : 0;
}
