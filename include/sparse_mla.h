/*
 * sparse_mla.h -- C ABI of the MI355X (gfx950) sparse top-k MLA attention
 * forward library (libsparse_mla.so).
 *
 * The operation (FlashMLA PR #196, "Problem" and "Fix"; PR #216, "Summary";
 * PR #198, "Summary" for the sink):
 *   every query row attends, with all h_q heads sharing one latent KV head
 *   (h_kv = 1), to the KV rows named by its own int32 index vector.  V is the
 *   first d_v columns of each KV row.  An index entry is valid iff
 *   0 <= idx < K (K = s_kv for prefill, the request's cache length for
 *   decode); invalid entries are masked.  The row length L is topk_length[r]
 *   clamped to [0, topk] when topk_length is given, else one past the last
 *   valid entry of the row (0 when none); positions >= L are never used to
 *   address KV.  With a per-head attn_sink, exp(sink[h]) joins the softmax
 *   denominator (out only).  A row without valid entries yields out = 0,
 *   lse = +inf and max_logits = -inf.
 *
 * Outputs, per row r and head h:
 *   out[r,h,:]     = sum_j softmax_j * V[key_j]            (bf16, RNE)
 *   lse[r,h]       = natural-log log-sum-exp of the scaled logits
 *                    sm_scale * q.k over the row's keys (without the sink)
 *   max_logits[r,h]= max of those scaled logits
 *
 * Conventions shared by all entry points
 *   Memory:    every pointer is a device pointer to caller-owned, contiguous,
 *              16-byte aligned memory.  The library allocates, frees and
 *              synchronises nothing; work is enqueued on `stream` only
 *              (0 = the null stream).
 *   Values:    index, length and block-table contents are data, never
 *              validated and never errors: invalid entries are masked.
 *   Errors:    shape and pointer problems are reported synchronously as a
 *              status code before anything is launched; a failed launch is
 *              SMLA_ERR_LAUNCH.  sparse_mla_last_error() returns a
 *              thread-local text for the last non-OK status.
 *   Threading: stateless apart from the thread-local error text.
 *   Support:   h_kv = 1; d_qk in {512, 576}; d_v = 512; h_q a multiple of 16
 *              in [16, 128]; page_size = 64 for decode; sm_scale positive
 *              and finite.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SMLA_OK = 0,
    SMLA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                 */
    SMLA_ERR_BAD_SHAPE = 2,   /* a size is non-positive or inconsistent     */
    SMLA_ERR_UNSUPPORTED = 3, /* outside the support list above             */
    SMLA_ERR_LAUNCH = 4       /* the kernel launch reported an error        */
} smla_status;

/* A HIP stream handle (hipStream_t); void* keeps this header free of HIP. */
typedef void *smla_stream_t;

/*
 * Sparse prefill forward (FlashMLA PR #196).
 *   q           bf16  [s_q, h_q, d_qk]
 *   kv          bf16  [s_kv, h_kv, d_qk]; V = kv[..., :d_v] (may be NULL when s_kv = 0)
 *   indices     int32 [s_q, h_kv, topk]
 *   topk_length int32 [s_q] or NULL (NULL: derive L by the tail scan)
 *   attn_sink   fp32  [h_q] or NULL
 *   out         bf16  [s_q, h_q, d_v]
 *   lse         fp32  [s_q, h_q]
 *   max_logits  fp32  [s_q, h_q]
 * s_q = 0 is a valid no-op (pointers may then be NULL).
 */
smla_status sparse_mla_fwd(const void *q, const void *kv, const int32_t *indices,
                           const int32_t *topk_length, const float *attn_sink, int32_t s_q,
                           int32_t s_kv, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                           int32_t topk, float sm_scale, void *out, float *lse,
                           float *max_logits, smla_stream_t stream);

/*
 * Paged sparse decode forward (FlashMLA PR #216: 64-token page blocks, a
 * block table, per-row dynamic top-k).
 *   q             bf16  [B, s_q, h_q, d_qk]
 *   kv_cache      bf16  [num_blocks, page_size, h_kv, d_qk] (NULL allowed when num_blocks = 0)
 *   block_table   int32 [B, max_blocks_per_seq]: physical page of each
 *                 64-token logical page of request b
 *   cache_seqlens int32 [B]: KV length of request b.  An index is valid iff
 *                 0 <= idx < min(cache_seqlens[b], max_blocks_per_seq*64);
 *                 a valid index whose page entry is outside [0, num_blocks)
 *                 is masked.
 *   indices       int32 [B, s_q, topk]: logical token positions
 *   topk_length   int32 [B, s_q] or NULL (one length per query row)
 *   attn_sink     fp32  [h_q] or NULL
 *   out           bf16  [B, s_q, h_q, d_v]
 *   lse           fp32  [B, s_q, h_q]
 *   max_logits    fp32  [B, s_q, h_q] or NULL (NULL: not stored; the
 *                 pages' decode returns out and lse only)
 * B = 0 is a valid no-op (pointers may then be NULL).
 */
smla_status sparse_mla_decode_fwd(const void *q, const void *kv_cache,
                                  const int32_t *block_table, const int32_t *cache_seqlens,
                                  const int32_t *indices, const int32_t *topk_length,
                                  const float *attn_sink, int32_t B, int32_t s_q, int32_t h_q,
                                  int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
                                  int32_t num_blocks, int32_t page_size,
                                  int32_t max_blocks_per_seq, float sm_scale, void *out,
                                  float *lse, float *max_logits, smla_stream_t stream);

/*
 * Bytes of workspace that sparse_mla_decode_fwd_split needs for num_splits
 * key-range splits of every row: B*s_q*num_splits*h_q*(d_v + 2) fp32 values
 * (each split's partial output and its lse and max).  0 for num_splits <= 1
 * or non-positive sizes.
 */
size_t sparse_mla_decode_split_workspace_bytes(int32_t B, int32_t s_q, int32_t h_q, int32_t d_v,
                                               int32_t num_splits);

/*
 * Split-KV paged decode: the scheduler-metadata path for batches too small to
 * fill the device (FlashMLA PR #216, "Kernel performance": the batch-2 runs
 * reuse scheduler metadata across calls).  Arguments as sparse_mla_decode_fwd.
 * Split s of a row takes its index blocks [s*n/num_splits, (s+1)*n/num_splits),
 * n = ceil(L/block), and writes its output normalised by its own softmax sum,
 * its lse and its max to the workspace; a second kernel merges them: lse =
 * logsumexp of the split lses (an empty split, lse = -inf, adds nothing),
 * out = sum of exp(lse_s - lse) * out_s, the sink joins the denominator once
 * after the merge, and a row whose splits are all empty gives (0, +inf, -inf)
 * as the unsplit path does.  Results equal the unsplit path's up to rounding.
 * max_logits may be NULL, as in sparse_mla_decode_fwd.
 *   num_splits       1 .. 1024; 1 runs the unsplit path (workspace unused)
 *   workspace        device memory of at least
 *                    sparse_mla_decode_split_workspace_bytes(...) bytes,
 *                    16-byte aligned, owned by the caller; its contents
 *                    need no initialisation and are garbage afterwards;
 *                    calls that overlap on the same workspace race
 *   workspace_bytes  its size (checked)
 * Supported for h_q = 128 (d_qk 512 or 576) and h_q = 64 at d_qk = 512;
 * other shapes return SMLA_ERR_UNSUPPORTED.  Both kernels are enqueued on
 * `stream`.
 */
smla_status sparse_mla_decode_fwd_split(const void *q, const void *kv_cache,
                                        const int32_t *block_table, const int32_t *cache_seqlens,
                                        const int32_t *indices, const int32_t *topk_length,
                                        const float *attn_sink, int32_t B, int32_t s_q,
                                        int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                                        int32_t topk, int32_t num_blocks, int32_t page_size,
                                        int32_t max_blocks_per_seq, float sm_scale,
                                        int32_t num_splits, void *workspace,
                                        size_t workspace_bytes, void *out, float *lse,
                                        float *max_logits, smla_stream_t stream);

/*
 * Split-KV paged decode that allocates nothing, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments and results as
 * sparse_mla_decode_fwd_split without the workspace: the partials live in a
 * static device array of sparse_mla_decode_split_noalloc_max_bytes() bytes
 * (256 (row, split) units at h_q = 128), which each GPU the library runs on
 * holds until the process ends.  Its device address is looked up on the
 * first call on a device.  The array needs no initialisation (every split
 * writes its partials before the merge reads them) and keeps the last
 * call's contents.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU race.  Partials larger than the array are rejected
 * with SMLA_ERR_BAD_SHAPE before anything is launched; num_splits = 1 runs
 * the unsplit path.  No allocation, free or synchronisation is made.
 */
size_t sparse_mla_decode_split_noalloc_max_bytes(void);

smla_status sparse_mla_decode_fwd_split_noalloc(const void *q, const void *kv_cache,
                                                const int32_t *block_table,
                                                const int32_t *cache_seqlens,
                                                const int32_t *indices,
                                                const int32_t *topk_length,
                                                const float *attn_sink, int32_t B, int32_t s_q,
                                                int32_t h_q, int32_t h_kv, int32_t d_qk,
                                                int32_t d_v, int32_t topk, int32_t num_blocks,
                                                int32_t page_size, int32_t max_blocks_per_seq,
                                                float sm_scale, int32_t num_splits, void *out,
                                                float *lse, float *max_logits,
                                                smla_stream_t stream);

/*
 * The row length L every kernel above uses (FlashMLA PR #196, "Fix": tail
 * scan for the last valid entry; PR #216, "Summary": explicit lengths), from
 * the same device routine.
 *   indices       int32 [rows, topk]
 *   topk_length   int32 [rows] or NULL
 *   cache_seqlens int32 [rows / rows_per_seq] or NULL.  NULL: the bound is
 *                 s_kv for every row.  Else the bound of row r is
 *                 min(cache_seqlens[r / rows_per_seq], addressable) with
 *                 addressable = max_blocks_per_seq * 64.
 *   row_len       int32 [rows] (output)
 */
smla_status sparse_mla_row_lengths(const int32_t *indices, const int32_t *topk_length,
                                   const int32_t *cache_seqlens, int32_t rows,
                                   int32_t rows_per_seq, int32_t topk, int32_t s_kv,
                                   int32_t max_blocks_per_seq, int32_t *row_len,
                                   smla_stream_t stream);

/*
 * Backward of the prefill operation (FlashMLA PR #198, "Summary", item 1:
 * sparse MLA backward from the forward's saved out and lse; key and value
 * gradients scattered into an fp32 accumulator with atomic adds).  Per query
 * row i, head h and key occurrence j (the forward's keys: valid entries
 * before the row length):
 *   p = exp(s_j - lse'),  ds = sm_scale p (dout_h . v_j - dout_h . out_h)
 *   dq[i][h]   = sum_j ds k_j
 *   dkv[idx_j] += ds q_h (all d_qk columns) + p dout_h (the d_v value columns)
 * lse' is the row's softmax normaliser: lse itself (natural log, as the
 * forward returns it; lse_base2 = 1 takes it in base 2, the pages' backward
 * contract), combined with attn_sink[h] when a sink is given (the forward's
 * lse leaves the sink out).
 *   q             bf16 [s_q, h_q, d_qk]
 *   kv            bf16 [s_kv, 1, d_qk]
 *   out, dout     bf16 [s_q, h_q, d_v]   forward output and its gradient
 *   indices       int32 [s_q, 1, topk]; topk_length int32 [s_q] or NULL
 *                 (same meaning as in sparse_mla_fwd)
 *   lse           fp32 [s_q, h_q]        forward lse (+inf: row without keys)
 *   attn_sink     fp32 [h_q] or NULL     the sink the forward used
 *   lse_base2     0: natural-log lse, 1: base-2 lse
 *   workspace     device memory of sparse_mla_bwd_workspace_bytes(s_q, s_kv,
 *                 d_qk) bytes, 16-byte aligned (the fp32 dkv accumulator, the
 *                 row lengths and, where s_kv <= 16384 and s_q * s_kv <= 2^28,
 *                 per-row statistics and key bitmaps of s_q * s_kv / 8 bytes);
 *                 no initialisation needed, garbage after; calls that overlap
 *                 on one workspace race
 *   dq            bf16 [s_q, h_q, d_qk]  (output)
 *   dkv           bf16 [s_kv, 1, d_qk]   (output; rows no query names are 0)
 *   d_sink        fp32 [h_q] or NULL     (output, needs attn_sink):
 *                 -sum_i exp(sink[h] - lse'_ih) (dout_ih . out_ih)
 * Supported: h_q = 64, h_kv = 1, d_qk 512 or 576, d_v = 512.  Two ways to
 * sum dkv, both in a run-dependent order (fp32 atomics):
 *   where the workspace holds the bitmaps and s_kv <= 4 topk, a key-outer
 *   pass ("bwd_key_outer" in sparse_mla_last_kernel): per block of 64 KV rows
 *   and chunk of 128 query rows, P and dS are recomputed for the rows that
 *   name a key of the block and dK + dV summed in registers, one atomic add
 *   per element of the block; rows that name a key twice scatter per pair;
 *   otherwise the row pass scatters every (row, key) pair ("bwd_scatter").
 * Enqueued on `stream`: zero fill, row lengths, [key bitmaps], the row pass
 * (dq, d_sink, and the scattered dkv), [the key-outer pass], dkv conversion.
 */
size_t sparse_mla_bwd_workspace_bytes(int32_t s_q, int32_t s_kv, int32_t d_qk);

smla_status sparse_mla_bwd(const void *q, const void *kv, const void *out, const void *dout,
                           const int32_t *indices, const int32_t *topk_length, const float *lse,
                           const float *attn_sink, int32_t s_q, int32_t s_kv, int32_t h_q,
                           int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
                           float sm_scale, int32_t lse_base2, void *workspace,
                           size_t workspace_bytes, void *dq, void *dkv, float *d_sink,
                           smla_stream_t stream);

/*
 * Block-sparse attention forward at the non-absorbed MLA shape (FlashMLA
 * PR #198, "Summary", item 3: each query block attends only its selected key
 * blocks; "Benchmarks": 192/128 heads, full-causal selection = dense).  One
 * sequence of s tokens.
 *   q            bf16 [s, h_q, 192]
 *   k            bf16 [s, h_kv, 192]; query head h reads KV head h / (h_q / h_kv)
 *   v            bf16 [s, h_kv, 128]
 *   q2k_row_ptr  int32 [ceil(s / q_block) + 1], non-decreasing from 0
 *   q2k_col_idx  int32 [q2k_row_ptr[last]]: the key-block ids of each query
 *                block (may be NULL when there are none).  Row i attends the
 *                keys of every listed id of block i / q_block, each listing
 *                once; ids outside [0, ceil(s / k_block)) are ignored
 *   q_block, k_block  multiples of 64 (the pages' forward uses 256 / 128)
 *   causal       1: only keys j <= i; 0: every key of the listed blocks
 *   out          bf16 [s, h_q, 128] (output)
 *   lse          fp32 [s, h_q] natural-log normaliser (output; +inf for a
 *                row without keys, whose out is 0)
 * The selection arrays are trusted to be consistent (they are read, not
 * checked).  One kernel is enqueued on `stream`.
 */
smla_status sparse_mla_block_sparse_fwd(const void *q, const void *k, const void *v,
                                        const int32_t *q2k_row_ptr, const int32_t *q2k_col_idx,
                                        int32_t s, int32_t h_q, int32_t h_kv, int32_t d_qk,
                                        int32_t d_v, int32_t q_block, int32_t k_block,
                                        int32_t causal, float sm_scale, void *out, float *lse,
                                        smla_stream_t stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char *sparse_mla_last_error(void);

/* Thread-local name of the attention kernel that the last call of
 * sparse_mla_fwd, sparse_mla_decode_fwd, sparse_mla_decode_fwd_split,
 * sparse_mla_decode_fwd_split_noalloc or sparse_mla_bwd on this thread
 * launched ("" if it launched none, or the last such call was another entry
 * point):
 *   "ring"        128 heads, rows of at most 2048 index positions
 *   "wide"        64 heads, or 128 heads with longer rows
 *   "ring_split"  split decode at 128 heads, at most 2048 positions per
 *                 split (the merge kernel follows it)
 *   "split"       other split decode (the wide kernel's split units)
 *   "heads16"     every other head count, and KV tables whose rows the
 *                 others cannot address (above about 550 GB)
 * with a suffix "_big" on all but the last for KV tables above 4 GiB, which
 * those kernels address through a buffer resource rebased per copied row;
 * and for the backward "bwd_key_outer" or "bwd_scatter", its dkv path.
 * The string is static; it is for tests and tools and is not an error
 * channel. */
const char *sparse_mla_last_kernel(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
