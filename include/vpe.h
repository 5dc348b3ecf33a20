/*
 * vpe.h - C ABI of the vocab-parallel embedding / LM-head library (libvpe.so).
 *
 * One tensor-parallel rank's share of the two vocabulary-sharded layers of a
 * decoder LLM, as the nano-vllm pages describe them:
 *   - the embedding: the table [V, D] is split by rows into tp contiguous
 *     shards; a shard looks up only the ids it owns and returns zero rows for
 *     the rest, and the ranks' partial outputs are summed;
 *   - the LM head: the same [V/tp, D] shard produces the logits of the words
 *     it owns, and the ranks' logits are concatenated along the vocabulary.
 *
 * Sources (page and section):
 *   [TP-vocab]  devpress.csdn.net/amd/6a3de260..., nano-vllm article on the
 *               vocab and head split: section 3 (VocabParallelEmbedding),
 *               section 4 (ParallelLMHead), section 6 (integration check).
 *   [TP-math]   devpress.csdn.net/amd/6a3b3792..., nano-vllm article on the
 *               mathematics of tensor parallelism: section 5.
 *   [vLLM-1.1]  blog.xiaohansong.com, "从零实现 vLLM (1.1)：并行词嵌入
 *               VocabParallelEmbedding": the rank-by-rank walkthrough and the
 *               nano-vllm source analysis.
 *   [Guide-3.3] caomaolufei.github.io AIInfraGuide, "3.3 模型骨架与核心算子",
 *               section 6 (vocab-parallel Embedding and LMHead).
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory (or memory
 *     the device can address) that the caller allocated and owns; the library
 *     allocates nothing, keeps no state between calls and never synchronises
 *     (vpe_lmhead_logsumexp_noalloc aside: it uses a static device array the
 *     library holds per GPU, see there).
 *   - Tensors are dense and row-major unless a stride is given.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     on it and the call returns without waiting for it.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-VPE_OK status means nothing was enqueued, except VPE_ERR_LAUNCH,
 *     which reports a launch the HIP runtime refused.
 *   - Values held in device memory (ids, cu_seqlens) are not validated: their
 *     out-of-range cases have defined results, stated per call.
 *   - Calls are thread-safe (no shared mutable state), except that calls of
 *     vpe_lmhead_logsumexp_noalloc on one GPU share that GPU's static array.
 */
#ifndef VPE_H
#define VPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vpe_status {
    VPE_OK = 0,
    VPE_ERR_NULL = 1,   /* a required pointer is NULL */
    VPE_ERR_SHAPE = 2,  /* a size is negative, zero where it may not be, or too large */
    VPE_ERR_DTYPE = 3,  /* unknown element or index type */
    VPE_ERR_ALIGN = 4,  /* a pointer is not aligned to its element size */
    VPE_ERR_SHARD = 5,  /* tp split invalid: V % tp != 0, rank outside [0, tp) */
    VPE_ERR_LAUNCH = 6, /* the HIP runtime refused a kernel launch */
    VPE_ERR_RANGE = 7,  /* an output column range does not fit its row stride */
    VPE_ERR_WORKSPACE = 8 /* a workspace is smaller than the call needs */
} vpe_status;

typedef enum vpe_dtype {
    VPE_F32 = 0,  /* IEEE binary32 */
    VPE_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} vpe_dtype;

typedef enum vpe_itype {
    VPE_I32 = 0,  /* int32 token ids */
    VPE_I64 = 1   /* int64 token ids */
} vpe_itype;

/* Largest number of partials vpe_sum_partials accepts in one call. */
#define VPE_MAX_PARTS 64

/*
 * Shard ownership of rank `tp_rank` among `tp_size` ranks over a vocabulary of
 * `vocab` ids ([TP-vocab] section 3 constructor; [vLLM-1.1] source analysis):
 * shard size R = vocab / tp_size, *vocab_start = R * tp_rank,
 * *vocab_end = *vocab_start + R.  Ranks own contiguous blocks in rank order.
 *
 * Host-only; touches no device.  Pointers are host pointers.
 * Errors: VPE_ERR_NULL (output pointer NULL); VPE_ERR_SHARD (vocab < 1,
 * tp_size < 1, tp_rank outside [0, tp_size), or vocab % tp_size != 0 -- the
 * vocabulary must split evenly, as [vLLM-1.1] asserts).
 */
vpe_status vpe_shard_range(int64_t vocab, int32_t tp_size, int32_t tp_rank,
                           int64_t *vocab_start, int64_t *vocab_end);

/*
 * One shard's masked embedding lookup, steps 1-4 of [TP-vocab] section 3
 * (mask, shift to a local index, look up, clear rows the shard does not own);
 * [vLLM-1.1] steps 1-4; [Guide-3.3] section 6:
 *
 *   out[i, :] = weight[ids[i] - vocab_start, :]  if vocab_start <= ids[i] < vocab_start + shard_rows
 *             = all-zero bits (+0.0)             otherwise
 *
 * ids     device, [n] of `itype`, any values (ids outside the shard, negative
 *         ids and ids >= V all give zero rows; no row is read for them).
 * weight  device, [shard_rows, dim] of `dt`: the shard (rows vocab_start ..
 *         vocab_start + shard_rows - 1 of the full table).
 * out     device, [n, dim] of `dt`; must not overlap ids or weight.
 * The copy is bit-exact (no arithmetic touches the values).
 * n == 0 is a no-op.  The full (tp = 1) lookup is vocab_start = 0,
 * shard_rows = V.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (n < 0, dim < 1, shard_rows < 1),
 * VPE_ERR_DTYPE, VPE_ERR_ALIGN (a pointer not aligned to its element size),
 * VPE_ERR_RANGE (vocab_start < 0, or vocab_start + shard_rows past INT64_MAX).
 */
vpe_status vpe_embed(const void *ids, vpe_itype itype, int64_t n,
                     const void *weight, vpe_dtype dt, int64_t shard_rows, int64_t dim,
                     int64_t vocab_start, void *out, void *stream);

/*
 * Step 5 of [TP-vocab] section 3, the all-reduce sum of the ranks' partial
 * embeddings, done on one device ([TP-vocab] section 6 and [vLLM-1.1]
 * "模拟 All-Reduce 聚合" emulate it the same way):
 *
 *   out[e] = partials[0][e] + partials[1][e] + ... + partials[n_parts-1][e]
 *
 * added in rank order in fp32 and rounded once to `dt` (round to nearest,
 * ties to even).  With masked partials exactly one term per row is non-zero,
 * so the sum is the owner's row bit for bit (tables without -0.0 entries).
 *
 * partials  HOST array of n_parts device pointers, each [n_elems] of `dt`.
 * out       device, [n_elems] of `dt`; may be exactly equal to one of the
 *           partials (in-place sum), must not partially overlap any.
 * n_elems == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (n_parts outside [1, VPE_MAX_PARTS],
 * n_elems < 0), VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_sum_partials(const void *const *partials, int32_t n_parts, int64_t n_elems,
                            vpe_dtype dt, void *out, void *stream);

/*
 * Prefill last-position select before the LM head ([Guide-3.3] section 6,
 * ParallelLMHead.forward; [TP-vocab] section 4):
 *
 *   out[s, :] = hidden[cu_seqlens[s + 1] - 1, :]   for s in [0, n_seqs)
 *
 * hidden      device, [n_tokens, dim] of `dt` (all packed sequences).
 * cu_seqlens  device, int32 [n_seqs + 1]: 0, then cumulative sequence lengths.
 * out         device, [n_seqs, dim] of `dt`.
 * Precondition: cu_seqlens starts at 0, rises strictly and ends at n_tokens.
 * A row whose index cu_seqlens[s+1]-1 falls outside [0, n_tokens) is written
 * as zeros and nothing is read for it (no out-of-bounds access).
 * n_seqs == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (n_tokens < 0, n_seqs < 0, dim < 1,
 * n_tokens >= 2^31), VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_last_token_select(const void *hidden, int64_t n_tokens, int64_t dim,
                                 vpe_dtype dt, const int32_t *cu_seqlens, int64_t n_seqs,
                                 void *out, void *stream);

/*
 * One shard's logits, F.linear with no bias ([TP-vocab] section 4,
 * [Guide-3.3] section 6), written at the shard's column offset of the full
 * vocabulary (the gather-and-concatenate of [TP-vocab] section 6 and
 * [TP-math] section 5):
 *
 *   logits[i * ld_out + col_offset + j] = sum_k x[i, k] * weight[j, k]
 *                                          for i < m, j < shard_rows
 *
 * x       device, [m, dim] of `dt` (last-position hidden states).
 * weight  device, [shard_rows, dim] of `dt` (the same shard layout as
 *         vpe_embed: vocabulary rows, dim contiguous).
 * logits  device, row-major with row stride ld_out elements, of `dt`; only
 *         columns [col_offset, col_offset + shard_rows) of rows [0, m) are
 *         written.  For one shard alone: ld_out = shard_rows, col_offset = 0.
 *         To concatenate tp shards: ld_out = V, col_offset = vocab_start.
 * Products are accumulated in fp32 (order unspecified) and rounded once to
 * `dt` (round to nearest, ties to even).
 * m == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (m < 0, m > 2^21, dim < 1,
 * dim > 2^20, shard_rows < 1), VPE_ERR_RANGE (col_offset < 0 or col_offset + shard_rows > ld_out),
 * VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_lmhead(const void *x, int64_t m, int64_t dim, const void *weight,
                      int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                      int64_t col_offset, void *stream);

/*
 * Prefill LM head with the last-position select folded in: the logits of the
 * last position of every packed sequence, read straight out of the prefill
 * activations ([Guide-3.3] section 6: only the last position of each
 * sequence is projected; [TP-vocab] sections 4 and 6 for the shard product
 * and its column offset).  Equal to vpe_last_token_select followed by
 * vpe_lmhead, without the [n_seqs, dim] intermediate or its launch:
 *
 *   logits[s * ld_out + col_offset + j] = sum_k hidden[cu_seqlens[s+1]-1, k] * weight[j, k]
 *
 * hidden      device, [n_tokens, dim] of `dt`.
 * cu_seqlens  device, int32 [n_seqs + 1] (same precondition as
 *             vpe_last_token_select; a sequence whose last index falls
 *             outside [0, n_tokens) gets all-zero logits, nothing is read).
 * weight, logits, ld_out, col_offset, accumulation and rounding: as vpe_lmhead.
 * n_seqs == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (n_tokens < 0 or >= 2^31, n_seqs < 0
 * or > 2^21, dim < 1 or > 2^20, shard_rows < 1), VPE_ERR_RANGE,
 * VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_lmhead_prefill(const void *hidden, int64_t n_tokens, int64_t dim,
                              const int32_t *cu_seqlens, int64_t n_seqs, const void *weight,
                              int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                              int64_t col_offset, void *stream);

/*
 * One rank's shard of the full table, loaded on the device: the rank keeps
 * rows [tp_rank * R, tp_rank * R + R) of the [vocab, dim] table, R = vocab /
 * tp_size ([TP-vocab] section 3 weight_loader: narrow along the vocabulary
 * dimension, then copy into the parameter; [vLLM-1.1] source analysis).
 *   full   device [vocab, dim] row-major, dtype dt (read only)
 *   shard  device [R, dim] row-major, written; must not overlap the rows
 *          copied from `full`
 * Element bits are copied unchanged.  The same shard serves vpe_embed and
 * vpe_lmhead (tied tables, [Guide-3.3] section 8).
 * Errors: VPE_ERR_DTYPE, VPE_ERR_SHAPE (vocab or dim < 1, too large),
 * VPE_ERR_SHARD (vocab % tp_size != 0, rank out of range), VPE_ERR_NULL,
 * VPE_ERR_ALIGN (pointers not aligned to the element size), VPE_ERR_RANGE
 * (shard overlaps its source rows).
 */
vpe_status vpe_load_shard(const void *full, int64_t vocab, int64_t dim, vpe_dtype dt,
                          int32_t tp_size, int32_t tp_rank, void *shard, void *stream);

/*
 * Greedy pick over the vocabulary without materialising the logits.  The
 * full-vocabulary logits exist to feed the sampler ([TP-vocab] section 4:
 * each rank's shard of the logits is gathered and concatenated; [Guide-3.3]
 * section 6); for greedy sampling each rank can instead reduce its shard to
 * (largest logit, its id) and the ranks combine those.  Here one 64-bit key
 * per row holds the running pick:
 *
 *   key = (order(v) << 32) | (0xFFFFFFFF - id)
 *
 * (order() maps binary32 bits to an unsigned integer ordered like the
 * values), so the largest key is the largest logit and, among equal logits,
 * the smallest id: the first maximum of the concatenated row.  Shards fold
 * their candidates in with atomic max, so calling vpe_lmhead_argmax for every
 * rank's shard on the same `best` is the combine.
 *
 * Sequence: vpe_argmax_init(best) once; vpe_lmhead_argmax(...) per shard;
 * vpe_argmax_decode(best) -> (max logit, token id) per row.  All on streams
 * ordered by the caller; concurrent shard calls on one `best` are fine (the
 * fold is an atomic max).  vpe_argmax_decode_clear also resets the keys it
 * reads, so a decode loop needs vpe_argmax_init only before its first step.
 *
 * The logit compared is the one vpe_lmhead would store: fp32 accumulation
 * rounded to `dt` (round to nearest even), widened back to fp32.
 */

/* best: device uint64 [m], m <= 2^21; sets every key to 0 (below every real
 * logit).  Errors: VPE_ERR_SHAPE, VPE_ERR_NULL, VPE_ERR_ALIGN (best not
 * 8-byte aligned). */
vpe_status vpe_argmax_init(uint64_t *best, int64_t m, void *stream);

/*
 * Folds one shard's logits x . weight^T into best[m]: for each row i the
 * largest logit over the shard's rows j, with id vocab_start + j.
 * x, weight, dt, dim, shard_rows: as vpe_lmhead.  best: device uint64 [m],
 * initialised by vpe_argmax_init.  m == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (m < 0 or > 2^21, dim < 1 or > 2^20,
 * shard_rows < 1), VPE_ERR_RANGE (vocab_start < 0 or vocab_start +
 * shard_rows >= 2^32), VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_lmhead_argmax(const void *x, int64_t m, int64_t dim, const void *weight,
                             int64_t shard_rows, vpe_dtype dt, int64_t vocab_start,
                             uint64_t *best, void *stream);

/*
 * vpe_lmhead_argmax over the last position of every packed sequence: the
 * prefill select folded into the pick as vpe_lmhead_prefill folds it into the
 * logits ([Guide-3.3] section 6: prefill logits come from each sequence's
 * last position; [TP-vocab] section 4).  Row s of best takes the largest
 * logit of hidden[cu_seqlens[s+1]-1] . weight^T with its id.
 * hidden, n_tokens, dim, cu_seqlens, n_seqs: as vpe_lmhead_prefill (a
 * sequence whose last index falls outside [0, n_tokens) folds in a row of
 * zero logits, nothing is read).  weight, shard_rows, dt, vocab_start: as
 * vpe_lmhead_argmax; best: device uint64 [n_seqs] from vpe_argmax_init.
 * n_seqs == 0 is a no-op.  The keys equal those of vpe_last_token_select
 * followed by vpe_lmhead_argmax on the selected rows.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (as vpe_lmhead_prefill),
 * VPE_ERR_RANGE (as vpe_lmhead_argmax), VPE_ERR_DTYPE, VPE_ERR_ALIGN.
 */
vpe_status vpe_lmhead_prefill_argmax(const void *hidden, int64_t n_tokens, int64_t dim,
                                     const int32_t *cu_seqlens, int64_t n_seqs,
                                     const void *weight, int64_t shard_rows, vpe_dtype dt,
                                     int64_t vocab_start, uint64_t *best, void *stream);

/*
 * max_logit[i] (device float [m], may be NULL) and token[i] (device int64
 * [m], may be NULL, not both) decoded from best[i], m <= 2^21.  A row no
 * shard folded into decodes to (NaN with the sign bit set, 0xFFFFFFFF).
 * Errors: VPE_ERR_SHAPE, VPE_ERR_NULL, VPE_ERR_ALIGN.
 */
vpe_status vpe_argmax_decode(const uint64_t *best, int64_t m, float *max_logit, int64_t *token,
                             void *stream);

/*
 * vpe_argmax_decode, after which every best[i] is 0 again (each key is
 * cleared by the thread that read it, in the same kernel), as
 * vpe_argmax_init would leave it: the next step's folds can follow without
 * an init call.  Same arguments, outputs and errors as vpe_argmax_decode.
 */
vpe_status vpe_argmax_decode_clear(uint64_t *best, int64_t m, float *max_logit,
                                   int64_t *token, void *stream);

/*
 * Log-sum-exp of the logits rows, the normaliser of the softmax the sampler
 * takes over the gathered logits ([Guide-3.3] section 6: compute_logits is
 * kept apart so that the sampler can take the logits; [TP-vocab] section 4:
 * each rank's shard of the logits is gathered into the full vocabulary
 * first).  Split over vocabulary shards it needs no gather: each rank reduces
 * its shard to one value per row,
 *
 *   shard_lse[i] = log(sum_j exp(z[i, j]))   over the shard's columns j,
 *
 * and the ranks combine those ([M] floats each) with
 *
 *   lse[i] = log(sum_r exp(shard_lse_r[i])).
 *
 * z is the logit as vpe_lmhead stores it: fp32 accumulation rounded to `dt`
 * (round to nearest even), widened to fp32.  The exponentials, sums and
 * logarithm are taken in fp32 with each set's largest logit factored out (no
 * overflow for any finite logits), merged in a fixed order: results do not
 * depend on timing.  Rows holding an infinite or NaN logit give an infinite
 * or NaN value.
 */

/* Bytes of workspace vpe_lmhead_logsumexp needs at most for m rows of a
 * shard of shard_rows rows (8 bytes per row per 64 shard rows).
 * Host-only.  Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (m < 0, shard_rows < 1,
 * or a size past INT64_MAX). */
vpe_status vpe_lmhead_logsumexp_workspace(int64_t m, int64_t shard_rows, int64_t *bytes);

/*
 * One shard's logits, as vpe_lmhead, and every row's shard_lse.
 * x, m, dim, weight, shard_rows, dt: as vpe_lmhead.
 * logits, ld_out, col_offset: as vpe_lmhead, or logits == NULL: nothing is
 *          stored (ld_out and col_offset are then ignored).
 * shard_lse  device float [m], written.
 * workspace  device, at least vpe_lmhead_logsumexp_workspace(m, shard_rows)
 *          bytes, 8-byte aligned; owned by the caller, needs no
 *          initialisation, holds nothing the caller uses afterwards, and must
 *          not be shared by calls that may run at the same time.
 * m == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (as vpe_lmhead_argmax), VPE_ERR_RANGE
 * (logits given and its column range does not fit ld_out), VPE_ERR_DTYPE,
 * VPE_ERR_ALIGN, VPE_ERR_WORKSPACE (workspace_bytes below the size above).
 */
vpe_status vpe_lmhead_logsumexp(const void *x, int64_t m, int64_t dim, const void *weight,
                                int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                                int64_t col_offset, float *shard_lse, void *workspace,
                                int64_t workspace_bytes, void *stream);

/*
 * vpe_lmhead_logsumexp over the last position of every packed sequence: the
 * prefill select folded in as vpe_lmhead_prefill folds it ([Guide-3.3]
 * section 6: in prefill only each sequence's last position is projected, and
 * its logits go to the sampler; [TP-vocab] section 4 for the shard product).
 * Row s of the logits (when stored) and shard_lse[s] are those of
 * hidden[cu_seqlens[s+1]-1] . weight^T.
 * hidden, n_tokens, dim, cu_seqlens, n_seqs: as vpe_lmhead_prefill (a
 * sequence whose last index falls outside [0, n_tokens) gets a row of zero
 * logits, nothing is read, and so shard_lse = log(shard_rows)).
 * weight, shard_rows, dt, logits, ld_out, col_offset, shard_lse: as
 * vpe_lmhead_logsumexp with m = n_seqs; workspace: at least
 * vpe_lmhead_logsumexp_workspace(n_seqs, shard_rows) bytes, as there.
 * n_seqs == 0 is a no-op.  Logits and values equal those of
 * vpe_last_token_select followed by vpe_lmhead_logsumexp on the selected
 * rows, bit for bit.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (as vpe_lmhead_prefill), VPE_ERR_RANGE,
 * VPE_ERR_DTYPE, VPE_ERR_ALIGN, VPE_ERR_WORKSPACE.
 */
vpe_status vpe_lmhead_prefill_logsumexp(const void *hidden, int64_t n_tokens, int64_t dim,
                                        const int32_t *cu_seqlens, int64_t n_seqs,
                                        const void *weight, int64_t shard_rows, vpe_dtype dt,
                                        void *logits, int64_t ld_out, int64_t col_offset,
                                        float *shard_lse, void *workspace,
                                        int64_t workspace_bytes, void *stream);

/* Bytes of the static device array vpe_lmhead_logsumexp_noalloc uses on each
 * GPU (held from the first call on that GPU until the process ends). */
#define VPE_NOALLOC_SCRATCH_BYTES (16 << 20)

/*
 * vpe_lmhead_logsumexp without a workspace, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates nothing: the tile pairs go to a
 * static array of VPE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on (the GPU of `stream`; the current one for the NULL stream).
 * Arguments and results as vpe_lmhead_logsumexp, bit for bit.
 * The array is shared by every call on that GPU and keeps nothing a call
 * needs from an earlier one: calls on one GPU that may overlap in time (on
 * different streams, or from several threads) race and must be ordered by the
 * caller, e.g. on one stream.
 * Errors: as vpe_lmhead_logsumexp (except those of the workspace arguments);
 * VPE_ERR_WORKSPACE, with nothing enqueued, when the call needs more than
 * VPE_NOALLOC_SCRATCH_BYTES (8 bytes per row per W tile: the chosen tiles
 * are 64 to 320 shard rows wide, so m * shard_rows / 64 * 8 bytes always
 * fits); VPE_ERR_LAUNCH also when the array's device address cannot be had.
 */
vpe_status vpe_lmhead_logsumexp_noalloc(const void *x, int64_t m, int64_t dim, const void *weight,
                                        int64_t shard_rows, vpe_dtype dt, void *logits,
                                        int64_t ld_out, int64_t col_offset, float *shard_lse,
                                        void *stream);

/*
 * The ranks' shard_lse values combined into the log-sum-exp of the full
 * rows: lse[i] = log(sum_r exp(shard_lse[r][i])), r in shard order (the
 * exchange step of the log-sum-exp, done on one device as vpe_sum_partials
 * does the embedding's).
 * shard_lse  HOST array of n_parts device pointers, each float [m].
 * lse        device float [m]; may equal one of the inputs.
 * m == 0 is a no-op.
 * Errors: VPE_ERR_NULL, VPE_ERR_SHAPE (n_parts outside [1, VPE_MAX_PARTS],
 * m < 0), VPE_ERR_ALIGN.
 */
vpe_status vpe_logsumexp_combine(const float *const *shard_lse, int32_t n_parts, int64_t m,
                                 float *lse, void *stream);

/* Static, NUL-terminated name of a status code ("VPE_OK", ...). */
const char *vpe_status_string(vpe_status s);

#ifdef __cplusplus
}
#endif

#endif /* VPE_H */
