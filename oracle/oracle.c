/*
 * CPU oracle for the vocab-parallel embedding and LM-head path.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct C loops that state
 * what the path computes.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library and includes nothing from it.
 *
 * Sources (cited by page title and section):
 *   [TP-vocab]  devpress.csdn.net/amd/6a3de260..., the nano-vllm article on
 *               splitting the vocabulary and the attention heads: section 3
 *               (VocabParallelEmbedding), section 4 (ParallelLMHead),
 *               section 6 (single-process integration check).
 *   [TP-math]   devpress.csdn.net/amd/6a3b3792..., the nano-vllm article on
 *               the mathematics of tensor parallelism: section 5 (Embedding
 *               and LM Head: sum versus concatenation).
 *   [vLLM-1.1]  blog.xiaohansong.com "从零实现 vLLM (1.1)：并行词嵌入
 *               VocabParallelEmbedding", the 12-word rank-by-rank walkthrough
 *               and the nano-vllm source analysis.
 *   [Guide-3.3] caomaolufei.github.io AIInfraGuide "3.3 模型骨架与核心算子",
 *               section 6 (vocab-parallel Embedding and LMHead).
 *
 * Readings taken where the pages are silent or disagree:
 *   - the vocabulary must divide evenly by tp ([vLLM-1.1] asserts it; the
 *     [TP-vocab] listing floors silently);
 *   - a row for an id outside the shard is written as all-zero bits (+0.0);
 *     the placeholder row the formula looks up is never read;
 *   - partial sums add in rank order in fp32 with one final rounding to the
 *     table dtype (round to nearest, ties to even);
 *   - logits are the exact products accumulated in fp64 (no rounding to the
 *     logits dtype here: the comparison tolerance covers that).
 *
 * Parity: every function here is pinned by tests that do not re-type it
 * (printed page values, closed forms, library routines, invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_SHARD 2
#define ORC_ERR_CUSEQ 3

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_I32 0
#define ORC_I64 1

/* ------------------------------------------------------------------ */
/* element decoding                                                    */
/* ------------------------------------------------------------------ */
static int64_t orc_id_at(const void *ids, int itype, int64_t i) {
    if (itype == ORC_I32) return (int64_t)((const int32_t *)ids)[i];
    return ((const int64_t *)ids)[i];
}

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest with ties to even; NaN stays a quiet NaN. */
static uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

static double orc_elem_f64(const void *base, int dtype, int64_t idx) {
    if (dtype == ORC_F32) return (double)((const float *)base)[idx];
    return (double)orc_bf16_to_f32(((const uint16_t *)base)[idx]);
}

static int orc_elem_bytes(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* exported for tests of the rounding rule itself */
uint16_t orc_round_bf16(float f) { return orc_f32_to_bf16(f); }
float orc_widen_bf16(uint16_t h) { return orc_bf16_to_f32(h); }

/* ------------------------------------------------------------------ */
/* shard ownership: [TP-vocab] section 3 __init__, [vLLM-1.1] source   */
/* analysis (per-partition size, start = size * rank, end = start+size) */
/* ------------------------------------------------------------------ */
int orc_shard_range(int64_t vocab, int32_t tp_size, int32_t tp_rank,
                    int64_t *vocab_start, int64_t *vocab_end) {
    if (!vocab_start || !vocab_end) return ORC_ERR_ARG;
    if (vocab < 1 || tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size) return ORC_ERR_SHARD;
    if (vocab % tp_size != 0) return ORC_ERR_SHARD;
    int64_t per = vocab / tp_size;
    *vocab_start = per * (int64_t)tp_rank;
    *vocab_end = *vocab_start + per;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* shard loading: [TP-vocab] section 3 weight_loader, [vLLM-1.1] source */
/* analysis: a rank keeps rows [rank*R, rank*R + R) of the full [V, D]  */
/* table (narrow along dim 0, then copy), element bits unchanged.       */
/* ------------------------------------------------------------------ */
int orc_load_shard(const void *full, int64_t vocab, int64_t dim, int dtype, int32_t tp_size,
                   int32_t tp_rank, void *shard) {
    int64_t start, end;
    int rc = orc_shard_range(vocab, tp_size, tp_rank, &start, &end);
    if (rc != ORC_OK) return rc;
    if (dim < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return ORC_ERR_ARG;
    if (!full || !shard) return ORC_ERR_ARG;
    const int64_t row_bytes = dim * orc_elem_bytes(dtype);
    for (int64_t r = start; r < end; ++r)
        memcpy((char *)shard + (r - start) * row_bytes, (const char *)full + r * row_bytes,
               (size_t)row_bytes);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* steps 1-2 of the masked lookup ([TP-vocab] section 3, [vLLM-1.1]     */
/* steps 1 and 2): mask = start <= x < end; local = mask ? x-start : 0  */
/* ------------------------------------------------------------------ */
int orc_mask_shift(const void *ids, int itype, int64_t n, int64_t vocab_start,
                   int64_t vocab_end, uint8_t *mask, int64_t *local) {
    if (n < 0 || (n > 0 && (!ids || !mask || !local))) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        int64_t x = orc_id_at(ids, itype, i);
        int in_shard = (x >= vocab_start) && (x < vocab_end);
        mask[i] = (uint8_t)in_shard;
        local[i] = in_shard ? (x - vocab_start) : 0;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* one shard's masked lookup, steps 1-4 ([TP-vocab] section 3,          */
/* [vLLM-1.1] steps 1-4, [Guide-3.3] section 6):                        */
/*   out[i,:] = W[x_i - start, :]   if start <= x_i < start + R         */
/*            = +0 (all bits clear) otherwise                           */
/* Element bits are copied: the lookup involves no arithmetic.          */
/* ------------------------------------------------------------------ */
typedef struct {
    const void *ids; int itype; const unsigned char *w; int64_t rows;
    int64_t row_bytes; int64_t start; unsigned char *out; int64_t i0, i1;
} orc_embed_job;

static void orc_embed_range(const orc_embed_job *j) {
    for (int64_t i = j->i0; i < j->i1; ++i) {
        int64_t x = orc_id_at(j->ids, j->itype, i);
        unsigned char *dst = j->out + i * j->row_bytes;
        if (x >= j->start && x < j->start + j->rows)
            memcpy(dst, j->w + (x - j->start) * j->row_bytes, (size_t)j->row_bytes);
        else
            memset(dst, 0, (size_t)j->row_bytes);
    }
}

static void *orc_embed_thread(void *p) { orc_embed_range((const orc_embed_job *)p); return NULL; }

int orc_embed(const void *ids, int itype, int64_t n, const void *weight, int dtype,
              int64_t shard_rows, int64_t dim, int64_t vocab_start, void *out,
              int nthreads) {
    if (n < 0 || dim < 1 || shard_rows < 1) return ORC_ERR_ARG;
    if (n == 0) return ORC_OK;
    if (!ids || !weight || !out) return ORC_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = (int)n;
    int64_t rb = dim * orc_elem_bytes(dtype);
    orc_embed_job *jobs = (orc_embed_job *)calloc((size_t)nthreads, sizeof *jobs);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    if (!jobs || !th) { free(jobs); free(th); return ORC_ERR_ARG; }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (orc_embed_job){ids, itype, (const unsigned char *)weight, shard_rows, rb,
                                  vocab_start, (unsigned char *)out,
                                  n * t / nthreads, n * (t + 1) / nthreads};
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, orc_embed_thread, &jobs[t]);
    orc_embed_range(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(jobs); free(th);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* step 5, the all-reduce sum of partials emulated in one process       */
/* ([TP-vocab] sections 3 and 6, [vLLM-1.1] "模拟 All-Reduce 聚合"):     */
/*   out = P_0 + P_1 + ... + P_{tp-1}, added in rank order in fp32,     */
/*   rounded once to the element type.                                  */
/* ------------------------------------------------------------------ */
int orc_sum_partials(const void *const *parts, int32_t n_parts, int64_t n_elems,
                     int dtype, void *out) {
    if (n_parts < 1 || n_elems < 0) return ORC_ERR_ARG;
    if (n_elems == 0) return ORC_OK;
    if (!parts || !out) return ORC_ERR_ARG;
    for (int r = 0; r < n_parts; ++r) if (!parts[r]) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n_elems; ++i) {
        float acc;
        if (dtype == ORC_F32) {
            acc = ((const float *)parts[0])[i];
            for (int r = 1; r < n_parts; ++r) acc = acc + ((const float *)parts[r])[i];
            ((float *)out)[i] = acc;
        } else {
            acc = orc_bf16_to_f32(((const uint16_t *)parts[0])[i]);
            for (int r = 1; r < n_parts; ++r)
                acc = acc + orc_bf16_to_f32(((const uint16_t *)parts[r])[i]);
            ((uint16_t *)out)[i] = orc_f32_to_bf16(acc);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* prefill last-position select ([Guide-3.3] section 6, ParallelLMHead */
/* forward; [TP-vocab] section 4): last = cu_seqlens[1:] - 1,           */
/* out[s,:] = H[last[s], :].  cu_seqlens must start at 0, rise strictly */
/* and end at the token count; anything else is rejected.               */
/* ------------------------------------------------------------------ */
int orc_last_token_select(const void *hidden, int64_t n_tokens, int64_t dim, int dtype,
                          const int32_t *cu_seqlens, int64_t n_seqs, void *out) {
    if (n_seqs < 0 || n_tokens < 0 || dim < 1) return ORC_ERR_ARG;
    if (!cu_seqlens) return ORC_ERR_ARG;
    if (cu_seqlens[0] != 0) return ORC_ERR_CUSEQ;
    for (int64_t s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] <= cu_seqlens[s]) return ORC_ERR_CUSEQ;
    if ((int64_t)cu_seqlens[n_seqs] != n_tokens) return ORC_ERR_CUSEQ;
    if (n_seqs == 0) return ORC_OK;
    if (!hidden || !out) return ORC_ERR_ARG;
    int64_t rb = dim * orc_elem_bytes(dtype);
    for (int64_t s = 0; s < n_seqs; ++s) {
        int64_t last = (int64_t)cu_seqlens[s + 1] - 1;
        memcpy((unsigned char *)out + s * rb, (const unsigned char *)hidden + last * rb, (size_t)rb);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* one shard's logits, F.linear without bias ([TP-vocab] section 4,     */
/* [Guide-3.3] section 6):  Z[m, j] = sum_k X[m,k] * W[j,k], j < R,      */
/* written at column col_offset + j of a row-major buffer of stride ld  */
/* (the gather-and-concatenate of [TP-vocab] section 6 and [TP-math]    */
/* section 5).  Products and sums are taken in fp64, k ascending.       */
/* ------------------------------------------------------------------ */
typedef struct {
    const void *x; int64_t k_dim; const void *w; int64_t rows; int dtype;
    double *out; int64_t ld; int64_t col_offset; int64_t m0, m1; int64_t j0, j1;
} orc_lm_job;

static void orc_lm_range(const orc_lm_job *jb) {
    for (int64_t m = jb->m0; m < jb->m1; ++m) {
        for (int64_t j = jb->j0; j < jb->j1; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < jb->k_dim; ++k)
                acc += orc_elem_f64(jb->x, jb->dtype, m * jb->k_dim + k) *
                       orc_elem_f64(jb->w, jb->dtype, j * jb->k_dim + k);
            jb->out[m * jb->ld + jb->col_offset + j] = acc;
        }
    }
}

static void *orc_lm_thread(void *p) { orc_lm_range((const orc_lm_job *)p); return NULL; }

int orc_lmhead_f64(const void *x, int64_t m, int64_t dim, const void *weight,
                   int64_t shard_rows, int dtype, double *out, int64_t ld_out,
                   int64_t col_offset, int nthreads) {
    if (m < 0 || dim < 1 || shard_rows < 1 || col_offset < 0) return ORC_ERR_ARG;
    if (col_offset + shard_rows > ld_out) return ORC_ERR_ARG;
    if (m == 0) return ORC_OK;
    if (!x || !weight || !out) return ORC_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    orc_lm_job *jobs = (orc_lm_job *)calloc((size_t)nthreads, sizeof *jobs);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    if (!jobs || !th) { free(jobs); free(th); return ORC_ERR_ARG; }
    /* split whichever of (rows of X, rows of W) is longer across threads */
    int split_m = m >= nthreads;
    for (int t = 0; t < nthreads; ++t) {
        orc_lm_job j = {x, dim, weight, shard_rows, dtype, out, ld_out, col_offset,
                        0, m, 0, shard_rows};
        if (split_m) { j.m0 = m * t / nthreads; j.m1 = m * (t + 1) / nthreads; }
        else { j.j0 = shard_rows * t / nthreads; j.j1 = shard_rows * (t + 1) / nthreads; }
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, orc_lm_thread, &jobs[t]);
    orc_lm_range(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(jobs); free(th);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* greedy pick over the concatenated logits ([TP-vocab] section 4: the  */
/* full-vocabulary logits feed the sampler; the first maximum wins, as */
/* an argmax over a row does): for each row m of a [m_rows, ld] fp64   */
/* buffer, the largest value in columns [0, n_cols) and its column.     */
/* ------------------------------------------------------------------ */
int orc_argmax_rows(const double *logits, int64_t m_rows, int64_t n_cols, int64_t ld,
                    double *max_out, int64_t *idx_out) {
    if (m_rows < 0 || n_cols < 1 || ld < n_cols) return ORC_ERR_ARG;
    if (m_rows == 0) return ORC_OK;
    if (!logits || !max_out || !idx_out) return ORC_ERR_ARG;
    for (int64_t m = 0; m < m_rows; ++m) {
        const double *row = logits + m * ld;
        int64_t best = 0;
        for (int64_t j = 1; j < n_cols; ++j)
            if (row[j] > row[best]) best = j;
        max_out[m] = row[best];
        idx_out[m] = best;
    }
    return ORC_OK;
}

/* single logit, for sampled checks at sizes the full product would take too long */
double orc_logit_f64(const void *x, int64_t dim, const void *weight, int dtype,
                     int64_t m, int64_t j) {
    double acc = 0.0;
    for (int64_t k = 0; k < dim; ++k)
        acc += orc_elem_f64(x, dtype, m * dim + k) * orc_elem_f64(weight, dtype, j * dim + k);
    return acc;
}

/*
 * Log-sum-exp of every row of fp64 logits: lse[m] = log(sum_j exp(z[m][j])),
 * the normaliser of the softmax that turns the gathered logits into sampling
 * probabilities ([Guide-3.3] section 6: compute_logits is kept apart from
 * the forward so that the sampler can take the logits; [TP-vocab] section 4:
 * the shard logits are gathered into the full vocabulary first).  Written
 * with the row's largest logit factored out, lse = mx + log(sum_j
 * exp(z[m][j] - mx)), which is the same number without overflow in exp.
 * Columns are visited in increasing order.
 */
int orc_logsumexp_rows(const double *logits, int64_t m_rows, int64_t n_cols, int64_t ld,
                       double *lse_out) {
    if (m_rows < 0 || n_cols < 1 || ld < n_cols) return ORC_ERR_ARG;
    if (m_rows == 0) return ORC_OK;
    if (!logits || !lse_out) return ORC_ERR_ARG;
    for (int64_t m = 0; m < m_rows; ++m) {
        const double *row = logits + m * ld;
        double mx = row[0];
        for (int64_t j = 1; j < n_cols; ++j)
            if (row[j] > mx) mx = row[j];
        double sum = 0.0;
        for (int64_t j = 0; j < n_cols; ++j) sum += exp(row[j] - mx);
        lse_out[m] = mx + log(sum);
    }
    return ORC_OK;
}
