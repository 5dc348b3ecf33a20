// Internal interface between the validating C-ABI layer (vpe_api.cpp, plain
// C++ with no HIP headers) and the kernel launchers (*.hip).  Every launcher
// receives arguments the API layer has already validated, enqueues its
// kernels on `stream` (a hipStream_t) and returns 0, or the hipError_t value
// the runtime reported for the launch.
#ifndef VPE_LAUNCH_H
#define VPE_LAUNCH_H

#include <stdint.h>

namespace vpe {

// out[i] = rows[id_i - start] for owned ids, zero bits otherwise.
// itype: 0 = int32 ids, 1 = int64 ids.  row_bytes = dim * element size.
int launch_embed(const void *ids, int itype, int64_t n, const void *weight,
                 int64_t shard_rows, int64_t row_bytes, int64_t vocab_start,
                 void *out, void *stream);

// out[s] = hidden[cu[s+1]-1] (zero row when that index is outside [0, n_tokens)).
int launch_last_token_select(const void *hidden, int64_t n_tokens, int64_t row_bytes,
                             const int32_t *cu_seqlens, int64_t n_seqs, void *out,
                             void *stream);

// dst[0, n_bytes) = src[0, n_bytes) (non-overlapping device buffers).
int launch_copy_bytes(const void *src, void *dst, int64_t n_bytes, void *stream);

// out = sum of n_parts partials in rank order (fp32 adds, one rounding).
// dtype: 0 = f32, 1 = bf16.  n_parts in [1, 64].
int launch_sum_partials(const void *const *parts, int n_parts, int64_t n_elems, int dtype,
                        void *out, void *stream);

// logits[i*ld + col_offset + j] = sum_k x[i,k] w[j,k].  dtype: 0 = f32, 1 = bf16.
// With cu != nullptr, x is hidden [n_tokens, k] and row i of the product is
// hidden[cu[i+1] - 1] (prefill: last position of packed sequence i).
// With best != nullptr, no logits are stored: each row's largest logit (as
// rounded to the dtype) and its id (id_base + column) are folded into the
// 64-bit key best[i] by atomic max.
// With lse_part != nullptr, every W tile also writes each row's log-sum-exp
// pair (tile maximum, sum of exp(logit - maximum)) over its columns into
// lse_part ([m][tiles] pairs of floats, at most lse_cap pairs), and a second
// kernel merges them into shard_lse[i] = log(sum_j exp(logit[i, j])) over the
// shard.  logits may then be nullptr (nothing stored).  Returns kErrWorkspace,
// launching nothing, when the pairs would not fit lse_cap.
int launch_lmhead(const void *x, int64_t m, int64_t k, const void *w, int64_t n, int dtype,
                  void *logits, int64_t ld, int64_t col_offset, void *stream,
                  const int32_t *cu = nullptr, int64_t n_tokens = 0, uint64_t *best = nullptr,
                  int64_t id_base = 0, float *lse_part = nullptr, int64_t lse_cap = 0,
                  float *shard_lse = nullptr);

// A launcher's status when a caller-sized buffer is too small for the launch
// it chose (no HIP error code is negative).
constexpr int kErrWorkspace = -1;

// Narrowest W tile of any LM-head kernel: a launch writes at most
// ceil(n / kMinTileRows) log-sum-exp pairs per row.
constexpr int64_t kMinTileRows = 64;

// Bytes of the static per-device array the allocation-free log-sum-exp uses
// for its tile pairs (8 bytes per row per W tile).
constexpr int64_t kNoAllocScratchBytes = int64_t(16) << 20;

// launch_lmhead with lse_part = that array (at most kNoAllocScratchBytes / 8
// pairs; kErrWorkspace beyond), on the device `stream` belongs to.  Allocates
// nothing.  Calls that overlap on one device share the array and race.
int launch_lmhead_logsumexp_noalloc(const void *x, int64_t m, int64_t k, const void *w,
                                    int64_t n, int dtype, void *logits, int64_t ld,
                                    int64_t col_offset, float *shard_lse, void *stream);

// lse[i] = log(sum_r exp(parts[r][i])) over n_parts <= 64 shards, in shard order.
int launch_logsumexp_combine(const float *const *parts, int n_parts, int64_t m, float *lse,
                             void *stream);

// best[i] = 0 for i < m.
int launch_argmax_init(uint64_t *best, int64_t m, void *stream);

// value[i], id[i] decoded from best[i] (either output may be null).
int launch_argmax_decode(const uint64_t *best, int64_t m, float *value, int64_t *id,
                         void *stream);

// As launch_argmax_decode, then best[i] = 0.
int launch_argmax_decode_clear(uint64_t *best, int64_t m, float *value, int64_t *id,
                               void *stream);

}  // namespace vpe

#endif
