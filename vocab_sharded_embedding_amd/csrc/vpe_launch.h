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

// out = sum of n_parts partials in rank order (fp32 adds, one rounding).
// dtype: 0 = f32, 1 = bf16.  n_parts in [1, 64].
int launch_sum_partials(const void *const *parts, int n_parts, int64_t n_elems, int dtype,
                        void *out, void *stream);

// logits[i*ld + col_offset + j] = sum_k x[i,k] w[j,k].  dtype: 0 = f32, 1 = bf16.
int launch_lmhead(const void *x, int64_t m, int64_t k, const void *w, int64_t n, int dtype,
                  void *logits, int64_t ld, int64_t col_offset, void *stream);

}  // namespace vpe

#endif
