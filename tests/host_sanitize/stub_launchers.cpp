// Host-only stand-ins for the kernel launchers, for the sanitized build of the
// validation layer: each records what it was asked to launch and touches no
// memory behind the pointers it receives.
#include <stdint.h>

#include "../../vocab_sharded_embedding_amd/csrc/vpe_launch.h"
#include "stub_record.h"

stub_call g_last;

namespace vpe {

int launch_embed(const void *ids, int itype, int64_t n, const void *weight, int64_t shard_rows,
                 int64_t row_bytes, int64_t vocab_start, void *out, void *) {
  g_last = stub_call{"embed", ids, weight, out, n, shard_rows, row_bytes, vocab_start, itype, 0};
  return 0;
}

int launch_last_token_select(const void *hidden, int64_t n_tokens, int64_t row_bytes,
                             const int32_t *cu, int64_t n_seqs, void *out, void *) {
  g_last = stub_call{"select", hidden, cu, out, n_tokens, n_seqs, row_bytes, 0, 0, 0};
  return 0;
}

int launch_sum_partials(const void *const *parts, int n_parts, int64_t n_elems, int dtype,
                        void *out, void *) {
  g_last = stub_call{"sum", parts[0], parts[n_parts - 1], out, n_elems, n_parts, 0, 0, dtype, 0};
  return 0;
}

int launch_lmhead(const void *x, int64_t m, int64_t k, const void *w, int64_t n, int dtype,
                  void *logits, int64_t ld, int64_t col_offset, void *, const int32_t *cu,
                  int64_t n_tokens, uint64_t *best, int64_t id_base, float *lse_part,
                  int64_t lse_cap, float *shard_lse) {
  g_last = stub_call{lse_part ? (cu ? "lmhead_prefill_logsumexp" : "lmhead_logsumexp")
                     : best   ? (cu ? "lmhead_prefill_argmax" : "lmhead_argmax")
                              : (cu ? "lmhead_prefill" : "lmhead"),
                     x, w, best ? static_cast<void *>(best) : logits,
                     m, n, k, best ? id_base : col_offset, dtype, cu ? n_tokens : ld,
                     lse_part, lse_cap, shard_lse};
  return 0;
}

int launch_lmhead_logsumexp_noalloc(const void *x, int64_t m, int64_t k, const void *w,
                                    int64_t n, int dtype, void *logits, int64_t ld,
                                    int64_t col_offset, float *shard_lse, void *) {
  g_last = stub_call{"lmhead_logsumexp_noalloc", x, w, logits, m, n, k, col_offset, dtype, ld,
                     nullptr, 0, shard_lse};
  return 0;
}

int launch_logsumexp_combine(const float *const *parts, int n_parts, int64_t m, float *lse,
                             void *) {
  g_last = stub_call{"logsumexp_combine", parts[0], parts[n_parts - 1], lse, m, n_parts, 0, 0, 0,
                     0};
  return 0;
}

int launch_argmax_init(uint64_t *best, int64_t m, void *) {
  g_last = stub_call{"argmax_init", best, nullptr, best, m, 0, 0, 0, 0, 0};
  return 0;
}

int launch_argmax_decode(const uint64_t *best, int64_t m, float *value, int64_t *id, void *) {
  g_last = stub_call{"argmax_decode", best, value, id, m, 0, 0, 0, 0, 0};
  return 0;
}

int launch_argmax_decode_clear(uint64_t *best, int64_t m, float *value, int64_t *id, void *) {
  g_last = stub_call{"argmax_decode_clear", best, value, id, m, 0, 0, 0, 0, 0};
  return 0;
}

int launch_copy_bytes(const void *src, void *dst, int64_t n_bytes, void *) {
  g_last = stub_call{"copy", src, nullptr, dst, n_bytes, 0, 0, 0, 0, 0};
  return 0;
}

}  // namespace vpe
