// The C ABI of libvpe.so: argument validation and dispatch to the kernel
// launchers.  Plain C++ with no HIP headers: everything here runs on the host
// before any HIP call, so every rejected call enqueues nothing.  The exported
// entry points and their contracts are declared in include/vpe.h.
#include "../../include/vpe.h"

#include <stdint.h>

#include "vpe_launch.h"

namespace {

bool known_dtype(vpe_dtype dt) { return dt == VPE_F32 || dt == VPE_BF16; }
bool known_itype(vpe_itype it) { return it == VPE_I32 || it == VPE_I64; }
int64_t dtype_bytes(vpe_dtype dt) { return dt == VPE_F32 ? 4 : 2; }
int64_t itype_bytes(vpe_itype it) { return it == VPE_I32 ? 4 : 8; }

bool aligned(const void *p, int64_t bytes) {
  return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(bytes)) == 0;
}

vpe_status launched(int rc) {
  if (rc == vpe::kErrWorkspace) return VPE_ERR_WORKSPACE;
  return rc == 0 ? VPE_OK : VPE_ERR_LAUNCH;
}

// Largest number of log-sum-exp pairs one LM-head call writes: one per row
// per W tile, tiles at least kMinTileRows rows wide (or -1 on overflow).
int64_t lse_pairs_bound(int64_t m, int64_t shard_rows) {
  // ceil(shard_rows / kMinTileRows) without forming shard_rows + kMinTileRows - 1
  const int64_t tiles = shard_rows / vpe::kMinTileRows + (shard_rows % vpe::kMinTileRows != 0);
  if (m > 0 && tiles > INT64_MAX / 8 / m) return -1;
  return m * tiles;
}

// Largest element count any single tensor may have (far above what one
// device holds): indexes inside the kernels are 64-bit and every grid stays
// below 2^32 work-items per dimension at this size.
constexpr int64_t kMaxElems = int64_t(1) << 39;

}  // namespace

extern "C" {

vpe_status vpe_shard_range(int64_t vocab, int32_t tp_size, int32_t tp_rank,
                           int64_t *vocab_start, int64_t *vocab_end) {
  if (!vocab_start || !vocab_end) return VPE_ERR_NULL;
  if (vocab < 1 || tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size) return VPE_ERR_SHARD;
  if (vocab % tp_size != 0) return VPE_ERR_SHARD;
  const int64_t rows = vocab / tp_size;
  *vocab_start = rows * tp_rank;
  *vocab_end = *vocab_start + rows;
  return VPE_OK;
}

vpe_status vpe_embed(const void *ids, vpe_itype itype, int64_t n, const void *weight,
                     vpe_dtype dt, int64_t shard_rows, int64_t dim, int64_t vocab_start,
                     void *out, void *stream) {
  if (!known_dtype(dt) || !known_itype(itype)) return VPE_ERR_DTYPE;
  if (n < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (n > kMaxElems / dim || shard_rows > kMaxElems / dim) return VPE_ERR_SHAPE;
  // the shard's ids [vocab_start, vocab_start + shard_rows) must be representable
  if (vocab_start < 0 || vocab_start > INT64_MAX - shard_rows) return VPE_ERR_RANGE;
  if (n == 0) return VPE_OK;
  if (!ids || !weight || !out) return VPE_ERR_NULL;
  if (!aligned(ids, itype_bytes(itype)) || !aligned(weight, dtype_bytes(dt)) ||
      !aligned(out, dtype_bytes(dt)))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_embed(ids, itype == VPE_I32 ? 0 : 1, n, weight, shard_rows,
                                    dim * dtype_bytes(dt), vocab_start, out, stream));
}

vpe_status vpe_sum_partials(const void *const *partials, int32_t n_parts, int64_t n_elems,
                            vpe_dtype dt, void *out, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (n_parts < 1 || n_parts > VPE_MAX_PARTS || n_elems < 0 || n_elems > kMaxElems)
    return VPE_ERR_SHAPE;
  if (n_elems == 0) return VPE_OK;
  if (!partials || !out) return VPE_ERR_NULL;
  for (int32_t r = 0; r < n_parts; ++r) {
    if (!partials[r]) return VPE_ERR_NULL;
    if (!aligned(partials[r], dtype_bytes(dt))) return VPE_ERR_ALIGN;
  }
  if (!aligned(out, dtype_bytes(dt))) return VPE_ERR_ALIGN;
  return launched(vpe::launch_sum_partials(partials, n_parts, n_elems, dt == VPE_BF16 ? 1 : 0,
                                           out, stream));
}

vpe_status vpe_last_token_select(const void *hidden, int64_t n_tokens, int64_t dim,
                                 vpe_dtype dt, const int32_t *cu_seqlens, int64_t n_seqs,
                                 void *out, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (n_tokens < 0 || n_seqs < 0 || dim < 1) return VPE_ERR_SHAPE;
  // cu_seqlens holds int32 positions, so the token count must fit in int32
  if (n_tokens > INT32_MAX || n_tokens > kMaxElems / dim || n_seqs > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (n_seqs == 0) return VPE_OK;
  if (!hidden || !cu_seqlens || !out) return VPE_ERR_NULL;
  if (!aligned(hidden, dtype_bytes(dt)) || !aligned(out, dtype_bytes(dt)) ||
      !aligned(cu_seqlens, 4))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_last_token_select(hidden, n_tokens, dim * dtype_bytes(dt),
                                                cu_seqlens, n_seqs, out, stream));
}

vpe_status vpe_lmhead(const void *x, int64_t m, int64_t dim, const void *weight,
                      int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                      int64_t col_offset, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (m < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (m > kMaxElems / dim || shard_rows > kMaxElems / dim) return VPE_ERR_SHAPE;
  // the fp32 kernel's grid has one y-block per 64 rows of X, and a grid's y
  // extent must stay below 65536 (bf16 tile counts are checked at launch)
  if (m > (int64_t(1) << 21)) return VPE_ERR_SHAPE;
  // a tile's rows are addressed with 32-bit byte offsets
  if (dim > (int64_t(1) << 20)) return VPE_ERR_SHAPE;
  if (col_offset < 0 || ld_out < 1 || shard_rows > ld_out - col_offset) return VPE_ERR_RANGE;
  if (m > kMaxElems / ld_out) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!x || !weight || !logits) return VPE_ERR_NULL;
  if (!aligned(x, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      !aligned(logits, dtype_bytes(dt)))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_lmhead(x, m, dim, weight, shard_rows, dt == VPE_BF16 ? 1 : 0,
                                     logits, ld_out, col_offset, stream));
}

vpe_status vpe_lmhead_prefill(const void *hidden, int64_t n_tokens, int64_t dim,
                              const int32_t *cu_seqlens, int64_t n_seqs, const void *weight,
                              int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                              int64_t col_offset, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (n_tokens < 0 || n_seqs < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (n_tokens > INT32_MAX || n_tokens > kMaxElems / dim || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (n_seqs > (int64_t(1) << 21) || dim > (int64_t(1) << 20)) return VPE_ERR_SHAPE;
  if (col_offset < 0 || ld_out < 1 || shard_rows > ld_out - col_offset) return VPE_ERR_RANGE;
  if (n_seqs > kMaxElems / ld_out) return VPE_ERR_SHAPE;
  if (n_seqs == 0) return VPE_OK;
  if (!hidden || !cu_seqlens || !weight || !logits) return VPE_ERR_NULL;
  if (!aligned(hidden, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      !aligned(logits, dtype_bytes(dt)) || !aligned(cu_seqlens, 4))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_lmhead(hidden, n_seqs, dim, weight, shard_rows,
                                     dt == VPE_BF16 ? 1 : 0, logits, ld_out, col_offset, stream,
                                     cu_seqlens, n_tokens));
}

vpe_status vpe_load_shard(const void *full, int64_t vocab, int64_t dim, vpe_dtype dt,
                          int32_t tp_size, int32_t tp_rank, void *shard, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (dim < 1 || vocab < 1 || vocab > kMaxElems / dim) return VPE_ERR_SHAPE;
  int64_t start = 0, end = 0;
  const vpe_status rs = vpe_shard_range(vocab, tp_size, tp_rank, &start, &end);
  if (rs != VPE_OK) return rs;
  if (!full || !shard) return VPE_ERR_NULL;
  const int64_t row_bytes = dim * dtype_bytes(dt);
  const char *src = static_cast<const char *>(full) + start * row_bytes;
  const int64_t n_bytes = (end - start) * row_bytes;
  if (!aligned(full, dtype_bytes(dt)) || !aligned(shard, dtype_bytes(dt))) return VPE_ERR_ALIGN;
  // the shard must not overlap the rows it is copied from
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(shard);
  const uintptr_t nb = static_cast<uintptr_t>(n_bytes);
  if (d0 < s0 + nb && s0 < d0 + nb) return VPE_ERR_RANGE;
  return launched(vpe::launch_copy_bytes(src, shard, n_bytes, stream));
}

vpe_status vpe_argmax_init(uint64_t *best, int64_t m, void *stream) {
  if (m < 0 || m > (int64_t(1) << 21)) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!best) return VPE_ERR_NULL;
  if (!aligned(best, 8)) return VPE_ERR_ALIGN;
  return launched(vpe::launch_argmax_init(best, m, stream));
}

vpe_status vpe_lmhead_argmax(const void *x, int64_t m, int64_t dim, const void *weight,
                             int64_t shard_rows, vpe_dtype dt, int64_t vocab_start,
                             uint64_t *best, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (m < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (m > (int64_t(1) << 21) || dim > (int64_t(1) << 20) || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  // ids travel in 32 bits inside the keys
  // (compared without forming vocab_start + shard_rows, which may overflow)
  if (vocab_start < 0 || vocab_start > (int64_t(1) << 32) - 1 - shard_rows) return VPE_ERR_RANGE;
  if (m == 0) return VPE_OK;
  if (!x || !weight || !best) return VPE_ERR_NULL;
  if (!aligned(x, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) || !aligned(best, 8))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_lmhead(x, m, dim, weight, shard_rows, dt == VPE_BF16 ? 1 : 0,
                                     nullptr, shard_rows, 0, stream, nullptr, 0, best,
                                     vocab_start));
}

vpe_status vpe_lmhead_prefill_argmax(const void *hidden, int64_t n_tokens, int64_t dim,
                                     const int32_t *cu_seqlens, int64_t n_seqs,
                                     const void *weight, int64_t shard_rows, vpe_dtype dt,
                                     int64_t vocab_start, uint64_t *best, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (n_tokens < 0 || n_seqs < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (n_tokens > INT32_MAX || n_tokens > kMaxElems / dim || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (n_seqs > (int64_t(1) << 21) || dim > (int64_t(1) << 20)) return VPE_ERR_SHAPE;
  // ids travel in 32 bits inside the keys (compared without forming the sum)
  if (vocab_start < 0 || vocab_start > (int64_t(1) << 32) - 1 - shard_rows) return VPE_ERR_RANGE;
  if (n_seqs == 0) return VPE_OK;
  if (!hidden || !cu_seqlens || !weight || !best) return VPE_ERR_NULL;
  if (!aligned(hidden, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      !aligned(cu_seqlens, 4) || !aligned(best, 8))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_lmhead(hidden, n_seqs, dim, weight, shard_rows,
                                     dt == VPE_BF16 ? 1 : 0, nullptr, shard_rows, 0, stream,
                                     cu_seqlens, n_tokens, best, vocab_start));
}

vpe_status vpe_argmax_decode(const uint64_t *best, int64_t m, float *max_logit, int64_t *token,
                             void *stream) {
  if (m < 0 || m > (int64_t(1) << 21)) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!best || (!max_logit && !token)) return VPE_ERR_NULL;
  if (!aligned(best, 8) || (max_logit && !aligned(max_logit, 4)) || (token && !aligned(token, 8)))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_argmax_decode(best, m, max_logit, token, stream));
}

vpe_status vpe_argmax_decode_clear(uint64_t *best, int64_t m, float *max_logit, int64_t *token,
                                   void *stream) {
  if (m < 0 || m > (int64_t(1) << 21)) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!best || (!max_logit && !token)) return VPE_ERR_NULL;
  if (!aligned(best, 8) || (max_logit && !aligned(max_logit, 4)) || (token && !aligned(token, 8)))
    return VPE_ERR_ALIGN;
  return launched(vpe::launch_argmax_decode_clear(best, m, max_logit, token, stream));
}

vpe_status vpe_lmhead_logsumexp_workspace(int64_t m, int64_t shard_rows, int64_t *bytes) {
  if (!bytes) return VPE_ERR_NULL;
  if (m < 0 || shard_rows < 1) return VPE_ERR_SHAPE;
  const int64_t pairs = lse_pairs_bound(m, shard_rows);
  if (pairs < 0) return VPE_ERR_SHAPE;
  *bytes = pairs * 8;
  return VPE_OK;
}

vpe_status vpe_lmhead_logsumexp(const void *x, int64_t m, int64_t dim, const void *weight,
                                int64_t shard_rows, vpe_dtype dt, void *logits, int64_t ld_out,
                                int64_t col_offset, float *shard_lse, void *workspace,
                                int64_t workspace_bytes, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (m < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (m > (int64_t(1) << 21) || dim > (int64_t(1) << 20) || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (logits != nullptr) {
    if (col_offset < 0 || ld_out < 1 || shard_rows > ld_out - col_offset) return VPE_ERR_RANGE;
    if (m > kMaxElems / ld_out) return VPE_ERR_SHAPE;
  }
  if (workspace_bytes < 0) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!x || !weight || !shard_lse || !workspace) return VPE_ERR_NULL;
  if (!aligned(x, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      (logits && !aligned(logits, dtype_bytes(dt))) || !aligned(shard_lse, 4) ||
      !aligned(workspace, 8))
    return VPE_ERR_ALIGN;
  const int64_t need = lse_pairs_bound(m, shard_rows);
  if (need < 0 || workspace_bytes / 8 < need) return VPE_ERR_WORKSPACE;
  return launched(vpe::launch_lmhead(x, m, dim, weight, shard_rows, dt == VPE_BF16 ? 1 : 0,
                                     logits, logits ? ld_out : shard_rows,
                                     logits ? col_offset : 0, stream, nullptr, 0, nullptr, 0,
                                     static_cast<float *>(workspace), workspace_bytes / 8,
                                     shard_lse));
}

vpe_status vpe_lmhead_prefill_logsumexp(const void *hidden, int64_t n_tokens, int64_t dim,
                                        const int32_t *cu_seqlens, int64_t n_seqs,
                                        const void *weight, int64_t shard_rows, vpe_dtype dt,
                                        void *logits, int64_t ld_out, int64_t col_offset,
                                        float *shard_lse, void *workspace,
                                        int64_t workspace_bytes, void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (n_tokens < 0 || n_seqs < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (n_tokens > INT32_MAX || n_tokens > kMaxElems / dim || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (n_seqs > (int64_t(1) << 21) || dim > (int64_t(1) << 20)) return VPE_ERR_SHAPE;
  if (logits != nullptr) {
    if (col_offset < 0 || ld_out < 1 || shard_rows > ld_out - col_offset) return VPE_ERR_RANGE;
    if (n_seqs > kMaxElems / ld_out) return VPE_ERR_SHAPE;
  }
  if (workspace_bytes < 0) return VPE_ERR_SHAPE;
  if (n_seqs == 0) return VPE_OK;
  if (!hidden || !cu_seqlens || !weight || !shard_lse || !workspace) return VPE_ERR_NULL;
  if (!aligned(hidden, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      (logits && !aligned(logits, dtype_bytes(dt))) || !aligned(cu_seqlens, 4) ||
      !aligned(shard_lse, 4) || !aligned(workspace, 8))
    return VPE_ERR_ALIGN;
  const int64_t need = lse_pairs_bound(n_seqs, shard_rows);
  if (need < 0 || workspace_bytes / 8 < need) return VPE_ERR_WORKSPACE;
  return launched(vpe::launch_lmhead(hidden, n_seqs, dim, weight, shard_rows,
                                     dt == VPE_BF16 ? 1 : 0, logits,
                                     logits ? ld_out : shard_rows, logits ? col_offset : 0,
                                     stream, cu_seqlens, n_tokens, nullptr, 0,
                                     static_cast<float *>(workspace), workspace_bytes / 8,
                                     shard_lse));
}

vpe_status vpe_lmhead_logsumexp_noalloc(const void *x, int64_t m, int64_t dim, const void *weight,
                                        int64_t shard_rows, vpe_dtype dt, void *logits,
                                        int64_t ld_out, int64_t col_offset, float *shard_lse,
                                        void *stream) {
  if (!known_dtype(dt)) return VPE_ERR_DTYPE;
  if (m < 0 || dim < 1 || shard_rows < 1) return VPE_ERR_SHAPE;
  if (m > (int64_t(1) << 21) || dim > (int64_t(1) << 20) || shard_rows > kMaxElems / dim)
    return VPE_ERR_SHAPE;
  if (logits != nullptr) {
    if (col_offset < 0 || ld_out < 1 || shard_rows > ld_out - col_offset) return VPE_ERR_RANGE;
    if (m > kMaxElems / ld_out) return VPE_ERR_SHAPE;
  }
  if (m == 0) return VPE_OK;
  if (!x || !weight || !shard_lse) return VPE_ERR_NULL;
  if (!aligned(x, dtype_bytes(dt)) || !aligned(weight, dtype_bytes(dt)) ||
      (logits && !aligned(logits, dtype_bytes(dt))) || !aligned(shard_lse, 4))
    return VPE_ERR_ALIGN;
  // the exact pair count depends on the tile width the launcher picks; it
  // refuses (kErrWorkspace) before launching anything when the array is short
  return launched(vpe::launch_lmhead_logsumexp_noalloc(
      x, m, dim, weight, shard_rows, dt == VPE_BF16 ? 1 : 0, logits, logits ? ld_out : shard_rows,
      logits ? col_offset : 0, shard_lse, stream));
}

vpe_status vpe_logsumexp_combine(const float *const *shard_lse, int32_t n_parts, int64_t m,
                                 float *lse, void *stream) {
  if (n_parts < 1 || n_parts > VPE_MAX_PARTS || m < 0 || m > kMaxElems) return VPE_ERR_SHAPE;
  if (m == 0) return VPE_OK;
  if (!shard_lse || !lse) return VPE_ERR_NULL;
  for (int32_t r = 0; r < n_parts; ++r) {
    if (!shard_lse[r]) return VPE_ERR_NULL;
    if (!aligned(shard_lse[r], 4)) return VPE_ERR_ALIGN;
  }
  if (!aligned(lse, 4)) return VPE_ERR_ALIGN;
  return launched(vpe::launch_logsumexp_combine(shard_lse, n_parts, m, lse, stream));
}

const char *vpe_status_string(vpe_status s) {
  switch (s) {
    case VPE_OK: return "VPE_OK";
    case VPE_ERR_NULL: return "VPE_ERR_NULL";
    case VPE_ERR_SHAPE: return "VPE_ERR_SHAPE";
    case VPE_ERR_DTYPE: return "VPE_ERR_DTYPE";
    case VPE_ERR_ALIGN: return "VPE_ERR_ALIGN";
    case VPE_ERR_SHARD: return "VPE_ERR_SHARD";
    case VPE_ERR_LAUNCH: return "VPE_ERR_LAUNCH";
    case VPE_ERR_RANGE: return "VPE_ERR_RANGE";
    case VPE_ERR_WORKSPACE: return "VPE_ERR_WORKSPACE";
  }
  return "VPE_ERR_UNKNOWN";
}

}  // extern "C"
