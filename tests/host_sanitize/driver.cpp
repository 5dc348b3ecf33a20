// Host-side driver for the sanitized build (AddressSanitizer + UBSan, host
// code only): every C-ABI entry point's validation, with edge and overflow-
// prone arguments, against stand-in launchers that record what they receive;
// and the CPU oracle's loops on small heap buffers, where any out-of-bounds
// access is reported.  Exits non-zero on the first failed expectation.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/vpe.h"
#include "stub_record.h"
#include "../../vocab_sharded_embedding_amd/csrc/vpe_bounds.h"

extern "C" {
int orc_shard_range(int64_t, int32_t, int32_t, int64_t *, int64_t *);
int orc_mask_shift(const void *, int, int64_t, int64_t, int64_t, uint8_t *, int64_t *);
int orc_embed(const void *, int, int64_t, const void *, int, int64_t, int64_t, int64_t, void *,
              int);
int orc_sum_partials(const void *const *, int32_t, int64_t, int, void *);
int orc_last_token_select(const void *, int64_t, int64_t, int, const int32_t *, int64_t, void *);
int orc_lmhead_f64(const void *, int64_t, int64_t, const void *, int64_t, int, double *, int64_t,
                   int64_t, int);
int orc_argmax_rows(const double *, int64_t, int64_t, int64_t, double *, int64_t *);
int orc_load_shard(const void *, int64_t, int64_t, int, int32_t, int32_t, void *);
}

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static void *fake(uintptr_t off = 0) { return reinterpret_cast<void *>(0x100000 + off); }

static void check_abi() {
  const int64_t kMax = INT64_MAX, kMin = INT64_MIN;
  int64_t s = -1, e = -1;
  EXPECT(vpe_shard_range(151936, 2, 1, &s, &e) == VPE_OK && s == 75968 && e == 151936);
  EXPECT(vpe_shard_range(kMax, 1, 0, &s, &e) == VPE_OK && s == 0 && e == kMax);
  EXPECT(vpe_shard_range(kMin, 2, 0, &s, &e) == VPE_ERR_SHARD);
  EXPECT(vpe_shard_range(10, INT32_MAX, 0, &s, &e) == VPE_ERR_SHARD);
  EXPECT(vpe_shard_range(10, 2, INT32_MIN, &s, &e) == VPE_ERR_SHARD);
  EXPECT(vpe_shard_range(10, 2, 0, nullptr, &e) == VPE_ERR_NULL);

  // embed: the launcher gets the row size in bytes and the id width code
  g_last = stub_call{};
  EXPECT(vpe_embed(fake(), VPE_I64, 7, fake(4096), VPE_BF16, 100, 3, 50, fake(8192), nullptr) ==
         VPE_OK);
  EXPECT(!strcmp(g_last.what, "embed") && g_last.n0 == 7 && g_last.n1 == 100 && g_last.n2 == 6 &&
         g_last.n3 == 50 && g_last.i0 == 1);
  EXPECT(vpe_embed(fake(), VPE_I32, kMax, fake(), VPE_F32, 1, 1, 0, fake(), nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_embed(fake(), VPE_I32, 1, fake(), VPE_F32, kMax, kMax, 0, fake(), nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_embed(fake(), VPE_I32, kMin, fake(), VPE_F32, 1, 1, 0, fake(), nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_embed(fake(), (vpe_itype)7, 1, fake(), VPE_F32, 1, 1, 0, fake(), nullptr) ==
         VPE_ERR_DTYPE);
  EXPECT(vpe_embed(fake(2), VPE_I32, 1, fake(), VPE_F32, 1, 1, 0, fake(), nullptr) ==
         VPE_ERR_ALIGN);
  EXPECT(vpe_embed(fake(), VPE_I64, 1, fake(), VPE_F32, 1, 1, -1, fake(), nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_embed(fake(), VPE_I64, 1, fake(), VPE_F32, 1, 1, kMin, fake(), nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_embed(fake(), VPE_I64, 1, fake(), VPE_F32, 100, 1, kMax - 100, fake(), nullptr) ==
         VPE_OK);
  EXPECT(vpe_embed(fake(), VPE_I64, 1, fake(), VPE_F32, 100, 1, kMax - 99, fake(), nullptr) ==
         VPE_ERR_RANGE);

  // sum: 64 partials accepted, 65 rejected, a null entry rejected
  std::vector<const void *> parts(65, fake());
  EXPECT(vpe_sum_partials(parts.data(), 64, 10, VPE_BF16, fake(), nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "sum") && g_last.n1 == 64 && g_last.i0 == 1);
  EXPECT(vpe_sum_partials(parts.data(), 65, 10, VPE_BF16, fake(), nullptr) == VPE_ERR_SHAPE);
  parts[3] = nullptr;
  EXPECT(vpe_sum_partials(parts.data(), 8, 10, VPE_BF16, fake(), nullptr) == VPE_ERR_NULL);
  EXPECT(vpe_sum_partials(parts.data(), 0, 10, VPE_BF16, fake(), nullptr) == VPE_ERR_SHAPE);

  // select
  EXPECT(vpe_last_token_select(fake(), (int64_t)INT32_MAX + 1, 4, VPE_F32, (const int32_t *)fake(),
                               1, fake(), nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_last_token_select(fake(), 10, 4, VPE_F32, (const int32_t *)fake(2), 1, fake(),
                               nullptr) == VPE_ERR_ALIGN);
  EXPECT(vpe_last_token_select(fake(), 10, 4, VPE_F32, (const int32_t *)fake(), 3, fake(),
                               nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "select") && g_last.n0 == 10 && g_last.n1 == 3 && g_last.n2 == 16);

  // LM head: column window and overflow-prone ranges
  EXPECT(vpe_lmhead(fake(), 4, 64, fake(), 100, VPE_BF16, fake(), 150, 50, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead") && g_last.n0 == 4 && g_last.n1 == 100 &&
         g_last.n2 == 64 && g_last.n3 == 50 && g_last.n4 == 150);
  EXPECT(vpe_lmhead(fake(), 4, 64, fake(), 100, VPE_BF16, fake(), 150, 51, nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_lmhead(fake(), 4, 64, fake(), 100, VPE_BF16, fake(), kMax, kMax, nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_lmhead(fake(), 4, 64, fake(), 100, VPE_BF16, fake(), kMin, 0, nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_lmhead(fake(), 4, 64, fake(), 100, VPE_BF16, fake(), 150, kMin, nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_lmhead(fake(), 1 << 21, 64, fake(), 100, VPE_BF16, fake(), kMax / 2, 0, nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_prefill(fake(), 100, 64, (const int32_t *)fake(), 9, fake(), 100, VPE_BF16,
                            fake(), 100, 0, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_prefill") && g_last.n0 == 9 && g_last.n4 == 100);

  // greedy pick: the id range must fit the keys' 32-bit id field
  EXPECT(vpe_lmhead_argmax(fake(), 4, 64, fake(), 100, VPE_BF16, 7, (uint64_t *)fake(), nullptr) ==
         VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_argmax") && g_last.n3 == 7);
  EXPECT(vpe_lmhead_argmax(fake(), 4, 64, fake(), 100, VPE_BF16, kMax, (uint64_t *)fake(),
                           nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_argmax(fake(), 4, 64, fake(), 100, VPE_BF16, kMin, (uint64_t *)fake(),
                           nullptr) == VPE_ERR_RANGE);
  // ids up to 2^32 - 2 fit (vocab_start + shard_rows <= 2^32 - 1)
  EXPECT(vpe_lmhead_argmax(fake(), 4, 64, fake(), 100, VPE_BF16, 4294967295LL - 99,
                           (uint64_t *)fake(), nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_argmax(fake(), 4, 64, fake(), 100, VPE_BF16, 4294967295LL - 100,
                           (uint64_t *)fake(), nullptr) == VPE_OK);
  // greedy pick over packed sequences: select and pick in one launch
  EXPECT(vpe_lmhead_prefill_argmax(fake(), 1000, 64, (const int32_t *)fake(), 9, fake(), 100,
                                   VPE_BF16, 7, (uint64_t *)fake(), nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_prefill_argmax") && g_last.n0 == 9 && g_last.n3 == 7 &&
         g_last.n4 == 1000);
  EXPECT(vpe_lmhead_prefill_argmax(fake(), kMax, 64, (const int32_t *)fake(), 9, fake(), 100,
                                   VPE_BF16, 7, (uint64_t *)fake(), nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_prefill_argmax(fake(), 1000, 64, (const int32_t *)fake(), 9, fake(), kMax,
                                   VPE_BF16, 7, (uint64_t *)fake(), nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_prefill_argmax(fake(), 1000, 64, (const int32_t *)fake(), 9, fake(), 100,
                                   VPE_BF16, kMin, (uint64_t *)fake(), nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_prefill_argmax(fake(), 1000, 64, (const int32_t *)fake(), 9, fake(), 100,
                                   VPE_BF16, 4294967295LL - 99, (uint64_t *)fake(),
                                   nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_argmax_init((uint64_t *)fake(), kMax, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_argmax_decode((const uint64_t *)fake(), 5, (float *)fake(), nullptr, nullptr) ==
         VPE_OK);
  EXPECT(vpe_argmax_decode_clear((uint64_t *)fake(), 5, nullptr, (int64_t *)fake(), nullptr) ==
         VPE_OK);
  EXPECT(!strcmp(g_last.what, "argmax_decode_clear") && g_last.n0 == 5);
  EXPECT(vpe_argmax_decode_clear((uint64_t *)fake(), 5, nullptr, nullptr, nullptr) ==
         VPE_ERR_NULL);

  // shard loading: the launcher copies the rank's contiguous rows
  EXPECT(vpe_load_shard(fake(), 100, 8, VPE_BF16, 4, 3, fake(1 << 20), nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "copy") && g_last.a == fake(75 * 16) && g_last.n0 == 25 * 16);
  EXPECT(vpe_load_shard(fake(), kMax, kMax, VPE_BF16, 1, 0, fake(1 << 20), nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_load_shard(fake(), 100, 8, VPE_BF16, 4, 3, fake(75 * 16 + 8), nullptr) ==
         VPE_ERR_RANGE);

  for (int c = -1; c <= 9; ++c) EXPECT(vpe_status_string((vpe_status)c) != nullptr);
}

static void check_oracle() {
  // a [6, 3] fp32 table, tp 2
  const int64_t V = 6, D = 3;
  std::vector<float> table(V * D);
  for (int64_t i = 0; i < V * D; ++i) table[i] = (float)i;
  int64_t s = 0, e = 0;
  EXPECT(orc_shard_range(V, 2, 1, &s, &e) == 0 && s == 3 && e == 6);
  std::vector<int64_t> ids = {-7, 0, 3, 5, 6, 1 << 30};
  std::vector<uint8_t> mask(ids.size());
  std::vector<int64_t> local(ids.size());
  EXPECT(orc_mask_shift(ids.data(), 1, (int64_t)ids.size(), s, e, mask.data(), local.data()) == 0);
  std::vector<float> part(ids.size() * D);
  EXPECT(orc_embed(ids.data(), 1, (int64_t)ids.size(), table.data() + s * D, 0, e - s, D, s,
                   part.data(), 3) == 0);
  EXPECT(part[2 * D] == table[3 * D] && part[0] == 0.0f);
  std::vector<float> other(ids.size() * D, 0.0f), sum(ids.size() * D);
  const void *pp[2] = {part.data(), other.data()};
  EXPECT(orc_sum_partials(pp, 2, (int64_t)sum.size(), 0, sum.data()) == 0);
  std::vector<int32_t> cu = {0, 2, 6};
  std::vector<float> sel(2 * D);
  EXPECT(orc_last_token_select(table.data(), V, D, 0, cu.data(), 2, sel.data()) == 0);
  std::vector<int32_t> bad = {0, 4, 2};
  EXPECT(orc_last_token_select(table.data(), V, D, 0, bad.data(), 2, sel.data()) != 0);
  std::vector<double> logits(2 * (V + 1), -1.0);
  EXPECT(orc_lmhead_f64(sel.data(), 2, D, table.data(), V, 0, logits.data(), V + 1, 1, 4) == 0);
  std::vector<double> mx(2);
  std::vector<int64_t> at(2);
  EXPECT(orc_argmax_rows(logits.data(), 2, V + 1, V + 1, mx.data(), at.data()) == 0);
  EXPECT(at[0] == 6 && at[1] == 6);  // the last table row has the largest entries
  std::vector<float> shard((V / 2) * D);
  EXPECT(orc_load_shard(table.data(), V, D, 0, 2, 1, shard.data()) == 0);
  EXPECT(shard[0] == table[3 * D]);
  EXPECT(orc_load_shard(table.data(), V, D, 0, 4, 0, shard.data()) != 0);
}

// The LM-head launchers' choice between buffer loads (masked loads at byte
// offset kLoadMask must read zeros, so a descriptor may cover at most
// kLoadMask bytes) and element-wise register staging, at the edges of the
// window (kLoadMask, 2^31) of gathered prefill activations.
static void check_load_paths() {
  using vpe::bf16_direct_loads_ok;
  using vpe::bf16_rows_fit_descriptor;
  using vpe::kLoadMask;
  EXPECT(kLoadMask == 0x7FFF0000);
  // K = 1024: 2048-byte rows; kLoadMask / 2048 = 1048544 rows exactly
  EXPECT(bf16_rows_fit_descriptor(1048544, 1024));
  EXPECT(!bf16_rows_fit_descriptor(1048545, 1024));
  EXPECT(!bf16_rows_fit_descriptor(1048575, 1024));  // 2^31 - 2048 bytes: inside the window
  EXPECT(!bf16_rows_fit_descriptor(1048576, 1024));  // 2^31 bytes
  EXPECT(bf16_rows_fit_descriptor(0, 1024) && bf16_rows_fit_descriptor(5, 0));
  EXPECT(!bf16_rows_fit_descriptor(-1, 8));
  EXPECT(!bf16_rows_fit_descriptor(INT64_MAX, 8) && !bf16_rows_fit_descriptor(2, INT64_MAX / 2));
  EXPECT(!bf16_rows_fit_descriptor(1, INT64_MAX) && bf16_rows_fit_descriptor(1, kLoadMask / 2));
  // K = 4096 (8 KB rows): kLoadMask / 8192 = 262136 rows
  EXPECT(bf16_rows_fit_descriptor(262136, 4096) && !bf16_rows_fit_descriptor(262137, 4096));
  // gathered X: the whole token range counts, not the tile
  EXPECT(bf16_direct_loads_ok(0x1000, 0x2000, 1024, true, 1048544, 32, 192));
  EXPECT(!bf16_direct_loads_ok(0x1000, 0x2000, 1024, true, 1048545, 32, 192));
  EXPECT(!bf16_direct_loads_ok(0x1000, 0x2000, 1024, true, 1048560, 32, 192));
  // contiguous X: only the tile's rows count
  EXPECT(bf16_direct_loads_ok(0x1000, 0x2000, 1024, false, 1048560, 256, 320));
  EXPECT(bf16_direct_loads_ok(0x1000, 0x2000, 1 << 20, false, 0, 256, 320));
  // alignment and K
  EXPECT(!bf16_direct_loads_ok(0x1008, 0x2000, 1024, false, 0, 256, 320));
  EXPECT(!bf16_direct_loads_ok(0x1000, 0x2002, 1024, false, 0, 256, 320));
  EXPECT(!bf16_direct_loads_ok(0x1000, 0x2000, 1020, false, 0, 256, 320));
}

// The log-sum-exp entry points: the workspace bound (8 bytes per row per 64
// shard rows, overflow refused), validation before any launch, and what the
// launcher is asked for.
static void check_logsumexp() {
  const int64_t kMax = INT64_MAX;
  int64_t bytes = -1;
  EXPECT(vpe_lmhead_logsumexp_workspace(256, 75968, &bytes) == VPE_OK && bytes == 256 * 1187 * 8);
  EXPECT(vpe_lmhead_logsumexp_workspace(1, 64, &bytes) == VPE_OK && bytes == 8);
  EXPECT(vpe_lmhead_logsumexp_workspace(1, 65, &bytes) == VPE_OK && bytes == 16);
  EXPECT(vpe_lmhead_logsumexp_workspace(0, 65, &bytes) == VPE_OK && bytes == 0);
  EXPECT(vpe_lmhead_logsumexp_workspace(1 << 21, kMax, &bytes) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp_workspace(kMax, kMax, &bytes) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp_workspace(-1, 8, &bytes) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp_workspace(4, 0, &bytes) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp_workspace(4, 8, nullptr) == VPE_ERR_NULL);

  float *lse = static_cast<float *>(fake(0x1000));
  void *ws = fake(0x2000);
  const int64_t need = 256 * 1187 * 8;
  g_last = stub_call{};
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, ws, need, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_logsumexp") && g_last.lse == ws &&
         g_last.lse_cap == need / 8 && g_last.shard_lse == lse && g_last.n0 == 256 &&
         g_last.n1 == 75968 && g_last.n2 == 1024 && g_last.out == fake(32));
  // no logits: nothing is stored, the stride and offset are ignored
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, nullptr, -5, kMax, lse,
                              ws, need, nullptr) == VPE_OK);
  EXPECT(g_last.out == nullptr && g_last.n3 == 0);
  g_last = stub_call{};
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, ws, need - 1, nullptr) == VPE_ERR_WORKSPACE);
  EXPECT(g_last.what == nullptr);  // nothing launched
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, ws, -8, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, nullptr, need, nullptr) == VPE_ERR_NULL);
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              nullptr, ws, need, nullptr) == VPE_ERR_NULL);
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, fake(0x2004), need, nullptr) == VPE_ERR_ALIGN);
  EXPECT(vpe_lmhead_logsumexp(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 1,
                              lse, ws, need, nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_logsumexp(fake(), kMax, 1024, fake(16), 75968, VPE_BF16, fake(32), 75968, 0,
                              lse, ws, kMax, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp(fake(), 4, 8, fake(16), kMax, VPE_F32, nullptr, 0, 0, lse, ws, kMax,
                              nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp(fake(), 0, 8, fake(16), 8, VPE_F32, nullptr, 0, 0, nullptr, nullptr,
                              0, nullptr) == VPE_OK);
  EXPECT(vpe_lmhead_logsumexp(fake(), 4, 8, fake(16), 8, (vpe_dtype)7, nullptr, 0, 0, lse, ws,
                              64, nullptr) == VPE_ERR_DTYPE);

  // prefill: the last-position select folded in, the same workspace rule
  const int32_t *cu = static_cast<const int32_t *>(fake(0x3000));
  const int64_t need_p = 32 * 2374 * 8;  // 32 sequences over 151936 shard rows
  g_last = stub_call{};
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, cu, 32, fake(16), 151936, VPE_BF16,
                                      fake(32), 151936, 0, lse, ws, need_p, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_prefill_logsumexp") && g_last.n0 == 32 &&
         g_last.n1 == 151936 && g_last.n2 == 1024 && g_last.n4 == 65536 && g_last.lse == ws &&
         g_last.lse_cap == need_p / 8 && g_last.shard_lse == lse && g_last.out == fake(32));
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, cu, 32, fake(16), 151936, VPE_BF16,
                                      nullptr, -1, kMax, lse, ws, need_p, nullptr) == VPE_OK);
  EXPECT(g_last.out == nullptr && g_last.n3 == 0);
  g_last = stub_call{};
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, cu, 32, fake(16), 151936, VPE_BF16,
                                      fake(32), 151936, 0, lse, ws, need_p - 1, nullptr) ==
         VPE_ERR_WORKSPACE);
  EXPECT(g_last.what == nullptr);
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, nullptr, 32, fake(16), 151936, VPE_BF16,
                                      fake(32), 151936, 0, lse, ws, need_p, nullptr) ==
         VPE_ERR_NULL);
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, static_cast<const int32_t *>(fake(0x3002)),
                                      32, fake(16), 151936, VPE_BF16, fake(32), 151936, 0, lse, ws,
                                      need_p, nullptr) == VPE_ERR_ALIGN);
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), int64_t(INT32_MAX) + 1, 8, cu, 32, fake(16), 64,
                                      VPE_BF16, nullptr, 0, 0, lse, ws, kMax, nullptr) ==
         VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), 65536, 1024, cu, 32, fake(16), 151936, VPE_BF16,
                                      fake(32), 151936, 1, lse, ws, need_p, nullptr) ==
         VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_prefill_logsumexp(fake(), kMax, 1024, cu, kMax, fake(16), 151936, VPE_BF16,
                                      nullptr, 0, 0, lse, ws, kMax, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_prefill_logsumexp(nullptr, 0, 8, nullptr, 0, nullptr, 8, VPE_F32, nullptr, 0, 0,
                                      nullptr, nullptr, 0, nullptr) == VPE_OK);

  const float *parts[65];
  for (int r = 0; r < 65; ++r) parts[r] = static_cast<const float *>(fake(0x4000 + 4096 * r));
  g_last = stub_call{};
  EXPECT(vpe_logsumexp_combine(parts, 3, 100, lse, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "logsumexp_combine") && g_last.a == parts[0] &&
         g_last.b == parts[2] && g_last.n0 == 100 && g_last.n1 == 3);
  EXPECT(vpe_logsumexp_combine(parts, 64, 100, lse, nullptr) == VPE_OK);
  EXPECT(vpe_logsumexp_combine(parts, 65, 100, lse, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_logsumexp_combine(parts, 0, 100, lse, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_logsumexp_combine(parts, 2, -1, lse, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_logsumexp_combine(parts, 2, 0, nullptr, nullptr) == VPE_OK);
  EXPECT(vpe_logsumexp_combine(nullptr, 2, 4, lse, nullptr) == VPE_ERR_NULL);
  const float *with_null[2] = {parts[0], nullptr};
  EXPECT(vpe_logsumexp_combine(with_null, 2, 4, lse, nullptr) == VPE_ERR_NULL);
  const float *odd[2] = {parts[0], static_cast<const float *>(fake(0x4002))};
  EXPECT(vpe_logsumexp_combine(odd, 2, 4, lse, nullptr) == VPE_ERR_ALIGN);
  EXPECT(!strcmp(vpe_status_string(VPE_ERR_WORKSPACE), "VPE_ERR_WORKSPACE"));

  // the allocation-free variant: same validation, no workspace arguments
  g_last = stub_call{};
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32),
                                      75968, 0, lse, nullptr) == VPE_OK);
  EXPECT(!strcmp(g_last.what, "lmhead_logsumexp_noalloc") && g_last.shard_lse == lse &&
         g_last.n0 == 256 && g_last.n1 == 75968 && g_last.n2 == 1024 && g_last.out == fake(32));
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), 256, 1024, fake(16), 75968, VPE_BF16, nullptr, -1,
                                      kMax, lse, nullptr) == VPE_OK);
  EXPECT(g_last.out == nullptr && g_last.n3 == 0);
  g_last = stub_call{};
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32),
                                      75968, 1, lse, nullptr) == VPE_ERR_RANGE);
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), 256, 1024, fake(16), 75968, VPE_BF16, fake(32),
                                      75968, 0, nullptr, nullptr) == VPE_ERR_NULL);
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), kMax, 1024, fake(16), 75968, VPE_BF16, nullptr, 0,
                                      0, lse, nullptr) == VPE_ERR_SHAPE);
  EXPECT(vpe_lmhead_logsumexp_noalloc(fake(), 4, 8, fake(16), 8, VPE_BF16, nullptr, 0, 0,
                                      static_cast<float *>(fake(0x1002)), nullptr) ==
         VPE_ERR_ALIGN);
  EXPECT(g_last.what == nullptr);  // nothing launched by the rejected calls
}

int main() {
  check_load_paths();
  check_logsumexp();
  check_abi();
  check_oracle();
  if (!g_fail) printf("host sanitizer driver: all expectations held\n");
  return g_fail;
}
