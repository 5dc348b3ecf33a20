// LM-head kernels for gfx950: one shard's logits Z = X . W^T, written at a
// column offset of a row-major logits buffer.
//
// Sources: devpress.csdn.net/amd/6a3de260... section 4 (ParallelLMHead: the
// shard's F.linear over its [V/tp, D] rows) and section 6 (shard logits
// concatenated along the vocabulary); caomaolufei.github.io AIInfraGuide 3.3
// section 6 (ParallelLMHead.forward).
//
// Both operands are K-contiguous: X is [M, K] (hidden states), W is [N, K]
// (vocabulary rows, the same layout the embedding reads).  That is the layout
// the MFMA operand fragments want, so no transpose is ever made.
//
// bf16: two matrix-core kernels built on v_mfma_f32_16x16x32_bf16.  W is the
// MFMA "A" operand (16 vocabulary rows per fragment) and X the "B" operand, so
// each lane owns 4 consecutive vocabulary columns of one logits row.
//  - lmhead_bf16_mfma: a workgroup (256 or 512 threads) owns a BN x BM tile
//    of Z^T (BN vocabulary rows by BM hidden rows).  W and X slices of BK
//    columns of K are staged through a multi-stage LDS ring, filled by
//    direct buffer-to-LDS loads (or through registers when the operands are
//    not 16-byte aligned).  Used for every M up to 256, and above that when
//    the next kernel does not apply.
//  - lmhead_bf16_xreg: for M > 256.  The workgroup's X rows stay in
//    registers for the whole K loop and only W streams through LDS, so the
//    LDS read traffic per MFMA is halved.
// Epilogues: a full tile is staged through LDS and written as 16-byte rows
// of logits; a partial tile pairs two lanes' 8-byte fragments into 16-byte
// stores where the alignment allows, else writes 8-byte or single elements.
// The greedy-pick variant stores no logits and folds each row's best
// candidate into a 64-bit key instead.
// fp32: a plain LDS-tiled FMA kernel (fp32 shards are small test shapes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "vpe_bounds.h"
#include "vpe_launch.h"

namespace vpe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
// dword 3 of a gfx9 buffer descriptor: 32-bit data format, raw (unswizzled) access
constexpr int kBufferFlags = 0x00020000;

// binary32 -> bf16 bits, round to nearest, ties to even; NaN becomes a quiet NaN
[[maybe_unused]] __device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rounded;
}

// ---------------------------------------------------------------------------
// Greedy-pick keys.  A logit v of vocabulary id t becomes the 64-bit key
//   (order(v) << 32) | (0xFFFFFFFF - t)
// where order() maps binary32 bits to an unsigned integer with the same
// order as the values.  The largest key is the largest logit, and among
// equal logits the smallest id (the first maximum, as an argmax over the
// concatenated row picks).  Shards fold their candidates into one key per row
// with an atomic max, so the combine across shards needs no extra step.
// ---------------------------------------------------------------------------
struct TileOut {
  uint64_t *best;   // [M] keys, or nullptr: write logits instead
  int64_t id_base;  // vocabulary id of the shard's first row (vocab_start)
  // Log-sum-exp partials, or nullptr: entry [row * lse_ld + tile] holds the
  // pair (tile maximum, sum of exp(logit - maximum)) of that row over the
  // columns of W tile `tile` (lse_ld = the number of W tiles, set by the
  // launcher that picks the tile width)
  float *lse;
  int64_t lse_ld;
  int64_t lse_cap;  // entries the partials buffer holds (checked by the launchers)
};

// ---------------------------------------------------------------------------
// Log-sum-exp partials.  A row's log-sum-exp over a set of logits is kept as
// the pair (m, s) = (largest logit, sum of exp(logit - m)); two disjoint sets
// merge into (max(m1, m2), s1 exp(m1 - m) + s2 exp(m2 - m)).  An empty set is
// (-inf, 0).  The logits are the stored values (fp32 accumulation rounded to
// the logits dtype), so the value is the log-sum-exp of the logits a caller
// reads back.  Merges happen in a fixed order, so results are reproducible.
// ---------------------------------------------------------------------------
// Maximum that keeps a NaN (fmaxf drops it): a row with a NaN logit must not
// lose it before the sum.
__device__ __forceinline__ float nan_max(float a, float b) { return (a != a || a > b) ? a : b; }

__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mx = nan_max(m, m2);
  // (-inf) - (-inf) would be NaN: an empty side contributes nothing
  const float a = (m == -__builtin_huge_valf()) ? 0.f : s * __expf(m - mx);
  const float b = (m2 == -__builtin_huge_valf()) ? 0.f : s2 * __expf(m2 - mx);
  m = mx;
  s = a + b;
}

// Two logits' stored values: each rounded to bf16 (nearest, ties to even, one
// v_cvt_pk_bf16_f32 for the pair) and widened back.
__device__ __forceinline__ void bf16_values(float &a, float &b) {
  const __bf16 x = static_cast<__bf16>(a), y = static_cast<__bf16>(b);
  a = static_cast<float>(x);
  b = static_cast<float>(y);
}

// Per row of a wave's fragments (acc[i][j][r]: row mb + 16 j, column
// nb + 16 i + r, nb the lane's first column), the pair over the tile's
// columns below N, reduced over the 4 lanes that hold the same row.
//  - Rounding to nearest even is monotone, so the largest stored logit is the
//    rounding of the largest accumulator: the maximum needs no rounding per
//    element.
//  - Each term is 2^((v - m) log2 e) on the exponent unit (v_exp_f32), v the
//    stored logit.  A NaN logit, or an infinite one (inf - inf), makes the
//    sum NaN, and a NaN sum makes the pair (NaN, NaN): no per-element test.
//  - A tile wholly inside N (`full`) runs without per-column checks; otherwise
//    columns at or past N are left out by selects (no branches).
template <int FN, int FM, bool BF16>
__device__ __forceinline__ void lse_rows(const f32x4 (&acc)[FN][FM], int64_t nb, int64_t N,
                                         bool full, float (&mx)[FM], float (&sm)[FM]) {
  constexpr float kLog2e = 1.4426950408889634f;
  // this lane's columns nb + c, c = 16 i + r, lie below N for c < lim
  const int64_t left = N - nb;
  const int lim = left < 0 ? 0 : (left < FN * 16 ? static_cast<int>(left) : FN * 16);
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    float a = -__builtin_huge_valf();
    if (full) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) a = fmaxf(a, acc[i][j][r]);
    } else {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) a = (i * 16 + r < lim) ? fmaxf(a, acc[i][j][r]) : a;
    }
    // (a is -inf for a lane with no column below N, or whose logits are all
    // -inf or NaN: its terms are then 0, or NaN)
    const bool any = a != -__builtin_huge_valf();
    float m = a, b2 = a;
    if (BF16 && any) bf16_values(m, b2);
    const float mb = any ? -m * kLog2e : 0.f;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        float v0 = acc[i][j][r], v1 = acc[i][j][r + 1];
        if (BF16) bf16_values(v0, v1);
        const float e0 = __builtin_amdgcn_exp2f(fmaf(v0, kLog2e, mb));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(v1, kLog2e, mb));
        if (full) {
          s += e0;
          s += e1;
        } else {
          s += (i * 16 + r < lim) ? e0 : 0.f;
          s += (i * 16 + r + 1 < lim) ? e1 : 0.f;
        }
      }
    float m2 = (s != s) ? s : m;  // NaN when a logit was NaN or infinite
    lse_merge(m2, s, __shfl_xor(m2, 16), __shfl_xor(s, 16));
    lse_merge(m2, s, __shfl_xor(m2, 32), __shfl_xor(s, 32));
    mx[j] = m2;
    sm[j] = s;
  }
}

__device__ __forceinline__ uint64_t pick_key(float v, int64_t id) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(id));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Makes v's value needed at this point of the program, so the load that
// produces it is issued earlier and waited on here, not later.
[[maybe_unused]] __device__ __forceinline__ void pin_vgpr(int32_t &v) { asm volatile("" : "+v"(v)); }

// ---------------------------------------------------------------------------
// LDS tile layout: a row holds BK bf16 = P = BK/8 pieces of 16 bytes.  The LDS
// serves a 16-byte read in passes of 8 lanes over 32 four-byte banks (128
// bytes), and the 8 lanes of a pass read the same piece of 8 consecutive
// rows.  Piece p of row r is stored at slot p ^ f(r) with
//   f(r) = (r / G) mod P,   G = rows per 128 bytes (2 for BK = 32, else 1),
// so those 8 rows' pieces land in 8 distinct 16-byte bank groups.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int lds_swizzle(int row) {
  constexpr int P = BK / 8;
  constexpr int G = (BK * 2 >= 128) ? 1 : 128 / (BK * 2);
  return (row / G) & (P - 1);
}

template <int BK>
__device__ __forceinline__ int lds_piece_offset(int row, int piece) {
  return row * BK + ((piece ^ lds_swizzle<BK>(row)) << 3);  // in bf16 elements
}

// Workgroup tile order.  Work-groups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8), and each XCD has its own L2.  Block b is
// mapped to a logical tile index so that every XCD works through one
// contiguous run of logical tiles.  Logical tiles are ordered in groups of
// GN W tiles: inside a group, X row blocks are the outer index and the GN W
// tiles the inner one.  The ~32 tiles an XCD runs at once then cover GN W
// tiles times 32/GN X tiles, so both operands are shared in that XCD's L2
// (GN = 1: all X blocks of one W tile, the order for few X blocks).
[[maybe_unused]] __device__ __forceinline__ void tile_of_block(int b, int tiles_n, int tiles_m, int group_n,
                                              int &tn, int &tm) {
  const int total = tiles_n * tiles_m;
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  const int t = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int per_group = group_n * tiles_m;
  const int g = t / per_group;
  const int in_g = t - g * per_group;
  const int gn = min(group_n, tiles_n - g * group_n);  // the last group may be narrower
  tm = in_g / gn;
  tn = g * group_n + (in_g - tm * gn);
}

// Offset past any descriptor's range: buffer loads at it return zeros.  Every
// descriptor built here covers at most kBig bytes (the launchers check it
// with bf16_direct_loads_ok before they take the buffer-load paths).
constexpr int kBig = kLoadMask;

// Writes a wave's accumulators.  acc[i][j][r] = Z^T[n][m] for the vocabulary
// row n = nb + 16 i + r and hidden row m = mb + 16 j, where nb and mb are the
// lane's first column and row (nb is a multiple of 4 from a multiple-of-4
// tile origin).  `full`: the workgroup tile lies wholly inside [0, N) x [0, M).
// ARGMAX folds each row's largest logit (rounded to bf16) into pick.best.
template <int FN, int FM>
__device__ __forceinline__ void argmax_keys(const f32x4 (&acc)[FN][FM], int64_t nb, bool full,
                                            int64_t N, TileOut pick, uint64_t (&keys)[FM]) {
  {
    // The 4 lanes l, l^16, l^32, l^48 hold the same row m (16 columns each).
    // Wanted: the row's first largest logit as rounded to bf16, compared in
    // the key order (16-bit order codes, -0 below +0, NaN outside +-Inf).
    //
    // Rounding to nearest even is monotone, so the largest rounded logit is
    // the rounding `top` of the largest fp32 logit, and the logits that round
    // to `top` are exactly those at or above the smallest fp32 value that
    // rounds to it (a bound derived from `top`'s bits).  Fast path: one pass
    // for the fp32 maximum, one compare per logit for the first column at or
    // above the bound.  Rows with an infinite or NaN logit, or whose maximum
    // rounds to +-0 (where fp32 compares do not see the signs of zeros), and
    // tiles that reach past column N take the exact per-logit path instead.
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      float mx = acc[0][j][0], bad = 0.f;  // bad becomes NaN on an infinite or NaN logit
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mx = fmaxf(mx, acc[i][j][r]);
          bad = fmaf(acc[i][j][r], 0.f, bad);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      bad = bad + __shfl_xor(bad, 16);
      bad = bad + __shfl_xor(bad, 32);
      const uint32_t top = f32_to_bf16_bits(mx);
      uint64_t key = 0;
      if (full && bad == 0.f && (top & 0x7FFFu) != 0) {
        // smallest fp32 rounding to `top`: the midpoint to the next bf16 value
        // below it, or one ulp past that midpoint when the tie rounds away
        float lo;
        if ((top & 0x8000u) == 0) {
          lo = __uint_as_float((((top - 1u) << 16) | 0x8000u) + (top & 1u));
        } else {
          const uint32_t mag = top & 0x7FFFu;  // top = -mag; -Inf: every logit
          lo = mag >= 0x7F80u ? -__builtin_huge_valf()
                              : __uint_as_float(0x80000000u | (((mag << 16) | 0x8000u) - (mag & 1u)));
        }
        int c = -1;  // this lane's first column at or above lo (columns visited last to first)
#pragma unroll
        for (int i = FN - 1; i >= 0; --i)
#pragma unroll
          for (int r = 3; r >= 0; --r) c = acc[i][j][r] >= lo ? i * 16 + r : c;
        if (c >= 0) key = pick_key(__uint_as_float(top << 16), pick.id_base + nb + c);
      } else {
        // exact path: visit the columns in increasing order and keep the first
        // largest 16-bit order code of the rounded logit
        uint32_t best_ord = 0, best_h = 0;
        int best_c = -1;  // column offset of the pick inside this lane's columns
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t h = f32_to_bf16_bits(acc[i][j][r]);
            const uint32_t ord = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
            const bool take = nb + i * 16 + r < N && (best_c < 0 || ord > best_ord);
            best_ord = take ? ord : best_ord;
            best_h = take ? h : best_h;
            best_c = take ? i * 16 + r : best_c;
          }
        if (best_c >= 0) key = pick_key(__uint_as_float(best_h << 16), pick.id_base + nb + best_c);
      }
      key = umax64(key, __shfl_xor(key, 16));
      key = umax64(key, __shfl_xor(key, 32));
      keys[j] = key;
    }
  }
}

// Folds a row's key into pick.best[m] (lanes with (threadIdx.x & 48) == 0
// hold the keys of rows mb + 16 j).
template <int FM>
__device__ __forceinline__ void argmax_fold(const uint64_t (&keys)[FM], int64_t mb, int64_t M,
                                            TileOut pick) {
#pragma unroll
  for (int j = 0; j < FM; ++j)
    if ((threadIdx.x & 48) == 0 && mb + j * 16 < M)
      atomicMax(reinterpret_cast<unsigned long long *>(pick.best + mb + j * 16),
                static_cast<unsigned long long>(keys[j]));
}

template <int FN, int FM, bool ARGMAX>
__device__ __forceinline__ void write_tile(const f32x4 (&acc)[FN][FM], int64_t nb, int64_t mb,
                                           bool full, int64_t M, int64_t N,
                                           uint16_t *__restrict__ out, int64_t ld,
                                           int64_t col_off, TileOut pick) {
  if constexpr (ARGMAX) {
    uint64_t keys[FM];
    argmax_keys<FN, FM>(acc, nb, full, N, pick, keys);
    argmax_fold<FM>(keys, mb, M, pick);
    return;
  }
  // 8-byte stores need every row start at a multiple of 4 elements from an
  // 8-byte-aligned base (column offsets inside a tile are multiples of 4).
  const bool pack_ok =
      ((ld | col_off) & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
  if constexpr (FN % 2 == 0) {
    // 16-byte stores: lanes l and l ^ 16 (k groups g, g ^ 1, same row) trade
    // halves of fragments i and i + 1 so that each holds 8 consecutive
    // columns: even g keeps columns 16i + 4g .. +3 of fragment i and takes
    // the partner's next 4; odd g keeps 16(i+1) + 4g .. +3 of fragment i + 1
    // and takes the partner's previous 4.  A store then writes 64 bytes of a
    // row per 4 lanes instead of 32 (measured on MI355X: the M = 256 LM head
    // 53.6 -> 50.2 us, the M = 1024 one 212 -> 196 us).
    const bool wide_ok =
        ((ld | col_off) & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    if (wide_ok && full) {
      const bool even = ((threadIdx.x >> 4) & 1) == 0;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        uint16_t *row = out + (mb + j * 16) * ld + col_off + nb;
#pragma unroll
        for (int i = 0; i < FN; i += 2) {
          const uint32_t a0 = f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16);
          const uint32_t a1 = f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16);
          const uint32_t b0 =
              f32_to_bf16_bits(acc[i + 1][j][0]) | (f32_to_bf16_bits(acc[i + 1][j][1]) << 16);
          const uint32_t b1 =
              f32_to_bf16_bits(acc[i + 1][j][2]) | (f32_to_bf16_bits(acc[i + 1][j][3]) << 16);
          const uint32_t r0 = __shfl_xor(even ? b0 : a0, 16);
          const uint32_t r1 = __shfl_xor(even ? b1 : a1, 16);
          const u32x4 v = even ? u32x4{a0, a1, r0, r1} : u32x4{r0, r1, b0, b1};
          // even: column nb + 16i; odd: nb + 16(i + 1) - 4 (both multiples of 8);
          // the logits are not read again here: streaming stores
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(row + i * 16 + (even ? 0 : 12)));
        }
      }
      return;
    }
  }
  if (pack_ok && full) {
    // whole tile in range: no per-element checks
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      uint16_t *row = out + (mb + j * 16) * ld + col_off + nb;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const u32x2 v{f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16),
                      f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16)};
        *reinterpret_cast<u32x2 *>(row + i * 16) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t m = mb + j * 16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int64_t n = nb + i * 16;
      uint16_t *dst = out + m * ld + col_off + n;
      if (pack_ok && n + 3 < N) {
        const u32x2 v{f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16),
                      f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16)};
        *reinterpret_cast<u32x2 *>(dst) = v;
      } else {
        for (int r = 0; r < 4; ++r)
          if (n + r < N) dst[r] = static_cast<uint16_t>(f32_to_bf16_bits(acc[i][j][r]));
      }
    }
  }
}

// Full-tile store through LDS.  A wave owns TN columns x FM*16 rows of the
// output; fragments j = jb .. jb+HALF-1 at a time are written to the wave's
// own LDS region as bf16 rows (row stride TN*2 + 16 bytes), then read back
// as 16-byte pieces in row order, so that each global store instruction
// covers whole contiguous runs of an output row (TN*2 bytes per row) rather
// than 16 row pieces of 64 bytes.  Requires a barrier before the first call
// (the region overlaps the K-loop stages) and 16-byte-aligned rows.
template <int FN, int FM, int TN, int HALF>
__device__ __forceinline__ void write_tile_lds(const f32x4 (&acc)[FN][FM], uint16_t *region,
                                               int64_t n_base, int64_t m_base,
                                               uint16_t *__restrict__ out, int64_t ld,
                                               int64_t col_off) {
  static_assert(FM % HALF == 0, "fragment rows must split into whole passes");
  constexpr int kStride = TN + 8;  // bf16 elements per LDS row (16 bytes of padding)
  constexpr int kRows = HALF * 16;
  constexpr int kPieces = TN / 8;  // 16-byte pieces per row
  static_assert(TN % 8 == 0 && (kRows * kPieces) % 64 == 0, "whole pieces per lane");
  const int lane = threadIdx.x & 63;
  const int frag_row = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jb = 0; jb < FM; jb += HALF) {
#pragma unroll
    for (int jj = 0; jj < HALF; ++jj)
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const u32x2 v{f32_to_bf16_bits(acc[i][jb + jj][0]) |
                          (f32_to_bf16_bits(acc[i][jb + jj][1]) << 16),
                      f32_to_bf16_bits(acc[i][jb + jj][2]) |
                          (f32_to_bf16_bits(acc[i][jb + jj][3]) << 16)};
        *reinterpret_cast<u32x2 *>(region + (jj * 16 + frag_row) * kStride + i * 16 + 4 * g) = v;
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int t = 0; t < kRows * kPieces / 64; ++t) {
      const int piece = t * 64 + lane;
      const int r = piece / kPieces, c = piece - r * kPieces;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(region + r * kStride + c * 8);
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4 *>(out + (m_base + jb * 16 + r) * ld + col_off + n_base + c * 8));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

// Tile configuration of the bf16 kernel.
//   BN x BM   tile of Z^T per workgroup (BN vocabulary rows of W, BM rows of X)
//   WN x WM   arrangement of the waves; a wave owns (BN/WN) x (BM/WM)
//   BK        K slice per pipeline step (64 or 128)
//   NS        LDS stages (filled by buffer loads that write LDS directly;
//             NS-1 steps in flight)
//   NTW       W's loads carry the non-temporal hint.  Decode-size launches
//             read every W row once (a single tile of hidden rows), and
//             streaming W that way measured 3-6% faster on MI355X for
//             M <= 32; where W tiles are shared by several row tiles the
//             hint is left off.
// The workgroup has WN * WM waves of 64 lanes.
template <int BN_, int BM_, int WN_, int WM_, int BK_, int NS_, bool NTW_ = false>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, BK = BK_, NS = NS_;
  static constexpr bool NTW = NTW_;
  static constexpr int NT = WN_ * WM_ * 64;
  static_assert(NS >= 2, "at least two LDS stages");
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LDS and export counters left alone).
[[maybe_unused]] constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Z^T tile = W_tile . X_tile^T over K, staged through LDS.  In LDS, rows
// [0, BN) of a stage hold the W slice and rows [BN, BN+BM) the X slice of a
// step.  VEC (16-byte-aligned operands, K % 8 == 0): NS stages filled by
// buffer loads that write LDS directly, NS-1 steps in flight, one barrier per
// step.  Otherwise: two stages, element-wise loads staged through registers
// (each step: barrier; read the step's fragments; write the next step from
// registers to the other stage; issue the loads of the step after; MFMAs).
//
// GX (prefill): the M rows of X are not stored contiguously; row i is the
// last position of packed sequence i, hidden[cu[i+1] - 1] with hidden
// [n_tokens, K] (so the last-position select is folded into the staging).
// ARGMAX: instead of storing logits, fold each row's largest logit (as
// rounded to bf16) and its vocabulary id into pick.best[row].
template <class C, bool VEC, bool GX, bool ARGMAX>
__global__ __launch_bounds__(C::NT) void lmhead_bf16_mfma(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, const uint16_t *__restrict__ W,
    int64_t N, uint16_t *__restrict__ out, int64_t ld, int64_t col_off, int tiles_n,
    int tiles_m, int group_n, const int32_t *__restrict__ cu, int64_t n_tokens,
    TileOut pick) {
  // (device pass only: the host pass needs no more than the launch stub)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = C::BN, BM = C::BM, WN = C::WN, WM = C::WM, BK = C::BK;
  constexpr int NT = C::NT;
  constexpr int TN = BN / WN, TM = BM / WM;
  constexpr int FN = TN / 16, FM = TM / 16;
  static_assert(FN * 16 == TN && FM * 16 == TM, "wave tile must be a multiple of 16");
  constexpr int kPieces = BK / 8;                  // 16-byte pieces per row
  constexpr int kRowsPerPass = NT / kPieces;       // rows staged per pass of the block
  constexpr int kRows = BN + BM;
  constexpr int kPPT = (kRows + kRowsPerPass - 1) / kRowsPerPass;  // pieces per thread
  constexpr int KS = BK / 32;                      // MFMA k-steps per pipeline step

  // a stage is padded to whole passes: every lane of a load writes inside it
  constexpr int kNumBuf = C::NS;
  constexpr int kBufElems = kPPT * kRowsPerPass * BK;
  __shared__ __attribute__((aligned(16))) uint16_t lds_all[kNumBuf * kBufElems];
  uint16_t(*lds)[kBufElems] = reinterpret_cast<uint16_t(*)[kBufElems]>(lds_all);

  int tn, tm;
  tile_of_block(blockIdx.x, tiles_n, tiles_m, group_n, tn, tm);
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int frag_row = lane & 15;  // row of the fragment this lane feeds
  const int frag_grp = lane >> 4;  // which 8-wide k group of a 32-wide step

  // Staging: thread t copies piece t % P of tile rows t / P + kRowsPerPass*p.
  const int srow = threadIdx.x / kPieces;
  const int spiece = threadIdx.x % kPieces;
  const int64_t nk = (K + BK - 1) / BK;
  const int64_t w_rows = (N - n0 < BN) ? N - n0 : BN;  // rows of this tile inside W / X
  const int64_t x_rows = (M - m0 < BM) ? M - m0 : BM;

  // VEC staging reads through buffer descriptors over this tile's rows: the
  // hardware range check returns zeros for rows past the end of W or X, the
  // row offset is one 32-bit register, and the K offset of a step is scalar.
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + n0 * K), 0, static_cast<int>(w_rows * K * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(GX ? X : X + m0 * K), 0,
      static_cast<int>((GX ? n_tokens : x_rows) * K * 2), kBufferFlags);
  const int row_bytes = static_cast<int>(K * 2);
  // Element offset of X-tile row r from the X descriptor's base, or -1 when
  // the row does not exist (past M, or a sequence end outside the tokens).
  auto x_row_off = [&](int r) -> int64_t {
    if (r >= x_rows) return -1;
    if constexpr (GX) {
      const int64_t t = static_cast<int64_t>(cu[m0 + r + 1]) - 1;
      return (static_cast<uint64_t>(t) < static_cast<uint64_t>(n_tokens)) ? t * K : -1;
    } else {
      return static_cast<int64_t>(r) * K;
    }
  };
  const int voff0 = srow * row_bytes + spiece * 16;
  const int row_stride_bytes = kRowsPerPass * row_bytes;

  u32x4 pre[1][kPPT];
  // Loads only; nothing waits on them before the LDS write that needs them.
  // Steps past the end are clamped to the last step (their data is unused).
  auto load_step = [&](u32x4 (&dst)[kPPT], int64_t step) {
    const int64_t k0 = (step < nk ? step : nk - 1) * BK;
#pragma unroll
    for (int p = 0; p < kPPT; ++p) {
      // tile row of this piece; passes that straddle the W/X boundary decide per lane
      const int row = srow + p * kRowsPerPass;
      const bool in_w = (BN % kRowsPerPass == 0) ? (p * kRowsPerPass < BN) : (row < BN);
      const int r = in_w ? row : row - BN;  // row inside W's or X's part of the tile
      if (VEC) {
        int voff;
        if (GX && !in_w) {
          const int64_t xo = (row < kRows) ? x_row_off(r) : -1;
          voff = xo >= 0 ? static_cast<int>(xo * 2) + spiece * 16 : kBig;
        } else {
          voff = (BN % kRowsPerPass == 0)
                     ? voff0 + (in_w ? p : p - BN / kRowsPerPass) * row_stride_bytes
                     : r * row_bytes + spiece * 16;
        }
        dst[p] = __builtin_amdgcn_raw_buffer_load_b128(in_w ? w_rsrc : x_rsrc, voff,
                                                       static_cast<int>(k0 * 2), 0);
      } else {
        const int64_t gk = k0 + spiece * 8;
        u32x4 v = u32x4(0);
        const int64_t xo = (!in_w && row < kRows) ? x_row_off(r) : -1;
        if (row < kRows && (in_w ? r < w_rows : xo >= 0)) {
          const uint16_t *q = (in_w ? W + (n0 + r) * K : (GX ? X : X + m0 * K) + xo) + gk;
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = (gk + i < K) ? q[i] : uint16_t(0);
          v = u32x4{e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                    e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)};
        }
        dst[p] = v;
      }
    }
  };
  // A step's last K slice may run past K (K is a multiple of 8 on the VEC
  // path, so a piece is either inside K or wholly past it): those pieces read
  // the next row's data through the buffer and are zeroed here.
  auto store_step = [&](const u32x4 (&src)[kPPT], uint16_t *buf, int64_t step) {
    const int64_t k0 = (step < nk ? step : nk - 1) * BK;
    const bool k_in = k0 + spiece * 8 < K;
#pragma unroll
    for (int p = 0; p < kPPT; ++p) {
      const int row = srow + p * kRowsPerPass;
      if (kRows % kRowsPerPass == 0 || row < kRows)
        *reinterpret_cast<u32x4 *>(buf + lds_piece_offset<BK>(row, spiece)) =
            (!VEC || k_in) ? src[p] : u32x4(0);
    }
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4(0.f);

  bf16x8 fa[1][KS][FN], fb[1][KS][FM];
  auto read_frags_set = [&](int set, const uint16_t *cur, int ks0, int ks1) {
#pragma unroll
    for (int ks = ks0; ks < ks1; ++ks) {
      const int piece = ks * 4 + frag_grp;
#pragma unroll
      for (int i = 0; i < FN; ++i)
        fa[set][ks][i] = *reinterpret_cast<const bf16x8 *>(
            cur + lds_piece_offset<BK>(wn * TN + i * 16 + frag_row, piece));
#pragma unroll
      for (int j = 0; j < FM; ++j)
        fb[set][ks][j] = *reinterpret_cast<const bf16x8 *>(
            cur + lds_piece_offset<BK>(BN + wm * TM + j * 16 + frag_row, piece));
    }
  };
  auto mfma_set = [&](int set, int ks0, int ks1) {
#pragma unroll
    for (int ks = ks0; ks < ks1; ++ks)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[set][ks][i], fb[set][ks][j],
                                                              acc[i][j], 0, 0, 0);
  };
  auto read_frags = [&](const uint16_t *cur, int ks0, int ks1) { read_frags_set(0, cur, ks0, ks1); };
  auto mfma_range = [&](int ks0, int ks1) { mfma_set(0, ks0, ks1); };

  if constexpr (VEC) {
    constexpr int NS = C::NS;
    constexpr int kRowsPerWaveLoad = 64 / kPieces;  // rows one wave load instruction fills
    static_assert(BN % kRowsPerWaveLoad == 0, "a load instruction must stay inside W or X");
    static_assert((NS - 2) * kPPT <= 63, "outstanding loads must fit the vmcnt counter");
    const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lrow = lane / kPieces, lslot = lane % kPieces;
    const int nk_i = static_cast<int>(nk);
    const int k_i = static_cast<int>(K);
    const int w_rows_i = static_cast<int>(w_rows), x_rows_i = static_cast<int>(x_rows);
    // One step into stage buffer `buf`: lane l of wave w fills LDS slot l % P
    // of tile row p * kRowsPerPass + w * (64 / P) + l / P, which holds piece
    // slot ^ f(row) of that row (the swizzle is applied on the global side).
    // byte offset of this lane's row in each pass from its descriptor's base,
    // or -1 for rows past the matrices (fixed for the whole tile)
    int row_off[kPPT];
    // gathered X: the sequence ends, loaded before any tile data (see below)
    int32_t cu_end[kPPT];
#pragma unroll
    for (int p = 0; p < kPPT; ++p) {
      const int row0 = p * kRowsPerPass + wave_u * kRowsPerWaveLoad;
      const int row = row0 + lrow;
      const bool in_w = (BN % kRowsPerPass == 0) ? (p * kRowsPerPass < BN) : (row0 < BN);
      cu_end[p] = 0;
      if (in_w) {
        row_off[p] = row < w_rows_i ? row * row_bytes : -1;
      } else if constexpr (GX) {
        const int r = row - BN;
        const bool exists = row < kRows && r < x_rows_i;
        row_off[p] = -1;
        if (exists) cu_end[p] = cu[m0 + r + 1];
      } else {
        const int64_t xo = (row < kRows) ? x_row_off(row - BN) : -1;
        row_off[p] = xo >= 0 ? static_cast<int>(xo * 2) : -1;
      }
    }
    // X row offsets of a gathered X, from the sequence ends; the first use of
    // the loaded ends comes after stage 0's W loads have been issued, so their
    // latency overlaps (vmcnt is in order: the ends were issued first)
    auto gather_offsets = [&]() {
#pragma unroll
      for (int p = 0; p < kPPT; ++p) {
        const int row0 = p * kRowsPerPass + wave_u * kRowsPerWaveLoad;
        const int row = row0 + lrow;
        const bool in_w = (BN % kRowsPerPass == 0) ? (p * kRowsPerPass < BN) : (row0 < BN);
        if (in_w) continue;
        pin_vgpr(cu_end[p]);
        const int r = row - BN;
        const int64_t t = static_cast<int64_t>(cu_end[p]) - 1;
        const bool ok = row < kRows && r < x_rows_i &&
                        static_cast<uint64_t>(t) < static_cast<uint64_t>(n_tokens);
        row_off[p] = ok ? static_cast<int>(t * K * 2) : -1;
      }
    };
    // part: 0 = the whole step, 1 = only passes that start inside W, 2 = the rest
    auto dma_step = [&](int step, int buf, int part = 0) {
      const int k0 = (step < nk_i ? step : nk_i - 1) * BK;
      uint16_t *base = lds[buf];
#pragma unroll
      for (int p = 0; p < kPPT; ++p) {
        const int row0 = p * kRowsPerPass + wave_u * kRowsPerWaveLoad;  // wave-uniform
        const int row = row0 + lrow;
        const int piece = lslot ^ lds_swizzle<BK>(row);
        bool in_w;
        if constexpr (BN % kRowsPerPass == 0) in_w = p * kRowsPerPass < BN;
        else in_w = row0 < BN;
        if (part == 1 && !in_w) continue;
        if (part == 2 && in_w) continue;
        const bool ok = row_off[p] >= 0 && k0 + piece * 8 < k_i;
        const int voff = ok ? row_off[p] + piece * 16 : kBig;
        // (cache-policy immediate: 2 is the non-temporal bit of gfx950's
        // buffer loads)
        if (in_w)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              w_rsrc, (__attribute__((address_space(3))) void *)(base + row0 * BK), 16, voff,
              k0 * 2, 0, C::NTW ? 2 : 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              x_rsrc, (__attribute__((address_space(3))) void *)(base + row0 * BK), 16, voff,
              k0 * 2, 0, 0);
      }
    };
    // Stage 0's W loads go out before the first use of the X row offsets, so
    // that a gathered X (whose offsets wait on loads of cu) costs no latency.
    // Stage 0 is still wholly issued before stages 1.., which is all the
    // vmcnt count below relies on.
    dma_step(0, 0, 1);
    if constexpr (GX) gather_offsets();
    dma_step(0, 0, 2);
#pragma unroll
    for (int st = 1; st < NS - 1; ++st) dma_step(st, st);
    int rd = 0, wr = NS - 1;  // stage buffers read and refilled by the current step
    for (int kt = 0; kt < nk_i; ++kt) {
      // this wave's loads of step kt have landed once at most the later
      // NS-2 steps' loads are outstanding; the barrier extends that to all
      // waves and also closes every wave's reads of step kt-1's buffer
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kPPT));
      asm volatile("s_barrier" ::: "memory");
      dma_step(kt + NS - 1, wr);
      read_frags(lds[rd], 0, KS);
      mfma_range(0, KS);
      rd = (rd + 1 == NS) ? 0 : rd + 1;
      wr = (wr + 1 == NS) ? 0 : wr + 1;
    }
  } else {
    // register-staged two-stage pipeline: step 0 in LDS stage 0, step 1 in
    // registers; the loads of step kt+2 are issued halfway through step kt's
    // MFMAs
    load_step(pre[0], 0);
    store_step(pre[0], lds[0], 0);
    load_step(pre[0], 1);
    for (int64_t kt = 0; kt < nk; ++kt) {
      __syncthreads();
      const uint16_t *cur = lds[kt & 1];
      read_frags(cur, 0, KS);
      store_step(pre[0], lds[(kt + 1) & 1], kt + 1);
      mfma_range(0, KS / 2);
      load_step(pre[0], kt + 2);
      mfma_range(KS / 2, KS);
      __builtin_amdgcn_sched_group_barrier(0x100, KS * (FN + FM), 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x200, kPPT, 0);            // LDS writes
      __builtin_amdgcn_sched_group_barrier(0x008, (KS / 2) * FN * FM, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, kPPT, 0);            // global loads
      __builtin_amdgcn_sched_group_barrier(0x008, (KS - KS / 2) * FN * FM, 0);
    }
  }

  // the clamped loads past the last step may still be landing in LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const bool full = n0 + BN <= N && m0 + BM <= M;
  if constexpr (!ARGMAX) {
    if (pick.lse != nullptr) {
      // this W tile's log-sum-exp pair of every row; the WN waves that hold
      // the same rows (different columns) merge theirs in LDS, in wave order
      float mx[FM], sm[FM];
      lse_rows<FN, FM, true>(acc, n0 + wn * TN + 4 * frag_grp, N, full, mx, sm);
      if constexpr (WN > 1) {
        float *pl = reinterpret_cast<float *>(lds_all);  // [WM][FM][16][WN] pairs
        static_assert(WM * FM * 16 * WN * 8 <= kNumBuf * kBufElems * 2, "pairs fit the stages");
        __syncthreads();  // every wave is done with the stages
        if ((threadIdx.x & 48) == 0) {
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            float *e = pl + (((wm * FM + j) * 16 + frag_row) * WN + wn) * 2;
            e[0] = mx[j];
            e[1] = sm[j];
          }
        }
        __syncthreads();
        if (wn == 0) {
#pragma unroll
          for (int j = 0; j < FM; ++j) {
            const float *e = pl + ((wm * FM + j) * 16 + frag_row) * WN * 2;
            float m = e[0], sv = e[1];
#pragma unroll
            for (int w2 = 1; w2 < WN; ++w2) lse_merge(m, sv, e[2 * w2], e[2 * w2 + 1]);
            mx[j] = m;
            sm[j] = sv;
          }
        }
      }
      if (wn == 0 && (threadIdx.x & 48) == 0) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int64_t row = m0 + wm * TM + j * 16 + frag_row;
          if (row < M) {
            float *e = pick.lse + (row * pick.lse_ld + tn) * 2;
            e[0] = mx[j];
            e[1] = sm[j];
          }
        }
      }
    }
    if (out == nullptr) return;  // log-sum-exp only: no logits stored
  }
  if constexpr (!ARGMAX && (FM % 2 == 0) && kNumBuf * kBufElems >= NT / 64 * 32 * (TN + 8)) {
    if (full && ((ld | col_off) & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      asm volatile("s_barrier" ::: "memory");  // every wave is done with the stages
      write_tile_lds<FN, FM, TN, 2>(acc, lds_all + wave * 32 * (TN + 8), n0 + wn * TN,
                                    m0 + wm * TM, out, ld, col_off);
      return;
    }
  }
  if constexpr (ARGMAX && WN > 1) {
    // the WN waves that hold the same rows (different columns) combine their
    // keys in LDS first: one atomic per row per workgroup instead of WN
    uint64_t keys[FM];
    argmax_keys<FN, FM>(acc, n0 + wn * TN + 4 * frag_grp, full, N, pick, keys);
    uint64_t *kl = reinterpret_cast<uint64_t *>(lds_all);  // [WM][FM][16][WN]
    static_assert(WM * FM * 16 * WN * 8 <= kNumBuf * kBufElems * 2, "key exchange fits the stages");
    __syncthreads();  // every wave is done with the stages
    if ((threadIdx.x & 48) == 0) {
#pragma unroll
      for (int j = 0; j < FM; ++j) kl[((wm * FM + j) * 16 + frag_row) * WN + wn] = keys[j];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int w2 = 1; w2 < WN; ++w2)
          keys[j] = umax64(keys[j], kl[((wm * FM + j) * 16 + frag_row) * WN + w2]);
      argmax_fold<FM>(keys, m0 + wm * TM + frag_row, M, pick);
    }
    return;
  }
  write_tile<FN, FM, ARGMAX>(acc, n0 + wn * TN + 4 * frag_grp, m0 + wm * TM + frag_row, full, M,
                             N, out, ld, col_off, pick);
#endif
}

// ---------------------------------------------------------------------------
// Prefill LM head over a few gathered rows with X resident in LDS.  The BM X
// rows are the last positions of packed sequences, rows of the prefill
// activations far apart (2048-token sequences put them 4 MB apart).  Staged
// at every k step, as the kernel above does, each step of every workgroup
// touches BM distinct pages; measured on MI355X that costs ~2-5 us at the
// [32, 151936] shape against the same kernel on adjacent rows.  Here the X
// rows are loaded into LDS KC columns at a time (one load per chunk instead
// of one per k step) and only W streams through the NS stages.  At the chunk
// boundary the next chunk is loaded after the step's barrier and waited for
// (one drain of the pipeline per chunk).
// Resident layout: row q holds its KC-column chunk as 16-byte pieces, piece p
// at slot p ^ (q & 7), so the 8 lanes of a fragment read pass (8 rows, one
// piece) hit 8 distinct bank groups.
// Every output element accumulates its k steps in the same order as in
// lmhead_bf16_mfma (64-wide steps of two 32-wide MFMAs), so the logits and
// greedy-pick keys equal those of the select followed by the LM head, bit
// for bit.  Requires 16-byte aligned operands, K % 8 == 0 and gathered rows
// that fit one descriptor (checked by the launcher).
// ---------------------------------------------------------------------------
template <class C, int KC, bool ARGMAX>
__global__ __launch_bounds__(C::NT) void lmhead_bf16_gxres(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, const uint16_t *__restrict__ W,
    int64_t N, uint16_t *__restrict__ out, int64_t ld, int64_t col_off, int tiles_n,
    int tiles_m, const int32_t *__restrict__ cu, int64_t n_tokens, TileOut pick) {
  // (device pass only: the host pass needs no more than the launch stub)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BN = C::BN, BM = C::BM, WN = C::WN, WM = C::WM, BK = C::BK, NS = C::NS;
  constexpr int NT = C::NT, NW = NT / 64;
  constexpr int TN = BN / WN, TM = BM / WM;
  constexpr int FN = TN / 16, FM = TM / 16;
  static_assert(FN * 16 == TN && FM * 16 == TM, "wave tile must be a multiple of 16");
  static_assert(BK == 64 && KC % BK == 0, "chunks of whole 64-wide k steps");
  constexpr int kPieces = BK / 8, kRowsPerPass = NT / kPieces;
  constexpr int kPPT = (BN + kRowsPerPass - 1) / kRowsPerPass;  // W loads per lane per step
  constexpr int kBufElems = kPPT * kRowsPerPass * BK;
  constexpr int kRowsPerWaveLoad = 64 / kPieces;
  constexpr int KS = BK / 32, SPC = KC / BK;  // MFMA k steps per step; steps per chunk
  constexpr int PX = KC / 8;                  // 16-byte pieces per resident row
  static_assert(PX % 8 == 0 && (BM * PX) % (64 * NW) == 0, "whole chunk loads per wave");
  constexpr int XL = BM * PX / 64 / NW;       // chunk loads per lane
  static_assert((NS - 2) * kPPT <= 63 && kPPT <= 63, "outstanding loads fit the vmcnt counter");
  __shared__ __attribute__((aligned(16))) uint16_t lds_all[NS * kBufElems + BM * KC];
  uint16_t(*lds)[kBufElems] = reinterpret_cast<uint16_t(*)[kBufElems]>(lds_all);
  uint16_t *xres = lds_all + NS * kBufElems;

  int tn, tm;
  tile_of_block(blockIdx.x, tiles_n, tiles_m, 1, tn, tm);
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int frag_row = lane & 15, frag_grp = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lrow = lane / kPieces, lslot = lane % kPieces;
  const int nk = static_cast<int>((K + BK - 1) / BK);
  const int k_i = static_cast<int>(K);
  const int row_bytes = k_i * 2;
  const int w_rows = static_cast<int>((N - n0 < BN) ? N - n0 : BN);
  const int x_rows = static_cast<int>((M - m0 < BM) ? M - m0 : BM);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(W + n0 * K), 0, w_rows * row_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, static_cast<int>(n_tokens * K * 2), kBufferFlags);
  // W rows of this lane's loads (byte offsets, -1 past W)
  int w_off[kPPT];
#pragma unroll
  for (int p = 0; p < kPPT; ++p) {
    const int row = p * kRowsPerPass + wave_u * kRowsPerWaveLoad + lrow;
    w_off[p] = row < w_rows ? row * row_bytes : -1;
  }
  // Chunk load t of this wave fills flat slots [64 q, 64 q + 64) of the
  // resident rows, q = t NW + wave: this lane's row is (64 q + lane) / PX.
  // Its sequence end is loaded first; the first use comes after stage 0's W
  // loads are out.
  int32_t cu_end[XL];
#pragma unroll
  for (int t = 0; t < XL; ++t) {
    const int r = ((t * NW + wave_u) * 64 + lane) / PX;
    cu_end[t] = r < x_rows ? cu[m0 + r + 1] : 0;
  }
  auto dma_w = [&](int step, int buf) {
    const int k0 = (step < nk ? step : nk - 1) * BK;  // steps past the end reload the last
    uint16_t *base = lds[buf];
#pragma unroll
    for (int p = 0; p < kPPT; ++p) {
      const int row0 = p * kRowsPerPass + wave_u * kRowsPerWaveLoad;  // wave-uniform
      if (BN % kRowsPerPass != 0 && row0 >= BN) continue;
      const int piece = lslot ^ lds_swizzle<BK>(row0 + lrow);
      const bool ok = w_off[p] >= 0 && k0 + piece * 8 < k_i;
      // (non-temporal: each W row is read once)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          w_rsrc, (__attribute__((address_space(3))) void *)(base + row0 * BK), 16,
          ok ? w_off[p] + piece * 16 : kBig, k0 * 2, 0, 2);
    }
  };
  int x_off[XL];  // byte offset of this lane's gathered row, -1 for none
  auto dma_x = [&](int c) {
#pragma unroll
    for (int t = 0; t < XL; ++t) {
      const int q = t * NW + wave_u;
      const int f = q * 64 + lane, r = f / PX;
      const int piece = (f - r * PX) ^ (r & 7);
      const bool ok = x_off[t] >= 0 && c * KC + piece * 8 < k_i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          x_rsrc, (__attribute__((address_space(3))) void *)(xres + q * 512), 16,
          ok ? x_off[t] + piece * 16 : kBig, c * KC * 2, 0, 0);
    }
  };
  // W stage 0, then chunk 0 (its offsets wait on cu), then W stages 1..NS-2:
  // the in-order vmcnt count at step 0 then covers the chunk too
  dma_w(0, 0);
#pragma unroll
  for (int t = 0; t < XL; ++t) {
    pin_vgpr(cu_end[t]);
    const int r = ((t * NW + wave_u) * 64 + lane) / PX;
    const int64_t tk = static_cast<int64_t>(cu_end[t]) - 1;
    x_off[t] = (r < x_rows && static_cast<uint64_t>(tk) < static_cast<uint64_t>(n_tokens))
                   ? static_cast<int>(tk * K * 2) : -1;
  }
  dma_x(0);
#pragma unroll
  for (int st = 1; st < NS - 1; ++st) dma_w(st, st);

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4(0.f);
  int rd = 0, wr = NS - 1;
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of step kt have landed once at most the later NS-2
    // steps' W loads are outstanding; the barrier extends that to all waves
    // and closes every wave's reads of the buffers refilled below
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kPPT));
    asm volatile("s_barrier" ::: "memory");
    if (kt > 0 && kt % SPC == 0) {
      // every wave is past the previous chunk: load the next one and wait
      // for it (only the W step issued after it may stay in flight)
      dma_x(kt / SPC);
      dma_w(kt + NS - 1, wr);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPPT));
      asm volatile("s_barrier" ::: "memory");
    } else {
      dma_w(kt + NS - 1, wr);
    }
    const uint16_t *cur = lds[rd];
    const int xp0 = (kt % SPC) * (BK / 8);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int piece = ks * 4 + frag_grp;
      bf16x8 fa[FN], fb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        fa[i] = *reinterpret_cast<const bf16x8 *>(
            cur + lds_piece_offset<BK>(wn * TN + i * 16 + frag_row, piece));
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int q = wm * TM + j * 16 + frag_row;
        fb[j] = *reinterpret_cast<const bf16x8 *>(xres + q * KC + (((xp0 + piece) ^ (q & 7)) << 3));
      }
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    rd = (rd + 1 == NS) ? 0 : rd + 1;
    wr = (wr + 1 == NS) ? 0 : wr + 1;
  }
  // the clamped loads past the last step may still be landing in LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const bool full = n0 + BN <= N && m0 + BM <= M;
  if constexpr (ARGMAX && WN > 1) {
    // the WN waves that hold the same rows combine their keys in LDS first
    uint64_t keys[FM];
    argmax_keys<FN, FM>(acc, n0 + wn * TN + 4 * frag_grp, full, N, pick, keys);
    uint64_t *kl = reinterpret_cast<uint64_t *>(lds_all);  // [WM][FM][16][WN]
    static_assert(WM * FM * 16 * WN * 8 <= NS * kBufElems * 2, "key exchange fits the stages");
    __syncthreads();  // every wave is done with the stages
    if ((threadIdx.x & 48) == 0) {
#pragma unroll
      for (int j = 0; j < FM; ++j) kl[((wm * FM + j) * 16 + frag_row) * WN + wn] = keys[j];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int w2 = 1; w2 < WN; ++w2)
          keys[j] = umax64(keys[j], kl[((wm * FM + j) * 16 + frag_row) * WN + w2]);
      argmax_fold<FM>(keys, m0 + wm * TM + frag_row, M, pick);
    }
    return;
  }
  write_tile<FN, FM, ARGMAX>(acc, n0 + wn * TN + 4 * frag_grp, m0 + wm * TM + frag_row, full, M,
                             N, out, ld, col_off, pick);
#endif
}

// One step of W into an LDS stage: lane l of wave w fills, in pass p, LDS
// slot l % 8 of tile row p * kRowsPerPass + 8 w + l / 8 with that row's piece
// slot ^ f(row); w_off[p] is the row's byte offset (-1: no such row).
// (The descriptor over [w, w + bytes) is built here from plain arguments.)
template <int kPPT, int kRowsPerPass, int BK>
__device__ __forceinline__ void xreg_dma_w(const uint16_t *w, int bytes, uint16_t *base,
                                           const int (&w_off)[kPPT], int k0, int k_i, int wave,
                                           int lrow, int lslot) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(w), 0, bytes, kBufferFlags);
#pragma unroll
  for (int p = 0; p < kPPT; ++p) {
    const int row0 = p * kRowsPerPass + wave * 8;  // wave-uniform
    const int piece = lslot ^ lds_swizzle<BK>(row0 + lrow);
    const bool ok = w_off[p] >= 0 && k0 + piece * 8 < k_i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void *)(base + row0 * BK), 16,
        ok ? w_off[p] + piece * 16 : kBig, k0 * 2, 0, 0);
  }
}

// One step of X fragments into registers, in the MFMA operand layout: lane l
// reads the 8 bf16 at k = k0 + 32 ks + 8 (l / 16) of its row j (byte offset
// x_off[j] from x, -1: no such row); pieces past K read as zeros.
template <int KS, int FM>
__device__ __forceinline__ void xreg_load_x(const uint16_t *x, int bytes, bf16x8 (&dst)[KS][FM],
                                            const int (&x_off)[FM], int k0, int k_i,
                                            int frag_grp) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, bytes, kBufferFlags);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int piece = ks * 4 + frag_grp;
      const bool ok = x_off[j] >= 0 && k0 + piece * 8 < k_i;
      dst[ks][j] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, ok ? x_off[j] + piece * 16 : kBig,
                                                        k0 * 2, 0));
    }
}

// ---------------------------------------------------------------------------
// bf16 with X in registers.  Workgroup tile: BN vocabulary rows x WV * TM
// hidden rows over WV waves; every wave owns all BN rows of W and its own TM
// hidden rows, so a W element read from LDS feeds TM / 16 MFMAs and an X
// element held in a register feeds BN / 16 MFMAs.
//
// Only W goes through LDS: NS stages of BN x 64 bf16 filled by buffer loads
// that write LDS directly.  Each wave loads its X fragments straight into
// registers, already in the MFMA operand layout (lane l: hidden row l % 16,
// k group l / 16), one register set per step in flight.  W and X of step
// kt + NS - 1 are issued together at step kt, so NS - 1 whole steps are in
// flight and the in-order vmcnt count covers both.  Compared with staging X
// through LDS as well, the same LDS holds three steps of W instead of two,
// and a W fragment read from LDS feeds the wave's 2 X fragments while each
// X fragment feeds 20 MFMAs from its register.  Measured on MI355X it is the
// faster kernel once M spans several 256-row tiles (8-10% over the two-stage
// kernel at M = 1024 and 4096); at M = 256 the two are even in the lookup-
// then-LM-head step (5-7% apart, the other way, in back-to-back launches).
// Requires 16-byte-aligned X and W with K % 8 == 0 (checked by the launcher).
// ---------------------------------------------------------------------------
template <int BN, int WV, int TM, int NS, bool GX, bool ARGMAX>
__global__ __launch_bounds__(WV * 64) void lmhead_bf16_xreg(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, const uint16_t *__restrict__ W,
    int64_t N, uint16_t *__restrict__ out, int64_t ld, int64_t col_off, int tiles_n,
    int tiles_m, int group_n, const int32_t *__restrict__ cu, int64_t n_tokens,
    TileOut pick) {
  // (device pass only: the host pass needs no more than the launch stub)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BK = 64, KS = BK / 32;
  constexpr int FM = TM / 16, BM = WV * TM;
  constexpr int FN = BN / 16;
  static_assert(FN * 16 == BN && FM * 16 == TM, "tile sides must be multiples of 16");
  constexpr int kRowsPerPass = WV * 8;  // one load instruction fills 8 rows
  static_assert(BN % kRowsPerPass == 0, "W rows must fill whole passes");
  constexpr int kPPT = BN / kRowsPerPass;  // W loads per lane per step
  constexpr int kLoadsPerStep = kPPT + KS * FM;
  constexpr int L = NS - 1;  // steps in flight
  static_assert(L >= 1 && (L - 1) * kLoadsPerStep <= 63, "vmcnt holds at most 63 loads");
  __shared__ __attribute__((aligned(16))) uint16_t lds_all[NS * BN * BK];
  uint16_t(*lds)[BN * BK] = reinterpret_cast<uint16_t(*)[BN * BK]>(lds_all);

  int tn, tm;
  tile_of_block(blockIdx.x, tiles_n, tiles_m, group_n, tn, tm);
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int frag_row = lane & 15, frag_grp = lane >> 4;
  const int nk = static_cast<int>((K + BK - 1) / BK);
  const int k_i = static_cast<int>(K);
  const int row_bytes = static_cast<int>(K * 2);
  const int w_rows = static_cast<int>((N - n0 < BN) ? N - n0 : BN);
  const int x_rows = static_cast<int>((M - m0 < BM) ? M - m0 : BM);

  // X rows of this lane's fragments (byte offsets from the X descriptor's
  // base, -1 for rows that do not exist).  The sequence ends of a gathered X
  // are loaded first; their first use comes after step 0's W loads are out.
  int x_off[FM];
  int32_t cu_end[FM];
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int r = wave * TM + j * 16 + frag_row;
    cu_end[j] = 0;
    if constexpr (GX) {
      x_off[j] = -1;
      if (r < x_rows) cu_end[j] = cu[m0 + r + 1];
    } else {
      x_off[j] = r < x_rows ? r * row_bytes : -1;
    }
  }
  // W rows this lane loads: pass p, tile row p * 8 WV + 8 wave + lane / 8,
  // LDS slot lane % 8 (holding that row's piece slot ^ f(row))
  const int lrow = lane >> 3, lslot = lane & 7;
  int w_off[kPPT];
#pragma unroll
  for (int p = 0; p < kPPT; ++p) {
    const int row = p * kRowsPerPass + wave * 8 + lrow;
    w_off[p] = row < w_rows ? row * row_bytes : -1;
  }
  const uint16_t *w_base = W + n0 * K;
  const int w_bytes = w_rows * row_bytes;
  const uint16_t *x_base = GX ? X : X + m0 * K;
  const int x_bytes = static_cast<int>((GX ? n_tokens : x_rows) * K * 2);
#define VPE_DMA_W(step, buf)                                                                  \
  xreg_dma_w<kPPT, kRowsPerPass, BK>(w_base, w_bytes, lds[buf], w_off,                       \
                                     ((step) < nk ? (step) : nk - 1) * BK, k_i, wave, lrow, lslot)
#define VPE_LOAD_X(step, dst)                                                                 \
  xreg_load_x<KS, FM>(x_base, x_bytes, dst, x_off, ((step) < nk ? (step) : nk - 1) * BK, k_i, \
                      frag_grp)

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4(0.f);
  bf16x8 xr[NS][KS][FM];

  VPE_DMA_W(0, 0);
  if constexpr (GX) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      pin_vgpr(cu_end[j]);
      const int r = wave * TM + j * 16 + frag_row;
      const int64_t t = static_cast<int64_t>(cu_end[j]) - 1;
      const bool ok = r < x_rows && static_cast<uint64_t>(t) < static_cast<uint64_t>(n_tokens);
      x_off[j] = ok ? static_cast<int>(t * K * 2) : -1;
    }
  }
  VPE_LOAD_X(0, xr[0]);
#pragma unroll
  for (int st = 1; st < L; ++st) {
    VPE_DMA_W(st, st);
    VPE_LOAD_X(st, xr[st]);
  }

  for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (kb + u >= nk) break;
      // this wave's W and X of step kb+u have landed once at most the later
      // L-1 steps' loads are outstanding; the barrier makes every wave's W
      // visible and closes all reads of the buffer refilled below
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((L - 1) * kLoadsPerStep));
      asm volatile("s_barrier" ::: "memory");
      VPE_DMA_W(kb + u + L, (u + L) % NS);
      VPE_LOAD_X(kb + u + L, xr[(u + L) % NS]);
      const uint16_t *cur = lds[u];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const bf16x8 wf = *reinterpret_cast<const bf16x8 *>(
              cur + lds_piece_offset<BK>(i * 16 + frag_row, ks * 4 + frag_grp));
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xr[u][ks][j], acc[i][j], 0,
                                                                0, 0);
        }
      // schedule: the step's loads first, then each W fragment read kAhead
      // fragments before the MFMAs that use it
      constexpr int kAhead = 3;
      __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerStep, 0);  // buffer loads
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);         // LDS reads
#pragma unroll
      for (int f = 0; f < KS * FN - kAhead; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);  // MFMAs of fragment f
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // read of fragment f + kAhead
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead * FM, 0);
    }
  }
#undef VPE_DMA_W
#undef VPE_LOAD_X
  // the clamped loads past the last step may still be landing
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const bool full = n0 + BN <= N && m0 + BM <= M;
  if constexpr (!ARGMAX) {
    if (pick.lse != nullptr) {
      // a wave holds whole rows of the tile: its pairs are the tile's
      float mx[FM], sm[FM];
      lse_rows<FN, FM, true>(acc, n0 + 4 * frag_grp, N, full, mx, sm);
      if ((threadIdx.x & 48) == 0) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int64_t row = m0 + wave * TM + j * 16 + frag_row;
          if (row < M) {
            float *e = pick.lse + (row * pick.lse_ld + tn) * 2;
            e[0] = mx[j];
            e[1] = sm[j];
          }
        }
      }
    }
    if (out == nullptr) return;  // log-sum-exp only: no logits stored
  }
  if constexpr (!ARGMAX && NS * BN * BK >= WV * 16 * (BN + 8)) {
    if (full && ((ld | col_off) & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      asm volatile("s_barrier" ::: "memory");  // every wave is done with the stages
      write_tile_lds<FN, FM, BN, 1>(acc, lds_all + wave * 16 * (BN + 8), n0, m0 + wave * TM,
                                    out, ld, col_off);
      return;
    }
  }
  write_tile<FN, FM, ARGMAX>(acc, n0 + 4 * frag_grp, m0 + wave * TM + frag_row, full, M, N, out,
                             ld, col_off, pick);
#endif
}

// ---------------------------------------------------------------------------
// fp32: 64 x 64 output tile per workgroup, 4 x 4 outputs per thread.
// ---------------------------------------------------------------------------
// With cu != nullptr, row i of X is hidden[cu[i+1] - 1] of X = hidden [n_tokens, K]
// (zeros when that index is outside [0, n_tokens)).
// With pick.best != nullptr each row's largest logit and its id are folded
// into pick.best[row] instead of storing the logits.
__global__ __launch_bounds__(kBlock) void lmhead_f32_tiled(const float *__restrict__ X, int64_t M,
                                                          int64_t K, const float *__restrict__ W,
                                                          int64_t N, float *__restrict__ out,
                                                          int64_t ld, int64_t col_off,
                                                          const int32_t *__restrict__ cu,
                                                          int64_t n_tokens, TileOut pick) {
  constexpr int T = 64, TK = 16;
  __shared__ float sX[TK][T + 1];
  __shared__ float sW[TK][T + 1];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * T;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += TK) {
    for (int e = threadIdx.x; e < T * TK; e += kBlock) {
      const int r = e / TK, kk = e % TK;
      const int64_t k = k0 + kk;
      int64_t xr = m0 + r;
      bool xok = xr < M && k < K;
      if (cu != nullptr && xok) {
        xr = static_cast<int64_t>(cu[m0 + r + 1]) - 1;
        xok = static_cast<uint64_t>(xr) < static_cast<uint64_t>(n_tokens);
      }
      sX[kk][r] = xok ? X[xr * K + k] : 0.f;
      sW[kk][r] = (n0 + r < N && k < K) ? W[(n0 + r) * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sX[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sW[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (pick.best != nullptr) {
    // the 16 threads with the same ty (consecutive lanes) share rows ty*4 + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + ty * 4 + i;
      uint64_t key = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tx * 4 + j;
        if (n < N) key = umax64(key, pick_key(acc[i][j], pick.id_base + n));
      }
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) key = umax64(key, __shfl_xor(key, d));
      if (tx == 0 && m < M) atomicMax(reinterpret_cast<unsigned long long *>(pick.best + m),
                                      static_cast<unsigned long long>(key));
    }
    return;
  }
  if (pick.lse != nullptr) {
    // the 16 threads with the same ty hold rows ty*4 + i: merge their pairs
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + ty * 4 + i;
      float mx = -__builtin_huge_valf(), sm = 0.f;
      const int64_t left = N - (n0 + tx * 4);  // this thread's columns below N: j < left
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = (j < left) ? nan_max(mx, acc[i][j]) : mx;
      const bool any = mx != -__builtin_huge_valf();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = __expf(acc[i][j] - mx);
        sm += (any && j < left) ? e : 0.f;
      }
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) lse_merge(mx, sm, __shfl_xor(mx, d), __shfl_xor(sm, d));
      if (tx == 0 && m < M) {
        float *e = pick.lse + (m * pick.lse_ld + blockIdx.x) * 2;
        e[0] = mx;
        e[1] = sm;
      }
    }
    if (out == nullptr) return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < N) out[m * ld + col_off + n] = acc[i][j];
    }
  }
}

__global__ __launch_bounds__(kBlock) void argmax_init_kernel(uint64_t *__restrict__ best, int64_t m) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < m) best[i] = 0;
}

// key -> (logit, id): the inverse of pick_key
// CLEAR: each key is also reset to 0 once read (by the thread that read it),
// which leaves best ready for the next fold without a separate init.
template <bool CLEAR>
__global__ __launch_bounds__(kBlock) void argmax_decode_kernel(uint64_t *__restrict__ best,
                                                              int64_t m, float *__restrict__ value,
                                                              int64_t *__restrict__ id) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= m) return;
  const uint64_t key = best[i];
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  if (value != nullptr) value[i] = __uint_as_float(u);
  if (id != nullptr) id[i] = static_cast<int64_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
  if constexpr (CLEAR) best[i] = 0;
}

// One shard's log-sum-exp of every row from its W tiles' pairs (row-major
// [m][tiles] pairs): one wave per row; lane l merges tiles l, l + 64, ... in
// order, then the lanes merge in a fixed butterfly, so the result does not
// depend on timing.
__global__ __launch_bounds__(kBlock) void lse_tiles_kernel(const float *__restrict__ part,
                                                          int tiles, int64_t m,
                                                          float *__restrict__ shard_lse) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + (threadIdx.x >> 6);
  if (row >= m) return;  // (wave-uniform)
  const int lane = threadIdx.x & 63;
  const float *p = part + row * tiles * 2;
  float mx = -__builtin_huge_valf(), sm = 0.f;
  for (int t = lane; t < tiles; t += 64) lse_merge(mx, sm, p[2 * t], p[2 * t + 1]);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) lse_merge(mx, sm, __shfl_xor(mx, d), __shfl_xor(sm, d));
  if (lane == 0) shard_lse[row] = mx + logf(sm);  // (-inf for a row with no finite pair)
}

struct LseParts {
  const float *p[64];
};

// The log-sum-exp of rows split over shards from the shards' values, merged
// in shard order: lse = mx + log(sum_r exp(lse_r - mx)), mx = max_r lse_r.
__global__ __launch_bounds__(kBlock) void lse_combine_kernel(LseParts parts, int n_parts,
                                                            int64_t m, float *__restrict__ lse) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= m) return;
  float mx = -__builtin_huge_valf();
  for (int r = 0; r < n_parts; ++r) mx = fmaxf(mx, parts.p[r][i]);
  float sm = 0.f;
  if (mx != -__builtin_huge_valf())
    for (int r = 0; r < n_parts; ++r) sm += expf(parts.p[r][i] - mx);
  lse[i] = mx == -__builtin_huge_valf() ? mx : mx + logf(sm);
}

template <class C>
int launch_bf16_cfg(const uint16_t *x, int64_t m, int64_t k, const uint16_t *w, int64_t n,
                    uint16_t *out, int64_t ld, int64_t col_off, hipStream_t st, int group_n,
                    const int32_t *cu, int64_t n_tokens, TileOut &pick) {
  const int64_t tn64 = (n + C::BN - 1) / C::BN, tm64 = (m + C::BM - 1) / C::BM;
  if (tn64 * tm64 > INT32_MAX) return static_cast<int>(hipErrorInvalidValue);
  pick.lse_ld = tn64;
  if (pick.lse != nullptr && tn64 > pick.lse_cap / m) return kErrWorkspace;
  const int tiles_n = static_cast<int>(tn64);
  const int tiles_m = static_cast<int>(tm64);
  const dim3 grid(static_cast<unsigned>(tiles_n) * static_cast<unsigned>(tiles_m));
  const bool gx = cu != nullptr;
  // 16-byte buffer loads need 16-byte rows and bases, and every descriptor
  // (the W tile, the X tile or all gathered tokens) must end at or before the
  // masked-load offset, so that masked loads read zeros
  const bool vec = bf16_direct_loads_ok(reinterpret_cast<uint64_t>(x),
                                        reinterpret_cast<uint64_t>(w), k, gx, n_tokens, C::BM,
                                        C::BN);
#define VPE_LAUNCH(V, G)                                                                     \
  do {                                                                                       \
    if (pick.best)                                                                           \
      hipLaunchKernelGGL((lmhead_bf16_mfma<C, V, G, true>), grid, dim3(C::NT), 0, st, x, m, k, w, \
                         n, out, ld, col_off, tiles_n, tiles_m, group_n, cu, n_tokens, pick);  \
    else                                                                                     \
      hipLaunchKernelGGL((lmhead_bf16_mfma<C, V, G, false>), grid, dim3(C::NT), 0, st, x, m, k,  \
                         w, n, out, ld, col_off, tiles_n, tiles_m, group_n, cu, n_tokens, pick); \
  } while (0)
  if (gx) {
    if (vec) VPE_LAUNCH(true, true);
    else VPE_LAUNCH(false, true);
  } else {
    if (vec) VPE_LAUNCH(true, false);
    else VPE_LAUNCH(false, false);
  }
#undef VPE_LAUNCH
  return 0;
}


// The X-in-registers kernel (see lmhead_bf16_xreg); false when its operand
// requirements do not hold and the caller must take another kernel.
template <int BN, int WV, int TM, int NS>
bool launch_bf16_xreg(const uint16_t *x, int64_t m, int64_t k, const uint16_t *w, int64_t n,
                      uint16_t *out, int64_t ld, int64_t col_off, hipStream_t st, int group_n,
                      const int32_t *cu, int64_t n_tokens, TileOut &pick, int *rc) {
  const bool gx = cu != nullptr;
  const bool vec = bf16_direct_loads_ok(reinterpret_cast<uint64_t>(x),
                                        reinterpret_cast<uint64_t>(w), k, gx, n_tokens, WV * TM,
                                        BN);
  if (!vec) return false;
  const int64_t tn64 = (n + BN - 1) / BN, tm64 = (m + WV * TM - 1) / (WV * TM);
  if (tn64 * tm64 > INT32_MAX) {
    *rc = static_cast<int>(hipErrorInvalidValue);
    return true;
  }
  const int tiles_n = static_cast<int>(tn64), tiles_m = static_cast<int>(tm64);
  const dim3 grid(static_cast<unsigned>(tiles_n) * static_cast<unsigned>(tiles_m));
  pick.lse_ld = tn64;
  if (pick.lse != nullptr && tn64 > pick.lse_cap / m) {
    *rc = kErrWorkspace;
    return true;
  }
#define VPE_XREG(G, A)                                                                       \
  hipLaunchKernelGGL((lmhead_bf16_xreg<BN, WV, TM, NS, G, A>), grid, dim3(WV * 64), 0, st, x, m, \
                     k, w, n, out, ld, col_off, tiles_n, tiles_m, group_n, cu, n_tokens, pick)
  if (gx) {
    if (pick.best) VPE_XREG(true, true);
    else VPE_XREG(true, false);
  } else {
    if (pick.best) VPE_XREG(false, true);
    else VPE_XREG(false, false);
  }
#undef VPE_XREG
  *rc = 0;
  return true;
}

// The resident-X gathered kernel (see lmhead_bf16_gxres); false when its
// operand requirements do not hold and the caller must take another kernel.
template <class C, int KC>
bool launch_bf16_gxres(const uint16_t *x, int64_t m, int64_t k, const uint16_t *w, int64_t n,
                       uint16_t *out, int64_t ld, int64_t col_off, hipStream_t st,
                       const int32_t *cu, int64_t n_tokens, TileOut &pick, int *rc) {
  if (cu == nullptr || pick.lse != nullptr ||
      !bf16_direct_loads_ok(reinterpret_cast<uint64_t>(x), reinterpret_cast<uint64_t>(w), k, true,
                            n_tokens, C::BM, C::BN))
    return false;
  const int64_t tn64 = (n + C::BN - 1) / C::BN, tm64 = (m + C::BM - 1) / C::BM;
  if (tn64 * tm64 > INT32_MAX) {
    *rc = static_cast<int>(hipErrorInvalidValue);
    return true;
  }
  const int tiles_n = static_cast<int>(tn64), tiles_m = static_cast<int>(tm64);
  const dim3 grid(static_cast<unsigned>(tiles_n) * static_cast<unsigned>(tiles_m));
  if (pick.best)
    hipLaunchKernelGGL((lmhead_bf16_gxres<C, KC, true>), grid, dim3(C::NT), 0, st, x, m, k, w, n,
                       out, ld, col_off, tiles_n, tiles_m, cu, n_tokens, pick);
  else
    hipLaunchKernelGGL((lmhead_bf16_gxres<C, KC, false>), grid, dim3(C::NT), 0, st, x, m, k, w, n,
                       out, ld, col_off, tiles_n, tiles_m, cu, n_tokens, pick);
  *rc = 0;
  return true;
}

// After an LM head whose tiles wrote log-sum-exp pairs (pick.lse), the merge
// of each row's pairs into shard_lse.
int finish_lse(const TileOut &pick, int64_t m, float *shard_lse, hipStream_t st) {
  const int rc = static_cast<int>(hipGetLastError());
  if (rc != 0 || pick.lse == nullptr) return rc;
  const dim3 grid(static_cast<unsigned>((m + kBlock / 64 - 1) / (kBlock / 64)));
  hipLaunchKernelGGL(lse_tiles_kernel, grid, dim3(kBlock), 0, st, pick.lse,
                     static_cast<int>(pick.lse_ld), m, shard_lse);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_lmhead(const void *x, int64_t m, int64_t k, const void *w, int64_t n, int dtype,
                  void *logits, int64_t ld, int64_t col_offset, void *stream,
                  const int32_t *cu, int64_t n_tokens, uint64_t *best, int64_t id_base,
                  float *lse_part, int64_t lse_cap, float *shard_lse) {
  TileOut pick{best, id_base, lse_part, 0, lse_cap};
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status below is this launch's
  if (dtype == 0) {
    const dim3 grid(static_cast<unsigned>((n + 63) / 64), static_cast<unsigned>((m + 63) / 64));
    pick.lse_ld = grid.x;
    if (pick.lse != nullptr && pick.lse_ld > pick.lse_cap / m) return kErrWorkspace;
    hipLaunchKernelGGL(lmhead_f32_tiled, grid, dim3(kBlock), 0, st, static_cast<const float *>(x),
                       m, k, static_cast<const float *>(w), n, static_cast<float *>(logits), ld,
                       col_offset, cu, n_tokens, pick);
    return finish_lse(pick, m, shard_lse, st);
  }
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  const uint16_t *wb = static_cast<const uint16_t *>(w);
  uint16_t *ob = static_cast<uint16_t *>(logits);
  // Tile shapes by the number of hidden rows M (measured on MI355X):
  //  - M <= 64 (decode-size batches): the LM head streams W once and is
  //    bound by HBM, so tiles are narrow and there are many of them, with
  //    two to four LDS stages keeping W loads well ahead of the MFMAs.
  //    M <= 16: 64 vocabulary rows with 128-wide k steps (a sweep over tile heights
  //    32-192, k steps 64/128 and 3-6 stages found it best or within 2% on
  //    75968- and 151936-row tables at D = 1024 and on 37984 x 4096).
  //    M <= 32: 128-row tiles, or 64-row ones when there would be fewer
  //    than 512 tiles (long rows, e.g. 37984 x 4096: 16% faster); M <= 64:
  //    128-row tiles.  The 128-row tiles take three stages, not four: at
  //    61-74 KB of LDS two workgroups share a CU (M = 64: 6% faster; the
  //    fused prefill select at M = 32: 3%).  Where 192-row tiles fit one
  //    round at two workgroups per CU (a 75968 x 1024 shard), they replace
  //    the 64- and 128-row ones: 4-10% faster for M = 16-64 there, within
  //    1% at M = 1 and 8 (and slower on the full table, where they do not).
  //    25 <= M <= 32 takes them on long tables too (the full 151936-row
  //    table: 2-3% faster, the fused prefill select included; at M = 24
  //    they were 3% slower there);
  //  - 64 < M <= 128: 256 x 128 tiles over 8 waves, three stages, or
  //    320 x 128 with two stages where that fits one round and 256 rows do
  //    not (the 75968-row shard: 20% faster at M = 96 and 128), its W read
  //    once and so loaded non-temporally (another 6% in the step);
  //  - 128 < M <= 256: 320 vocabulary rows x 256 hidden rows over 8 waves
  //    (a wave owns 160 x 64), W and X both staged through two LDS stages.
  //    A 75968-row shard is 238 W tiles: one round over 256 CUs, with 0.35
  //    KB of LDS fragment reads per MFMA;
  //  - M > 256: the same tile with X in registers (lmhead_bf16_xreg), three
  //    W stages in LDS; tiles ordered in groups of 8 W tiles, so that an
  //    XCD's ~32 concurrent tiles share 8 W tiles and 4 X tiles in its L2
  //    (groups of 8 measured 5-7% faster than groups of 2 or 4 at M = 4096).
  // 16-byte loads straight to LDS need K % 8 == 0, 16-byte-aligned bases and
  // descriptors that end before the masked-load offset (every tile below has
  // at most 320 W rows and 256 X rows; gathered X spans all n_tokens rows)
  const bool direct_ok = bf16_direct_loads_ok(reinterpret_cast<uint64_t>(x),
                                              reinterpret_cast<uint64_t>(w), k, cu != nullptr,
                                              n_tokens, 256, 320);
  int rc;
  const bool few_tiles = (n + 127) / 128 < 512;
  // 192-row decode tiles (two LDS stages, two workgroups per CU) when they
  // fit one round over the 256 CUs at two per CU, e.g. a 75968-row shard
  // (396 tiles, where 128-row tiles spill 82 tiles into a second round)
  const bool one_round_192 = !few_tiles && (n + 191) / 192 <= 2 * 256;
  // 320 x 128 tiles (one workgroup per CU) when 256-row ones would spill past
  // one round and 320-row ones fit it (the 75968-row shard: 238 tiles)
  const bool one_round_320 = direct_ok && (n + 255) / 256 > 256 && (n + 319) / 320 <= 256;
  // Prefill over at most 32 gathered rows (the last positions of packed
  // sequences): X resident in LDS, 128 x 32 tiles, three W stages, 256-column
  // chunks (64 KB of LDS with the stages: two workgroups per CU).  On the
  // [32, 151936] prefill shape 58.1-58.3 against 60.3-60.7 us for the kernel
  // that restages the gathered rows at every k step; 55.0 against 59.0 us at
  // 16 rows; 73.1 against 75.5 us on 37984 x 4096.
  if (cu != nullptr && m <= 32 &&
      launch_bf16_gxres<Cfg<128, 32, 4, 1, 64, 3, true>, 256>(xb, m, k, wb, n, ob, ld, col_offset,
                                                              st, cu, n_tokens, pick, &rc))
    ;
  else if (m <= 16 && one_round_192)
    rc = launch_bf16_cfg<Cfg<192, 16, 4, 1, 64, 2, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 16)
    rc = launch_bf16_cfg<Cfg<64, 16, 4, 1, 128, 4, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 32 && few_tiles)
    rc = launch_bf16_cfg<Cfg<64, 32, 4, 1, 64, 4, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 32 && (one_round_192 || m > 24))
    rc = launch_bf16_cfg<Cfg<192, 32, 4, 1, 64, 2, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 32)
    rc = launch_bf16_cfg<Cfg<128, 32, 4, 1, 64, 3, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 64 && one_round_192)
    rc = launch_bf16_cfg<Cfg<192, 64, 4, 1, 64, 2, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 64)
    rc = launch_bf16_cfg<Cfg<128, 64, 4, 1, 64, 3, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 128 && one_round_320)
    rc = launch_bf16_cfg<Cfg<320, 128, 4, 2, 64, 2, true>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  else if (m <= 128 || !direct_ok)
    // (operands that cannot take 16-byte loads go through registers; the
    // 256 x 128 tile keeps that path free of spills)
    rc = launch_bf16_cfg<Cfg<256, 128, 4, 2, 64, 3>>(xb, m, k, wb, n, ob, ld, col_offset, st, 4, cu, n_tokens, pick);
  else if (m <= 256 || !launch_bf16_xreg<320, 8, 32, 3>(xb, m, k, wb, n, ob, ld, col_offset, st,
                                                       8, cu, n_tokens, pick, &rc))
    rc = launch_bf16_cfg<Cfg<320, 256, 2, 4, 64, 2>>(xb, m, k, wb, n, ob, ld, col_offset, st, 1, cu, n_tokens, pick);
  if (rc != 0) return rc;
  return finish_lse(pick, m, shard_lse, st);
}

// ---------------------------------------------------------------------------
// Allocation-free log-sum-exp: the tile pairs go to a static device array the
// library holds on every GPU it runs on, instead of a caller workspace.  Host
// code never uses the array's name as an address: each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device the stream's work runs on (the current device for the null
// stream), and that device's address of `scratch`, resolved on first use.
int scratch_for_stream(hipStream_t st, void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (st != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(st, &sd);
    if (e != hipSuccess) return static_cast<int>(e);
    dev = static_cast<int>(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = 0;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void *p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = err;
  });
  if (g_scratch_err[dev] != hipSuccess) return static_cast<int>(g_scratch_err[dev]);
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace

int launch_lmhead_logsumexp_noalloc(const void *x, int64_t m, int64_t k, const void *w,
                                    int64_t n, int dtype, void *logits, int64_t ld,
                                    int64_t col_offset, float *shard_lse, void *stream) {
  void *ptr = nullptr;
  const int rc = scratch_for_stream(static_cast<hipStream_t>(stream), &ptr);
  if (rc != 0) return rc;
  return launch_lmhead(x, m, k, w, n, dtype, logits, ld, col_offset, stream, nullptr, 0, nullptr,
                       0, static_cast<float *>(ptr),
                       static_cast<int64_t>(kNoAllocScratchBytes / 8), shard_lse);
}

int launch_logsumexp_combine(const float *const *parts, int n_parts, int64_t m, float *lse,
                             void *stream) {
  (void)hipGetLastError();
  LseParts pl{};
  for (int r = 0; r < n_parts; ++r) pl.p[r] = parts[r];
  const dim3 grid(static_cast<unsigned>((m + kBlock - 1) / kBlock));
  hipLaunchKernelGGL(lse_combine_kernel, grid, dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     pl, n_parts, m, lse);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpe

namespace vpe {

int launch_argmax_init(uint64_t *best, int64_t m, void *stream) {
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>((m + kBlock - 1) / kBlock));
  hipLaunchKernelGGL(argmax_init_kernel, grid, dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                     best, m);
  return static_cast<int>(hipGetLastError());
}

int launch_argmax_decode(const uint64_t *best, int64_t m, float *value, int64_t *id,
                         void *stream) {
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>((m + kBlock - 1) / kBlock));
  // (the non-clearing kernel only reads best)
  hipLaunchKernelGGL(argmax_decode_kernel<false>, grid, dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), const_cast<uint64_t *>(best), m, value, id);
  return static_cast<int>(hipGetLastError());
}

int launch_argmax_decode_clear(uint64_t *best, int64_t m, float *value, int64_t *id,
                               void *stream) {
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>((m + kBlock - 1) / kBlock));
  hipLaunchKernelGGL(argmax_decode_kernel<true>, grid, dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), best, m, value, id);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpe
