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
// bf16: matrix-core kernel.  Each 256-thread workgroup owns a BN x BM tile
// of Z^T (BN vocabulary rows by BM hidden rows); tiles of W and X for a
// 64-wide slice of K are staged through LDS and consumed by
// v_mfma_f32_16x16x32_bf16.  W is the MFMA "A" operand (16 vocabulary rows per
// fragment) and X the "B" operand, so each lane ends up owning 4 consecutive
// vocabulary columns of one logits row: the epilogue writes 8-byte pieces.
// fp32: a plain LDS-tiled FMA kernel (fp32 shards are small test shapes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vpe_launch.h"

namespace vpe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;

// binary32 -> bf16 bits, round to nearest, ties to even; NaN becomes a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// LDS tile layout: rows of BK = 64 bf16 (128 bytes = 8 pieces of 16 bytes).
// Piece p of row r is stored at piece slot p ^ (r & 7), so the 16 rows one
// MFMA fragment reads at the same k land in 8 different bank groups.
// ---------------------------------------------------------------------------
constexpr int BK = 64;
constexpr int kPieces = BK / 8;

__device__ __forceinline__ int lds_piece_offset(int row, int piece) {
  return row * BK + ((piece ^ (row & 7)) << 3);  // in bf16 elements
}

// Workgroup tile order.  Work-groups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8), and each XCD has its own L2.  Block b is
// mapped to a logical tile index so that every XCD works through one
// contiguous run of logical tiles, and logical tiles are ordered W-tile-major
// (all X row blocks of one W tile are consecutive): the tiles an XCD runs at
// the same time share W tiles, the large operand, in that XCD's L2.
__device__ __forceinline__ void tile_of_block(int b, int tiles_n, int tiles_m, int &tn, int &tm) {
  const int total = tiles_n * tiles_m;
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  const int t = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  tn = t / tiles_m;
  tm = t - tn * tiles_m;
}

// BN x BM tile of Z^T per workgroup (BN vocabulary rows of W, BM rows of X);
// waves arranged WN x WM, each owning FN x FM fragments of 16 x 16.
// K is walked in 64-wide steps through two LDS buffers: while the MFMAs of
// step k read one buffer, the global loads of step k+1 are in flight into
// registers, and are written to the other buffer afterwards (one barrier per
// step).  In LDS, rows [0, BN) hold the W slice and rows [BN, BN+BM) the X
// slice of the step.
template <int BN, int BM, int WN, int WM, bool VEC>
__global__ __launch_bounds__(kBlock) void lmhead_bf16_mfma(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, const uint16_t *__restrict__ W,
    int64_t N, uint16_t *__restrict__ out, int64_t ld, int64_t col_off, int tiles_n,
    int tiles_m) {
  static_assert(WN * WM == kBlock / 64, "4 waves per workgroup");
  constexpr int TN = BN / WN, TM = BM / WM;
  constexpr int FN = TN / 16, FM = TM / 16;
  static_assert(FN * 16 == TN && FM * 16 == TM, "wave tile must be a multiple of 16");
  constexpr int kRows = BN + BM;
  constexpr int kTilePieces = kRows * kPieces;
  constexpr int kPiecesPerThread = (kTilePieces + kBlock - 1) / kBlock;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kRows * BK];

  int tn, tm;
  tile_of_block(blockIdx.x, tiles_n, tiles_m, tn, tm);
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int frag_row = lane & 15;  // row of the fragment this lane feeds
  const int frag_grp = lane >> 4;  // which 8-wide k group of a 32-wide step

  // Staging: thread t copies piece t % 8 (8 k values) of tile rows
  // t / 8 + 32 p, p = 0, 1, ...; tile rows [0, BN) are W rows n0 + r, rows
  // [BN, BN + BM) are X rows m0 + r - BN.  BN is a multiple of 32, so each p
  // falls wholly in the W part or the X part, and in LDS the pieces of one
  // thread sit 32 rows (32 * BK elements) apart: the XOR swizzle depends on
  // the row modulo 8 only.
  static_assert(BN % 32 == 0, "W part of the tile must be a multiple of 32 rows");
  constexpr int kRowsPerPass = kBlock / kPieces;  // 32
  const int srow = threadIdx.x / kPieces;
  const int spiece = threadIdx.x % kPieces;
  const int64_t w_left = N - n0 - srow;        // W rows this thread may still stage
  const int64_t x_left = M - m0 - srow;
  const uint16_t *w_src = W + (w_left > 0 ? n0 + srow : 0) * K + spiece * 8;
  const uint16_t *x_src = X + (x_left > 0 ? m0 + srow : 0) * K + spiece * 8;
  const int lds_off0 = lds_piece_offset(srow, spiece);

  // piece p of this thread is in range (row exists, k slice inside K)
  auto piece_ok = [&](int p, int64_t k0) {
    const int row = srow + p * kRowsPerPass;
    const bool in_w = p * kRowsPerPass < BN;
    const int64_t r = in_w ? p * kRowsPerPass : p * kRowsPerPass - BN;
    return row < kRows && (in_w ? r < w_left : r < x_left) && k0 + spiece * 8 < K;
  };
  auto piece_src = [&](int p, int64_t k0) {
    const bool in_w = p * kRowsPerPass < BN;
    const int64_t r = in_w ? p * kRowsPerPass : p * kRowsPerPass - BN;
    return (in_w ? w_src : x_src) + r * K + k0;
  };

  u32x4 pre[kPiecesPerThread];
  // Loads only: out-of-range pieces are loaded from the operand's first row
  // (always valid) and replaced by zeros when stored, so nothing waits on a
  // load before the LDS store that needs it.
  auto load_step = [&](int64_t k0) {
#pragma unroll
    for (int p = 0; p < kPiecesPerThread; ++p) {
      if (VEC) {
        const bool ok = piece_ok(p, k0);
        const uint16_t *q = ok ? piece_src(p, k0) : ((p * kRowsPerPass < BN) ? W : X);
        pre[p] = *reinterpret_cast<const u32x4 *>(q);
      } else {
        const int64_t gk = k0 + spiece * 8;
        u32x4 v = u32x4(0);
        if (piece_ok(p, k0)) {
          const uint16_t *q = piece_src(p, k0);
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = (gk + i < K) ? q[i] : uint16_t(0);
          v = u32x4{e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                    e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)};
        }
        pre[p] = v;
      }
    }
  };
  auto store_step = [&](uint16_t *buf, int64_t k0) {
#pragma unroll
    for (int p = 0; p < kPiecesPerThread; ++p)
      if (srow + p * kRowsPerPass < kRows)
        *reinterpret_cast<u32x4 *>(buf + lds_off0 + p * kRowsPerPass * BK) =
            (!VEC || piece_ok(p, k0)) ? pre[p] : u32x4(0);
  };

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4(0.f);

  const int64_t nk = (K + BK - 1) / BK;
  load_step(0);
  store_step(lds[0], 0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const uint16_t *cur = lds[kt & 1];
    if (kt + 1 < nk) load_step((kt + 1) * BK);
    // every fragment of the step is requested before the first MFMA: LDS
    // returns in order, so MFMAs on the first 32-wide half start while the
    // second half is still arriving
    constexpr int KS = BK / 32;
    bf16x8 a[KS][FN], b[KS][FM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int piece = ks * 4 + frag_grp;
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[ks][i] = *reinterpret_cast<const bf16x8 *>(
            cur + lds_piece_offset(wn * TN + i * 16 + frag_row, piece));
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[ks][j] = *reinterpret_cast<const bf16x8 *>(
            cur + lds_piece_offset(BN + wm * TM + j * 16 + frag_row, piece));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
    // keep that order through scheduling: all LDS reads, then the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, KS * (FN + FM), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KS * FN * FM, 0);
    if (kt + 1 < nk) store_step(lds[(kt + 1) & 1], (kt + 1) * BK);
    __syncthreads();
  }

  // acc[i][j][r] = Z^T[n = 4*(lane/16) + r][m = lane%16] of fragment (i, j).
  // 8-byte stores need every row start at a multiple of 4 elements from an
  // 8-byte-aligned base (column offsets inside a tile are multiples of 4).
  const bool pack_ok =
      ((ld | col_off) & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
  const int64_t nb = n0 + wn * TN + 4 * frag_grp;
  const int64_t mb = m0 + wm * TM + frag_row;
  if (pack_ok && n0 + BN <= N && m0 + BM <= M) {
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

// ---------------------------------------------------------------------------
// fp32: 64 x 64 output tile per workgroup, 4 x 4 outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void lmhead_f32_tiled(const float *__restrict__ X, int64_t M,
                                                          int64_t K, const float *__restrict__ W,
                                                          int64_t N, float *__restrict__ out,
                                                          int64_t ld, int64_t col_off) {
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
      sX[kk][r] = (m0 + r < M && k < K) ? X[(m0 + r) * K + k] : 0.f;
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

template <int BN, int BM, int WN, int WM>
int launch_bf16_cfg(const uint16_t *x, int64_t m, int64_t k, const uint16_t *w, int64_t n,
                    uint16_t *out, int64_t ld, int64_t col_off, hipStream_t st) {
  const int64_t tn64 = (n + BN - 1) / BN, tm64 = (m + BM - 1) / BM;
  if (tn64 * tm64 > INT32_MAX) return static_cast<int>(hipErrorInvalidValue);
  const int tiles_n = static_cast<int>(tn64);
  const int tiles_m = static_cast<int>(tm64);
  const dim3 grid(static_cast<unsigned>(tiles_n) * static_cast<unsigned>(tiles_m));
  const bool vec = (k % 8 == 0) && ((reinterpret_cast<uint64_t>(x) | reinterpret_cast<uint64_t>(w)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((lmhead_bf16_mfma<BN, BM, WN, WM, true>), grid, dim3(kBlock), 0, st, x, m,
                       k, w, n, out, ld, col_off, tiles_n, tiles_m);
  else
    hipLaunchKernelGGL((lmhead_bf16_mfma<BN, BM, WN, WM, false>), grid, dim3(kBlock), 0, st, x,
                       m, k, w, n, out, ld, col_off, tiles_n, tiles_m);
  return 0;
}

}  // namespace

int launch_lmhead(const void *x, int64_t m, int64_t k, const void *w, int64_t n, int dtype,
                  void *logits, int64_t ld, int64_t col_offset, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status below is this launch's
  if (dtype == 0) {
    const dim3 grid(static_cast<unsigned>((n + 63) / 64), static_cast<unsigned>((m + 63) / 64));
    hipLaunchKernelGGL(lmhead_f32_tiled, grid, dim3(kBlock), 0, st, static_cast<const float *>(x),
                       m, k, static_cast<const float *>(w), n, static_cast<float *>(logits), ld,
                       col_offset);
    return static_cast<int>(hipGetLastError());
  }
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  const uint16_t *wb = static_cast<const uint16_t *>(w);
  uint16_t *ob = static_cast<uint16_t *>(logits);
  int rc;
  if (m <= 16)
    rc = launch_bf16_cfg<256, 16, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 32)
    rc = launch_bf16_cfg<256, 32, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 64)
    rc = launch_bf16_cfg<256, 64, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 128)
    rc = launch_bf16_cfg<256, 128, 2, 2>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 256)
    rc = launch_bf16_cfg<128, 256, 2, 2>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else
    rc = launch_bf16_cfg<256, 256, 2, 2>(xb, m, k, wb, n, ob, ld, col_offset, st);
  if (rc != 0) return rc;
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpe
