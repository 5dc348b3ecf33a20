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

// Copy a rows x BK slice (rows [r0, r0+ROWS) of a [nrows, K] matrix, columns
// [k0, k0+BK)) into LDS.  Out-of-range rows and columns are filled with zero.
// VEC: rows are 16-byte aligned and K % 8 == 0, so each piece is one load.
template <int ROWS, bool VEC>
__device__ __forceinline__ void stage_tile(uint16_t *__restrict__ lds,
                                           const uint16_t *__restrict__ g, int64_t r0,
                                           int64_t nrows, int64_t K, int64_t k0) {
  constexpr int kTotal = ROWS * kPieces;
#pragma unroll
  for (int c = threadIdx.x; c < kTotal; c += kBlock) {
    const int row = c / kPieces;
    const int piece = c % kPieces;
    const int64_t grow = r0 + row;
    const int64_t gk = k0 + piece * 8;
    u32x4 v = u32x4(0);
    if (grow < nrows) {
      const uint16_t *p = g + grow * K + gk;
      if (VEC) {
        if (gk < K) v = *reinterpret_cast<const u32x4 *>(p);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = (gk + q < K) ? p[q] : uint16_t(0);
        v = u32x4{e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                  e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16)};
      }
    }
    *reinterpret_cast<u32x4 *>(lds + lds_piece_offset(row, piece)) = v;
  }
}

// BN x BM tile of Z^T per workgroup; waves arranged WN x WM; each wave owns
// (BN/WN) x (BM/WM) = FN x FM fragments of 16 x 16.
template <int BN, int BM, int WN, int WM, bool VEC>
__global__ __launch_bounds__(kBlock) void lmhead_bf16_mfma(
    const uint16_t *__restrict__ X, int64_t M, int64_t K, const uint16_t *__restrict__ W,
    int64_t N, uint16_t *__restrict__ out, int64_t ld, int64_t col_off) {
  static_assert(WN * WM == kBlock / 64, "4 waves per workgroup");
  constexpr int TN = BN / WN, TM = BM / WM;
  constexpr int FN = TN / 16, FM = TM / 16;
  static_assert(FN * 16 == TN && FM * 16 == TM, "wave tile must be a multiple of 16");

  __shared__ __attribute__((aligned(16))) uint16_t sW[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[BM * BK];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;

  f32x4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x4(0.f);

  const int frag_row = lane & 15;   // row of the fragment this lane feeds
  const int frag_grp = lane >> 4;   // which 8-wide k group of a 32-wide step

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    stage_tile<BN, VEC>(sW, W, n0, N, K, k0);
    stage_tile<BM, VEC>(sX, X, m0, M, K, k0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int piece = ks * 4 + frag_grp;
      bf16x8 a[FN], b[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(
            sW + lds_piece_offset(wn * TN + i * 16 + frag_row, piece));
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(
            sX + lds_piece_offset(wm * TM + j * 16 + frag_row, piece));
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // acc[i][j][r] = Z^T[n = 4*(lane/16) + r][m = lane%16] of fragment (i, j)
  // 8-byte stores need every row start at a multiple of 4 elements from an
  // 8-byte-aligned base (column offsets inside a tile are multiples of 4)
  const bool pack_ok =
      ((ld | col_off) & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int64_t n = n0 + wn * TN + i * 16 + 4 * frag_grp;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t m = m0 + wm * TM + j * 16 + frag_row;
      if (m >= M) continue;
      uint16_t *dst = out + m * ld + col_off + n;
      if (pack_ok && n + 3 < N) {
        const u32x2 v{f32_to_bf16_bits(acc[i][j][0]) | (f32_to_bf16_bits(acc[i][j][1]) << 16),
                      f32_to_bf16_bits(acc[i][j][2]) | (f32_to_bf16_bits(acc[i][j][3]) << 16)};
        *reinterpret_cast<u32x2 *>(dst) = v;
      } else {
#pragma unroll
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
void launch_bf16_cfg(const uint16_t *x, int64_t m, int64_t k, const uint16_t *w, int64_t n,
                     uint16_t *out, int64_t ld, int64_t col_off, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((n + BN - 1) / BN), static_cast<unsigned>((m + BM - 1) / BM));
  const bool vec = (k % 8 == 0) && ((reinterpret_cast<uint64_t>(x) | reinterpret_cast<uint64_t>(w)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((lmhead_bf16_mfma<BN, BM, WN, WM, true>), grid, dim3(kBlock), 0, st, x, m,
                       k, w, n, out, ld, col_off);
  else
    hipLaunchKernelGGL((lmhead_bf16_mfma<BN, BM, WN, WM, false>), grid, dim3(kBlock), 0, st, x,
                       m, k, w, n, out, ld, col_off);
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
  if (m <= 16)
    launch_bf16_cfg<128, 16, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 32)
    launch_bf16_cfg<128, 32, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else if (m <= 64)
    launch_bf16_cfg<128, 64, 4, 1>(xb, m, k, wb, n, ob, ld, col_offset, st);
  else
    launch_bf16_cfg<128, 128, 2, 2>(xb, m, k, wb, n, ob, ld, col_offset, st);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpe
