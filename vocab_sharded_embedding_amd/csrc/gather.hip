// Row-gather kernels for gfx950: the shard's masked embedding lookup, the
// prefill last-position select, and the on-device sum of embedding partials.
//
// All three are HBM-bound copies.  The design keeps every byte moved once:
//  - rows are moved in 16-byte vectors (the widest global load/store), one
//    64-lane wavefront per row (several rows per wave for short rows), with
//    lanes of a wave covering consecutive 16-byte pieces of a row so that a
//    wave's access is one contiguous span;
//  - the row index is computed once per wave from a scalar load of the id:
//    the mask and shift of the lookup never touch vector registers;
//  - rows the shard does not own are written as zero vectors and the table is
//    not read for them (the page formula would look up a placeholder row and
//    multiply it by zero);
//  - outputs are written with non-temporal stores: they are not re-read here.
//
// Sources: devpress.csdn.net/amd/6a3de260... section 3 (the masked lookup in
// five steps; steps 1-4 happen here, step 5 is the partial sum below) and
// section 6 (the sum of partials done in one process); blog.xiaohansong.com
// "从零实现 vLLM (1.1)" walkthrough steps 1-4; caomaolufei.github.io
// AIInfraGuide 3.3 section 6 (ParallelLMHead's last-position select).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vpe_launch.h"

namespace vpe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;          // 4 wavefronts of 64 lanes
constexpr int kWavesPerBlock = kBlock / 64;

// ---------------------------------------------------------------------------
// row index policies: map an output row to a source row, or -1 for "zeros"
// ---------------------------------------------------------------------------
// `advanced(r)` is the same policy for output rows starting at row r (the
// launcher splits very long gathers into several grids).
template <typename IdT>
struct ShardIndex {
  const IdT *ids;
  int64_t start;
  int64_t rows;
  // owned iff start <= id < start + rows; one unsigned compare covers both
  // ends.  The shift is done modulo 2^64 (no signed overflow for any id); with
  // 0 <= start <= INT64_MAX - rows (checked on the host) a wrapped difference
  // is never below rows.
  __device__ __forceinline__ int64_t operator()(int64_t i) const {
    const uint64_t local =
        static_cast<uint64_t>(static_cast<int64_t>(ids[i])) - static_cast<uint64_t>(start);
    return local < static_cast<uint64_t>(rows) ? static_cast<int64_t>(local) : -1;
  }
  ShardIndex advanced(int64_t r) const { return ShardIndex{ids + r, start, rows}; }
};

struct LastTokenIndex {
  const int32_t *cu;
  int64_t n_tokens;
  __device__ __forceinline__ int64_t operator()(int64_t s) const {
    const int64_t last = static_cast<int64_t>(cu[s + 1]) - 1;
    return (static_cast<uint64_t>(last) < static_cast<uint64_t>(n_tokens)) ? last : -1;
  }
  LastTokenIndex advanced(int64_t r) const { return LastTokenIndex{cu + r, n_tokens}; }
};

template <typename V>
__device__ __forceinline__ V zero_vec() {
  return V(0);
}

// ---------------------------------------------------------------------------
// Long rows (more than 64 vectors): one wave per row, RPW rows per wave, VPL
// vectors per lane per row in flight before any store is issued.
// ---------------------------------------------------------------------------
template <typename V, int VPL, int RPW, class Index>
__global__ __launch_bounds__(kBlock) void gather_rows_wide(Index index, int64_t n_rows,
                                                          const V *__restrict__ src,
                                                          V *__restrict__ dst, int64_t vr) {
  const int lane = threadIdx.x & 63;
  // wave-uniform row number, so the id load and the mask are scalar work
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t row0 = wave * RPW;
  if (row0 >= n_rows) return;

  int64_t srow[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) srow[r] = (row0 + r < n_rows) ? index(row0 + r) : -2;

  for (int64_t c0 = 0; c0 < vr; c0 += VPL * 64) {
    V v[RPW][VPL];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int64_t col = c0 + c * 64 + lane;
        v[r][c] = zero_vec<V>();
        if (srow[r] >= 0 && col < vr) v[r][c] = src[srow[r] * vr + col];
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const int64_t col = c0 + c * 64 + lane;
        if (srow[r] != -2 && col < vr)
          __builtin_nontemporal_store(v[r][c], &dst[(row0 + r) * vr + col]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Short rows (at most 64 vectors): a group of 2^LOG2G lanes per row.
// ---------------------------------------------------------------------------
template <typename V, int LOG2G, class Index>
__global__ __launch_bounds__(kBlock) void gather_rows_narrow(Index index, int64_t n_rows,
                                                            const V *__restrict__ src,
                                                            V *__restrict__ dst, int64_t vr) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t row = t >> LOG2G;
  const int64_t col = t & ((1 << LOG2G) - 1);
  if (row >= n_rows || col >= vr) return;
  const int64_t s = index(row);
  V v = zero_vec<V>();
  if (s >= 0) v = src[s * vr + col];
  dst[row * vr + col] = v;
}

int ceil_log2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

template <typename V, class Index>
void launch_gather_chunk(Index index, int64_t n_rows, const V *s, V *d, int64_t vr,
                         hipStream_t stream) {
  if (vr <= 64) {
    const int lg = ceil_log2(vr);
    const int64_t threads = n_rows << lg;
    const dim3 grid(static_cast<unsigned>((threads + kBlock - 1) / kBlock));
    switch (lg) {
#define VPE_NARROW(L) \
  case L: hipLaunchKernelGGL((gather_rows_narrow<V, L, Index>), grid, dim3(kBlock), 0, stream, index, n_rows, s, d, vr); break;
      VPE_NARROW(0) VPE_NARROW(1) VPE_NARROW(2) VPE_NARROW(3) VPE_NARROW(4) VPE_NARROW(5)
      VPE_NARROW(6)
#undef VPE_NARROW
      default: break;  // unreachable: vr <= 64
    }
  } else {
    const int64_t vpl = (vr + 63) / 64;  // vectors per lane to cover one row
#define VPE_WIDE(VPL, RPW)                                                                   \
  do {                                                                                       \
    const int64_t waves = (n_rows + (RPW)-1) / (RPW);                                        \
    const dim3 grid(static_cast<unsigned>((waves + kWavesPerBlock - 1) / kWavesPerBlock));   \
    hipLaunchKernelGGL((gather_rows_wide<V, VPL, RPW, Index>), grid, dim3(kBlock), 0, stream, \
                       index, n_rows, s, d, vr);                                             \
  } while (0)
    // Several rows per wave put more bytes in flight per wave, but only pay
    // when the grid still has enough waves to fill the chip (8 per SIMD over
    // 256 CUs); short gathers take one row per wave.  For 8 KB rows, 4 rows
    // per wave measured 8% faster than 1 on 131072 ids with a quarter owned
    // (and 13% faster with none owned, where the wave only stores zeros):
    // a wave's id loads are paid once for 32 KB of stores.
    const bool many = n_rows >= int64_t(4) * 8 * 4 * 256;
    if (vpl <= 2 && many) VPE_WIDE(2, 4);
    else if (vpl <= 2) VPE_WIDE(2, 1);
    else if (vpl <= 4 && many) VPE_WIDE(4, 2);
    else if (vpl <= 4) VPE_WIDE(4, 1);
    else if (many) VPE_WIDE(8, 4);
    else VPE_WIDE(8, 1);
#undef VPE_WIDE
  }
}

// Rows per grid: keeps every grid well inside the 32-bit work-item range.
constexpr int64_t kRowsPerLaunch = int64_t(1) << 24;

template <typename V, class Index>
int launch_gather_v(Index index, int64_t n_rows, const void *src, void *dst, int64_t vr,
                    hipStream_t stream) {
  const V *s = static_cast<const V *>(src);
  V *d = static_cast<V *>(dst);
  for (int64_t r0 = 0; r0 < n_rows; r0 += kRowsPerLaunch) {
    const int64_t rows = (n_rows - r0 < kRowsPerLaunch) ? (n_rows - r0) : kRowsPerLaunch;
    launch_gather_chunk<V>(index.advanced(r0), rows, s, d + r0 * vr, vr, stream);
  }
  return static_cast<int>(hipGetLastError());
}

// Widest vector (16, 8, 4 or 2 bytes) that divides the row and both bases.
int pick_vec_bytes(int64_t row_bytes, const void *a, const void *b) {
  const uint64_t al = reinterpret_cast<uint64_t>(a) | reinterpret_cast<uint64_t>(b) |
                      static_cast<uint64_t>(row_bytes);
  if ((al & 15) == 0) return 16;
  if ((al & 7) == 0) return 8;
  if ((al & 3) == 0) return 4;
  return 2;
}

template <class Index>
int launch_gather(Index index, int64_t n_rows, const void *src, void *dst, int64_t row_bytes,
                  void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status returned is this launch's
  switch (pick_vec_bytes(row_bytes, src, dst)) {
    case 16: return launch_gather_v<u32x4>(index, n_rows, src, dst, row_bytes / 16, st);
    case 8: return launch_gather_v<u32x2>(index, n_rows, src, dst, row_bytes / 8, st);
    case 4: return launch_gather_v<uint32_t>(index, n_rows, src, dst, row_bytes / 4, st);
    default: return launch_gather_v<uint16_t>(index, n_rows, src, dst, row_bytes / 2, st);
  }
}

// ---------------------------------------------------------------------------
// Sum of partials.  fp32 adds in rank order starting from partial 0 (so a
// one-partial sum is the identity, -0.0 included), one rounding for bf16.
// ---------------------------------------------------------------------------
struct PartList {
  const void *p[64];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> bf16 bits, round to nearest, ties to even; NaN becomes a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rounded;
}

// EPV elements per thread: 4 (fp32, 16 B), 8 (bf16, 16 B) or 1 (tail / unaligned)
template <bool BF16, int EPV>
__global__ __launch_bounds__(kBlock) void sum_partials_kernel(PartList parts, int n_parts,
                                                             int64_t e0, int64_t n_elems,
                                                             void *out) {
  const int64_t i = e0 + (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * EPV;
  if (i >= n_elems) return;
  if constexpr (!BF16) {
    if constexpr (EPV == 4) {
      float4 acc = *reinterpret_cast<const float4 *>(static_cast<const float *>(parts.p[0]) + i);
      for (int r = 1; r < n_parts; ++r) {
        const float4 v = *reinterpret_cast<const float4 *>(static_cast<const float *>(parts.p[r]) + i);
        acc.x = acc.x + v.x; acc.y = acc.y + v.y; acc.z = acc.z + v.z; acc.w = acc.w + v.w;
      }
      __builtin_nontemporal_store(acc.x, static_cast<float *>(out) + i);
      __builtin_nontemporal_store(acc.y, static_cast<float *>(out) + i + 1);
      __builtin_nontemporal_store(acc.z, static_cast<float *>(out) + i + 2);
      __builtin_nontemporal_store(acc.w, static_cast<float *>(out) + i + 3);
    } else {
      float acc = static_cast<const float *>(parts.p[0])[i];
      for (int r = 1; r < n_parts; ++r) acc = acc + static_cast<const float *>(parts.p[r])[i];
      static_cast<float *>(out)[i] = acc;
    }
  } else {
    if constexpr (EPV == 8) {
      u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(parts.p[0]) + i);
      float acc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
        acc[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
      }
      for (int r = 1; r < n_parts; ++r) {
        w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(parts.p[r]) + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = acc[2 * e] + bf16_bits_to_f32(w[e] & 0xffffu);
          acc[2 * e + 1] = acc[2 * e + 1] + bf16_bits_to_f32(w[e] >> 16);
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = f32_to_bf16_bits(acc[2 * e]) | (f32_to_bf16_bits(acc[2 * e + 1]) << 16);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(out) + i));
    } else {
      float acc = bf16_bits_to_f32(static_cast<const uint16_t *>(parts.p[0])[i]);
      for (int r = 1; r < n_parts; ++r)
        acc = acc + bf16_bits_to_f32(static_cast<const uint16_t *>(parts.p[r])[i]);
      static_cast<uint16_t *>(out)[i] = static_cast<uint16_t>(f32_to_bf16_bits(acc));
    }
  }
}

template <bool BF16, int EPV>
void launch_sum_range(const PartList &pl, int n_parts, int64_t e0, int64_t e1, void *out,
                      hipStream_t st) {
  const int64_t threads = (e1 - e0 + EPV - 1) / EPV;
  if (threads <= 0) return;
  const dim3 grid(static_cast<unsigned>((threads + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((sum_partials_kernel<BF16, EPV>), grid, dim3(kBlock), 0, st, pl, n_parts,
                     e0, e1, out);
}

// Contiguous copy (a rank's rows of the full table are one contiguous block).
// 16-byte vectors, two in flight per thread, grid-stride over the vectors;
// the tail (and any copy whose ends are not 16-byte aligned) goes bytewise.
// Measured on MI355X for a 311 MB copy: two vectors per thread over 8192
// blocks reach 5.9 TB/s; four per thread over 4096 blocks 4.8 TB/s.
__global__ __launch_bounds__(kBlock) void copy_vec_kernel(const u32x4 *__restrict__ src,
                                                          u32x4 *__restrict__ dst, int64_t n_vec) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  for (; i + stride < n_vec; i += 2 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
  }
  if (i < n_vec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kBlock) void copy_bytes_kernel(const uint8_t *__restrict__ src,
                                                            uint8_t *__restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

int launch_copy_bytes(const void *src, void *dst, int64_t n_bytes, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status returned is this launch's
  const uint8_t *s8 = static_cast<const uint8_t *>(src);
  uint8_t *d8 = static_cast<uint8_t *>(dst);
  const bool aligned16 =
      ((reinterpret_cast<uint64_t>(src) | reinterpret_cast<uint64_t>(dst)) & 15) == 0;
  const int64_t n_vec = aligned16 ? n_bytes / 16 : 0;
  constexpr int64_t kMaxBlocks = 8192;  // 32 per CU; the loops stride over the rest
  if (n_vec > 0) {
    const int64_t blocks = std::min<int64_t>((n_vec + 2 * kBlock - 1) / (2 * kBlock), kMaxBlocks);
    hipLaunchKernelGGL(copy_vec_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, st,
                       reinterpret_cast<const u32x4 *>(s8), reinterpret_cast<u32x4 *>(d8), n_vec);
  }
  const int64_t rest = n_bytes - n_vec * 16;
  if (rest > 0) {
    const int64_t blocks = std::min<int64_t>((rest + kBlock - 1) / kBlock, kMaxBlocks);
    hipLaunchKernelGGL(copy_bytes_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, st,
                       s8 + n_vec * 16, d8 + n_vec * 16, rest);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_embed(const void *ids, int itype, int64_t n, const void *weight, int64_t shard_rows,
                 int64_t row_bytes, int64_t vocab_start, void *out, void *stream) {
  if (itype == 0) {
    ShardIndex<int32_t> idx{static_cast<const int32_t *>(ids), vocab_start, shard_rows};
    return launch_gather(idx, n, weight, out, row_bytes, stream);
  }
  ShardIndex<int64_t> idx{static_cast<const int64_t *>(ids), vocab_start, shard_rows};
  return launch_gather(idx, n, weight, out, row_bytes, stream);
}

int launch_last_token_select(const void *hidden, int64_t n_tokens, int64_t row_bytes,
                             const int32_t *cu_seqlens, int64_t n_seqs, void *out,
                             void *stream) {
  LastTokenIndex idx{cu_seqlens, n_tokens};
  return launch_gather(idx, n_seqs, hidden, out, row_bytes, stream);
}

int launch_sum_partials(const void *const *parts, int n_parts, int64_t n_elems, int dtype,
                        void *out, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the status returned is this launch's
  PartList pl{};
  uint64_t al = reinterpret_cast<uint64_t>(out);
  for (int r = 0; r < n_parts; ++r) {
    pl.p[r] = parts[r];
    al |= reinterpret_cast<uint64_t>(parts[r]);
  }
  const bool aligned16 = (al & 15) == 0;
  const int epv = dtype == 1 ? 8 : 4;
  const int64_t n_vec = aligned16 ? (n_elems / epv) * epv : 0;  // elements done 16 B at a time
  if (dtype == 1) {
    if (n_vec) launch_sum_range<true, 8>(pl, n_parts, 0, n_vec, out, st);
    launch_sum_range<true, 1>(pl, n_parts, n_vec, n_elems, out, st);
  } else {
    if (n_vec) launch_sum_range<false, 4>(pl, n_parts, 0, n_vec, out, st);
    launch_sum_range<false, 1>(pl, n_parts, n_vec, n_elems, out, st);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace vpe
