// Range rules of the LM-head kernels' buffer loads, shared by the kernel
// launchers and the host tests (plain C++, no HIP headers).
//
// The bf16 LM-head kernels read W and X through raw buffer descriptors.  A
// descriptor covers `bytes` bytes from its base; a load whose offset lies at
// or past that range returns zeros.  Loads that must read zeros (rows past M
// or N, pieces past K, a sequence end outside the packed tokens) are issued
// at the byte offset kLoadMask, so every descriptor must cover at most
// kLoadMask bytes: a larger range would put the masked offset inside it, and
// the load would return real data (or read past the buffer) instead of zeros.
#ifndef VPE_BOUNDS_H
#define VPE_BOUNDS_H

#include <stdint.h>

namespace vpe {

// Byte offset of a masked load; the largest range a descriptor may cover.
constexpr int kLoadMask = 0x7FFF0000;

// True when `rows` rows of `k` bf16 elements fit one descriptor, so that a
// masked load at kLoadMask reads zeros.
constexpr bool bf16_rows_fit_descriptor(int64_t rows, int64_t k) {
  return rows >= 0 && k >= 0 && (k == 0 || (k <= kLoadMask / 2 && rows <= kLoadMask / (2 * k)));
}

// The bf16 LM-head kernels take 16-byte buffer loads (straight to LDS, or to
// registers) when K is a multiple of 8 elements, both bases are 16-byte
// aligned and every descriptor they build fits the rule above: the W tile's
// rows (w_tile_rows), and X either the tile's rows (x_tile_rows) or, for X
// rows gathered out of packed prefill activations, all n_tokens rows.
// Otherwise they stage operands through registers with element-wise loads.
constexpr bool bf16_direct_loads_ok(uint64_t x_addr, uint64_t w_addr, int64_t k, bool gathered,
                                    int64_t n_tokens, int64_t x_tile_rows,
                                    int64_t w_tile_rows) {
  return k % 8 == 0 && ((x_addr | w_addr) & 15) == 0 &&
         bf16_rows_fit_descriptor(gathered ? n_tokens : x_tile_rows, k) &&
         bf16_rows_fit_descriptor(w_tile_rows, k);
}

}  // namespace vpe

#endif
