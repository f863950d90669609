// Tiled fp8 (OCP E4M3) layouts of the low-precision attention path, in the
// operand order of the 32x32x64 f8 MFMA (each lane holds 32 bytes of its row
// or column: two 16-byte halves h, stored 1 KB apart so that a wave reads a
// half as one contiguous 1 KB block).
//
// The MFMA pairs byte e of lane (i + 32g) of A with byte e of lane (j + 32g)
// of B, for both lane halves g: any assignment of contraction indices to
// (g, e) works as long as both operands use the same one.
#pragma once

#include <stdint.h>

namespace vsa {

// Q and K: 2 KB blocks of 32 slots x 64 channels, block
// (s/32)*(D/64) + c/64. Lane s%32 + 32g holds channels 64*(c/64) + 32g + e,
// e = 0..31, byte e in half e/16.
__host__ __device__ inline int fp8_row_offset(int s, int c, int D) {
  const int blk = (s / 32) * (D / 64) + c / 64, w = c % 64;
  const int g = w / 32, e = w % 32;
  return blk * 2048 + (e / 16) * 1024 + (s % 32 + 32 * g) * 16 + e % 16;
}

// V: 2 KB blocks of 64 keys x 32 channels, block c/32. Lane c%32 + 32g holds
// the 32 keys that lane half g of the S^T = K Q^T accumulator holds for a
// query (key (e/16)*32 + 8*((e%16)/4) + 4g + e%4 at byte e), so the
// probabilities, packed to fp8 in accumulator order, are the B operand of
// O^T = V^T P^T as they stand.
__host__ __device__ inline int fp8_col_offset(int s, int c, int D) {
  (void)D;
  const int kb = s / 32, w = s % 32;
  const int g = (w / 4) % 2, r = (w / 8) * 4 + w % 4;
  return (c / 32) * 2048 + kb * 1024 + (c % 32 + 32 * g) * 16 + r;
}

// Per (batch*head, tile) scale word: byte 0 = Q's, 1 = K's, 2 = V's biased
// exponent e + 127 (the tile's values are code * 2^e); byte 3 unused.
constexpr int kFp8ExpBias = 127;

}  // namespace vsa
