// Tiled fp8 (OCP E4M3) layouts of the low-precision attention path, in the
// operand order of the 32x32x64 f8 MFMA (each lane holds 32 bytes of its row
// or column: two 16-byte halves h, stored 1 KB apart so that a wave reads a
// half as one contiguous 1 KB block).
//
// The MFMA pairs byte e of lane (i + 32g) of A with byte e of lane (j + 32g)
// of B, for both lane halves g: any assignment of contraction indices to
// (g, e) works as long as both operands use the same one.
#pragma once

#include "device_common.h"

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

// The tile's scale exponent: the least e with amax * 2^-e <= 448 (the
// largest E4M3 value), clamped to >= -127 so that e + 127 fits the scale
// byte; 0 for an all-zero tile. amax = m * 2^E with 0.5 <= m < 1, and
// 448 = 0.875 * 2^9.
__device__ inline int fp8_tile_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = frexpf(amax, &E);
  const int e = m <= 0.875f ? E - 9 : E - 8;
  return e < -kFp8ExpBias ? -kFp8ExpBias : e;
}

__device__ inline uint32_t fp8_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);     // bytes 0, 1 (RNE)
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);          // bytes 2, 3
  return (uint32_t)w;
}

// Writes one tile, held in LDS as plain bf16 rows (slot-major, row stride
// LD), in the fp8 layout of Q/K (col = false) or V (col = true), scaled by
// 2^-e: 16-byte chunk ch is block ch/128, half (ch/64)%2, lane ch%64. The
// nthreads threads of the workgroup share the chunks.
template <int D, int LD>
__device__ inline void fp8_write_tile(const bf16_bits *xs, bool col, int e, uint8_t *dst,
                                      int nthreads) {
  for (int ch = threadIdx.x; ch < kTile * D / 16; ch += nthreads) {
    const int blk = ch / 128, half = (ch / 64) % 2, lane = ch % 64, g = lane / 32;
    float x[16];
    if (col) {
      const int c = blk * 32 + lane % 32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = half * 32 + 8 * (j / 4) + 4 * g + j % 4;
        x[j] = bf16_to_float(xs[key * LD + c]);
      }
    } else {
      const int slot = (blk / (D / 64)) * 32 + lane % 32;
      const int c0 = (blk % (D / 64)) * 64 + 32 * g + 16 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = bf16_to_float(xs[slot * LD + c0 + j]);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = ldexpf(x[j], -e);    // exact: a power of two
    uint4 o;
    o.x = fp8_pack4(x[0], x[1], x[2], x[3]);
    o.y = fp8_pack4(x[4], x[5], x[6], x[7]);
    o.z = fp8_pack4(x[8], x[9], x[10], x[11]);
    o.w = fp8_pack4(x[12], x[13], x[14], x[15]);
    *reinterpret_cast<uint4 *>(dst + ch * 16) = o;
  }
}

// Largest |x| of a workgroup's per-thread partial maxima (red: one float per
// wave in LDS; ends with a barrier, so every thread gets the result).
__device__ inline float block_amax(float amax, float *red, int nthreads) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = amax;
  __syncthreads();
  amax = red[0];
  for (int w = 1; w < nthreads / 64; ++w) amax = fmaxf(amax, red[w]);
  return amax;
}

}  // namespace vsa
