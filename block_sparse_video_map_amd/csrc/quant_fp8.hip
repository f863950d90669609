// fp8 inputs of the low-precision attention path: every bf16 Q, K and V tile
// of a head is scaled by a power of two 2^-e (the least e that brings the
// tile's largest |x| to at most 448, the largest E4M3 value; e = 0 for an
// all-zero tile, e >= -127 so that e + 127 fits the scale byte), rounded to
// OCP E4M3 (nearest, ties to even) and written in the fp8 operand layouts.
// The node runs its attention as a quantized kernel ("Veda Sparse Attention
// в ComfyUI", section "Узел ComfyUI"); E4M3 is the MI355X matrix core's
// 8-bit format.
//
// One workgroup per (tile, batch*head, tensor): the tile is unpacked into
// LDS in plain slot-major order while its largest |x| is reduced, then every
// thread packs 16-byte chunks of the output layout from LDS. The gather can
// do the same in its own pass (launch_gather with fp8 outputs); this kernel
// serves tiles that are already gathered.
#include "device_common.h"
#include "fp8_layout.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kQThreads = 256;

template <int D>
__global__ __launch_bounds__(kQThreads) void quant_fp8_kernel(
    Plan p, const bf16_bits *__restrict__ qt, const bf16_bits *__restrict__ kt,
    const bf16_bits *__restrict__ vt, uint8_t *__restrict__ q8, uint8_t *__restrict__ k8,
    uint8_t *__restrict__ v8, uint8_t *__restrict__ exps) {
  constexpr int LD = D + 8;                    // bf16 row stride in LDS
  __shared__ bf16_bits xs[kTile * LD];
  __shared__ float wmax[kQThreads / 64];
  const int tile = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int h = bh % p.H, s = h % p.n_shapes;
  if (tile >= p.n_tiles[s]) return;
  const int64_t off = ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
  const bf16_bits *src = (which == 0 ? qt : which == 1 ? kt : vt) + off;
  uint8_t *dst = (which == 0 ? q8 : which == 1 ? k8 : v8) + off;

  float amax = 0.f;
  for (int vec = threadIdx.x; vec < kTile * D / 8; vec += kQThreads) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(src + vec * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const bf16_bits u = (bf16_bits)(w[e8 / 2] >> (16 * (e8 % 2)));
      int sl, c;
      if (which == 2)
        col_layout_decode(vec, e8, D, sl, c);
      else
        row_layout_decode(vec, e8, D, sl, c);
      xs[sl * LD + c] = u;
      amax = fmaxf(amax, fabsf(bf16_to_float(u)));
    }
  }
  const int e = fp8_tile_exponent(block_amax(amax, wmax, kQThreads));
  fp8_write_tile<D, LD>(xs, which == 2, e, dst, kQThreads);
  if (threadIdx.x == 0)
    exps[((int64_t)bh * p.max_tiles + tile) * 4 + which] = (uint8_t)(e + kFp8ExpBias);
}

}  // namespace
}  // namespace vsa

hipError_t launch_quant_fp8(const Plan &p, const void *qt, const void *kt, const void *vt,
                            uint8_t *q8, uint8_t *k8, uint8_t *v8, uint8_t *exps,
                            hipStream_t stream) {
  dim3 grid(p.max_tiles, p.B * p.H, 3);
  const bf16_bits *q = (const bf16_bits *)qt, *k = (const bf16_bits *)kt,
                  *v = (const bf16_bits *)vt;
  if (p.d == 128)
    hipLaunchKernelGGL(vsa::quant_fp8_kernel<128>, grid, dim3(vsa::kQThreads), 0, stream, p, q,
                       k, v, q8, k8, v8, exps);
  else
    hipLaunchKernelGGL(vsa::quant_fp8_kernel<64>, grid, dim3(vsa::kQThreads), 0, stream, p, q,
                       k, v, q8, k8, v8, exps);
  return hipGetLastError();
}
