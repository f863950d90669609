// Step 1: the tile map and the 3D-to-tile gather of Q, K and V.
//
// One workgroup per (tile, batch*head, tensor). The tile's 64 rows are read
// once with 16-byte coalesced loads into LDS (pads become zero rows), then
// written out in the tiled operand layout as contiguous 16-byte vectors, so
// both the HBM reads and the HBM writes are full-width. For the fp8 path the
// same pass also writes the tile's E4M3 copy and scale byte from LDS (the
// quantizer's rule), so the bf16 tiles are not read back. With `means` the
// pass also writes, for the video tiles of Q and K, each channel's mean over
// the tile's real rows (pads are zero rows in LDS and are not counted), in
// double and in the summation order of the mean-gate pooling kernel, so the
// pooling need not read the tiles again.
#include "device_common.h"
#include "fp8_layout.h"
#include "kernels.h"

namespace vsa {
namespace {

__global__ void build_map_kernel(Plan p, int32_t *s2t) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)p.n_shapes * p.max_tiles * kTile;
  if (i >= total) return;
  int slot = (int)(i % kTile);
  int tile = (int)((i / kTile) % p.max_tiles);
  int s = (int)(i / ((int64_t)kTile * p.max_tiles));
  s2t[i] = slot_token(p, s, tile, slot);
}

// T: element type (bf16 bits or float); D: head dim.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(Plan p, const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const int32_t *__restrict__ s2t,
                                                     T *__restrict__ qt, T *__restrict__ kt,
                                                     T *__restrict__ vt, uint8_t *q8,
                                                     uint8_t *k8, uint8_t *v8,
                                                     uint8_t *scales, double *means) {
  constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int CPR = D / EPC;           // chunks per row
  constexpr int LD = D + EPC;            // padded LDS row (keeps 16 B alignment)
  __shared__ __attribute__((aligned(16))) T tile_lds[kTile * LD];
  __shared__ float red[4];
  __shared__ int n_real;

  const int tile = blockIdx.x;
  const int bh = blockIdx.y;
  const int which = blockIdx.z;          // 0: Q, 1: K, 2: V
  const int h = bh % p.H;
  const int s = h % p.n_shapes;
  if (tile >= p.n_tiles[s]) return;
  const T *src = which == 0 ? q : which == 1 ? k : v;
  T *dst = which == 0 ? qt : which == 1 ? kt : vt;
  if (!src) return;

  const bool fp8 = sizeof(T) == 2 && q8 != nullptr;      // uniform over the launch
  const int32_t *map = s2t + ((int64_t)s * p.max_tiles + tile) * kTile;
  const bool take_mean = means != nullptr && which < 2 && tile >= p.n_prefix_tiles;
  if (take_mean && threadIdx.x < kTile) {
    const uint64_t real = __ballot(map[threadIdx.x] >= 0);
    if (threadIdx.x == 0) n_real = __popcll(real);
  }
  const T *src_bh = src + (int64_t)bh * p.N * D;
  float amax = 0.f;
  for (int i = threadIdx.x; i < kTile * CPR; i += blockDim.x) {
    int row = i / CPR, cc = i % CPR;
    int32_t tok = map[row];
    uint4 val = make_uint4(0, 0, 0, 0);
    if (tok >= 0) val = *reinterpret_cast<const uint4 *>(src_bh + (int64_t)tok * D + cc * EPC);
    *reinterpret_cast<uint4 *>(&tile_lds[row * LD + cc * EPC]) = val;
    if (fp8) {
      const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        amax = fmaxf(amax, fabsf(bf16_to_float((bf16_bits)(w[j / 2] >> (16 * (j % 2))))));
    }
  }
  __syncthreads();

  if (take_mean) {
    // Per channel: slot pairs (r, r + 32) first, then the 32 pairs in order,
    // as the pooling kernel adds them.
    double *mrow = means + (((int64_t)which * p.B * p.H + bh) * p.max_vt +
                            (tile - p.n_prefix_tiles)) * D;
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
      double sum = 0.0;
#pragma unroll 4
      for (int r = 0; r < 32; ++r) {   // a full unroll hoists every read: 4x the registers
        double pair = 0.0;
        pair += (double)to_float<T>(tile_lds[r * LD + c]);
        pair += (double)to_float<T>(tile_lds[(r + 32) * LD + c]);
        sum += pair;
      }
      mrow[c] = sum / (double)n_real;
    }
  }

  T *out = dst + ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
  const bool col = which == 2;
  for (int vec = threadIdx.x; vec < kTile * D / 8; vec += blockDim.x) {
    __attribute__((aligned(16))) T e8[8];
    if (!col) {
      int sl, c;
      row_layout_decode(vec, 0, D, sl, c);
      const uint4 *srcv = reinterpret_cast<const uint4 *>(&tile_lds[sl * LD + c]);
      uint4 *e8v = reinterpret_cast<uint4 *>(e8);
#pragma unroll
      for (int u = 0; u < (int)(8 * sizeof(T) / 16); ++u) e8v[u] = srcv[u];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int sl, c;
        col_layout_decode(vec, e, D, sl, c);
        e8[e] = tile_lds[sl * LD + c];
      }
    }
    if (sizeof(T) == 2) {
      *reinterpret_cast<uint4 *>(out + vec * 8) = *reinterpret_cast<uint4 *>(e8);
    } else {
      reinterpret_cast<uint4 *>(out + vec * 8)[0] = reinterpret_cast<uint4 *>(e8)[0];
      reinterpret_cast<uint4 *>(out + vec * 8)[1] = reinterpret_cast<uint4 *>(e8)[1];
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (fp8) {
      const int e = fp8_tile_exponent(block_amax(amax, red, 256));
      uint8_t *dst8 = (which == 0 ? q8 : which == 1 ? k8 : v8) +
                      ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
      fp8_write_tile<D, LD>(tile_lds, col, e, dst8, 256);
      if (threadIdx.x == 0)
        scales[((int64_t)bh * p.max_tiles + tile) * 4 + which] = (uint8_t)(e + kFp8ExpBias);
    }
  }
}

template <typename T, int D>
hipError_t gather_t(const Plan &p, const void *q, const void *k, const void *v,
                    const int32_t *s2t, void *qt, void *kt, void *vt, uint8_t *q8,
                    uint8_t *k8, uint8_t *v8, uint8_t *scales, double *means,
                    hipStream_t st) {
  dim3 grid(p.max_tiles, p.B * p.H, 3);
  hipLaunchKernelGGL((gather_kernel<T, D>), grid, dim3(256), 0, st, p,
                     (const T *)q, (const T *)k, (const T *)v, s2t, (T *)qt, (T *)kt,
                     (T *)vt, q8, k8, v8, scales, means);
  return hipGetLastError();
}

}  // namespace
}  // namespace vsa

hipError_t launch_build_map(const Plan &p, int32_t *s2t, hipStream_t stream) {
  int64_t total = (int64_t)p.n_shapes * p.max_tiles * vsa::kTile;
  int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(vsa::build_map_kernel, dim3(blocks), dim3(256), 0, stream, p, s2t);
  return hipGetLastError();
}

hipError_t launch_gather(const Plan &p, const void *q, const void *k, const void *v,
                         const int32_t *s2t, void *qt, void *kt, void *vt, uint8_t *q8,
                         uint8_t *k8, uint8_t *v8, uint8_t *scales, hipStream_t stream,
                         double *means) {
  if (p.dtype == VSA_BF16) {
    if (p.d == 128)
      return vsa::gather_t<bf16_bits, 128>(p, q, k, v, s2t, qt, kt, vt, q8, k8, v8, scales,
                                           means, stream);
    return vsa::gather_t<bf16_bits, 64>(p, q, k, v, s2t, qt, kt, vt, q8, k8, v8, scales,
                                        means, stream);
  }
  if (p.d == 128)
    return vsa::gather_t<float, 128>(p, q, k, v, s2t, qt, kt, vt, nullptr, nullptr, nullptr,
                                     nullptr, means, stream);
  return vsa::gather_t<float, 64>(p, q, k, v, s2t, qt, kt, vt, nullptr, nullptr, nullptr,
                                  nullptr, means, stream);
}
