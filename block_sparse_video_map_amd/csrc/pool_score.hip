// Step 2: pooled tile descriptors (double) and their dot products (float).
//
// Pooling runs one workgroup per (video tile, batch*head, Q|K): the tile is
// read once from the tiled layout into LDS, reduced over its real slots in
// double, and projected (mean gate) or projected-then-reduced (TripPool).
// Scoring is a double-precision GEMM per head, 64x64 outputs per workgroup,
// rounded once to float on the way out.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

// Unpacks one row-layout tile of T into LDS as float [64][LD].
template <typename T, int D, int LD>
__device__ inline void load_tile_f32(const T *__restrict__ src, float *xs) {
  for (int vec = threadIdx.x; vec < kTile * D / 8; vec += blockDim.x) {
    int sl, c;
    row_layout_decode(vec, 0, D, sl, c);
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[sl * LD + c + e] = to_float<T>(src[vec * 8 + e]);
  }
}

// VSA: desc = mean over real slots, times the head's gate.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_mean_gate_kernel(
    Plan p, const T *__restrict__ qt, const T *__restrict__ kt,
    const int32_t *__restrict__ s2t, const float *__restrict__ wq,
    const float *__restrict__ wk, double *__restrict__ pooled) {
  constexpr int LD = D + 1;
  __shared__ float xs[kTile * LD];
  __shared__ double mean[D];
  __shared__ int valid[kTile];

  const int vt_i = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int h = bh % p.H, s = h % p.n_shapes;
  if (vt_i >= p.n_vt[s]) return;
  const int tile = p.n_prefix_tiles + vt_i;
  const T *src = (which == 0 ? qt : kt) + ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
  const float *w = (which == 0 || !wk ? wq : wk) + (int64_t)h * D * D;

  if (threadIdx.x < kTile)
    valid[threadIdx.x] = s2t[((int64_t)s * p.max_tiles + tile) * kTile + threadIdx.x] >= 0;
  load_tile_f32<T, D, LD>(src, xs);
  __syncthreads();

  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    double sum = 0.0;
    int n = 0;
    for (int sl = 0; sl < kTile; ++sl) {
      if (valid[sl]) {
        sum += (double)xs[sl * LD + c];
        ++n;
      }
    }
    mean[c] = sum / (double)n;
  }
  __syncthreads();

  if (threadIdx.x < D) {
    const int j = threadIdx.x;
    double acc = 0.0;
    for (int c = 0; c < D; ++c) acc = fma(mean[c], (double)w[c * D + j], acc);
    pooled[(((int64_t)which * p.B * p.H + bh) * p.max_vt + vt_i) * D + j] = acc;
  }
}

// Veda TripPool: project every real token (d -> R), then [Avg | Max | Min].
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void pool_trippool_kernel(
    Plan p, const T *__restrict__ qt, const T *__restrict__ kt,
    const int32_t *__restrict__ s2t, const float *__restrict__ wq,
    const float *__restrict__ wk, double *__restrict__ pooled) {
  constexpr int LD = D + 1;
  constexpr int G = 256 / R;          // token groups
  constexpr int TPT = kTile / G;      // tokens per thread
  __shared__ float xs[kTile * LD];
  __shared__ float ws[D * R];
  __shared__ double red_sum[G * R], red_max[G * R], red_min[G * R];
  __shared__ int valid[kTile];

  const int vt_i = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int h = bh % p.H, s = h % p.n_shapes;
  if (vt_i >= p.n_vt[s]) return;
  const int tile = p.n_prefix_tiles + vt_i;
  const T *src = (which == 0 ? qt : kt) + ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
  const float *w = (which == 0 ? wq : wk) + (int64_t)h * D * R;

  if (threadIdx.x < kTile)
    valid[threadIdx.x] = s2t[((int64_t)s * p.max_tiles + tile) * kTile + threadIdx.x] >= 0;
  for (int i = threadIdx.x; i < D * R; i += blockDim.x) ws[i] = w[i];
  load_tile_f32<T, D, LD>(src, xs);
  __syncthreads();

  const int j = threadIdx.x % R, g = threadIdx.x / R;
  double acc[TPT];
#pragma unroll
  for (int t = 0; t < TPT; ++t) acc[t] = 0.0;
  for (int c = 0; c < D; ++c) {
    const double wc = (double)ws[c * R + j];
#pragma unroll
    for (int t = 0; t < TPT; ++t) acc[t] = fma((double)xs[(g + t * G) * LD + c], wc, acc[t]);
  }
  double sum = 0.0, mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int t = 0; t < TPT; ++t) {
    if (valid[g + t * G]) {
      sum += acc[t];
      mx = fmax(mx, acc[t]);
      mn = fmin(mn, acc[t]);
    }
  }
  red_sum[g * R + j] = sum;
  red_max[g * R + j] = mx;
  red_min[g * R + j] = mn;
  __syncthreads();

  if (threadIdx.x < R) {
    int n = 0;
    for (int sl = 0; sl < kTile; ++sl) n += valid[sl];
    double ts = 0.0, tx = -INFINITY, tn = INFINITY;
    for (int gg = 0; gg < G; ++gg) {
      ts += red_sum[gg * R + j];
      tx = fmax(tx, red_max[gg * R + j]);
      tn = fmin(tn, red_min[gg * R + j]);
    }
    double *out = pooled + (((int64_t)which * p.B * p.H + bh) * p.max_vt + vt_i) * (3 * R);
    out[j] = ts / (double)n;
    out[R + j] = tx;
    out[2 * R + j] = tn;
  }
}

// s[bh][i][j] = <Qdesc_i, Kdesc_j>, double accumulation, one float rounding.
constexpr int kSB = 64;   // output block edge
constexpr int kSK = 32;   // reduction chunk

__global__ __launch_bounds__(256) void scores_kernel(Plan p, int r,
                                                     const double *__restrict__ pooled,
                                                     float *__restrict__ scores) {
  __shared__ double As[kSB][kSK + 1];
  __shared__ double Bs[kSB][kSK + 1];
  const int bh = blockIdx.z, h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s];
  const int i0 = blockIdx.y * kSB, j0 = blockIdx.x * kSB;
  if (i0 >= n || j0 >= n) return;
  const double *Qd = pooled + (int64_t)bh * p.max_vt * r;
  const double *Kd = pooled + ((int64_t)p.B * p.H + bh) * p.max_vt * r;
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;

  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;

  for (int k0 = 0; k0 < r; k0 += kSK) {
    for (int e = threadIdx.x; e < kSB * kSK; e += blockDim.x) {
      int row = e / kSK, kk = e % kSK;
      bool kin = k0 + kk < r;
      As[row][kk] = (i0 + row < n && kin) ? Qd[(int64_t)(i0 + row) * r + k0 + kk] : 0.0;
      Bs[row][kk] = (j0 + row < n && kin) ? Kd[(int64_t)(j0 + row) * r + k0 + kk] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kSK; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[ty + 16 * a][kk];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[tx + 16 * b][kk];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  float *out = scores + (int64_t)bh * p.max_vt * p.max_vt;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    int i = i0 + ty + 16 * a;
    if (i >= n) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int j = j0 + tx + 16 * b;
      if (j < n) out[(int64_t)i * p.max_vt + j] = (float)acc[a][b];
    }
  }
}

template <typename T, int D>
hipError_t pool_t(const Plan &p, int mode, int R, const void *qt, const void *kt,
                  const int32_t *s2t, const float *wq, const float *wk, double *pooled,
                  hipStream_t st) {
  dim3 grid(p.max_vt, p.B * p.H, 2);
  if (mode == VSA_SCORE_MEAN_GATE) {
    hipLaunchKernelGGL((pool_mean_gate_kernel<T, D>), grid, dim3(256), 0, st, p,
                       (const T *)qt, (const T *)kt, s2t, wq, wk, pooled);
  } else {
    switch (R) {
#define VSA_TRIP(RR)                                                                    \
  case RR:                                                                              \
    hipLaunchKernelGGL((pool_trippool_kernel<T, D, RR>), grid, dim3(256), 0, st, p,     \
                       (const T *)qt, (const T *)kt, s2t, wq, wk, pooled);               \
    break;
      VSA_TRIP(8) VSA_TRIP(16) VSA_TRIP(32) VSA_TRIP(64)
#undef VSA_TRIP
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace vsa

hipError_t launch_pool(const Plan &p, int mode, int proj_dim, const void *qt,
                       const void *kt, const int32_t *s2t, const float *wq,
                       const float *wk, double *pooled, hipStream_t stream) {
  if (p.dtype == VSA_BF16) {
    if (p.d == 128)
      return vsa::pool_t<bf16_bits, 128>(p, mode, proj_dim, qt, kt, s2t, wq, wk, pooled, stream);
    return vsa::pool_t<bf16_bits, 64>(p, mode, proj_dim, qt, kt, s2t, wq, wk, pooled, stream);
  }
  if (p.d == 128)
    return vsa::pool_t<float, 128>(p, mode, proj_dim, qt, kt, s2t, wq, wk, pooled, stream);
  return vsa::pool_t<float, 64>(p, mode, proj_dim, qt, kt, s2t, wq, wk, pooled, stream);
}

hipError_t launch_scores(const Plan &p, int r, const double *pooled, float *scores,
                         hipStream_t stream) {
  int nb = (p.max_vt + vsa::kSB - 1) / vsa::kSB;
  dim3 grid(nb, nb, p.B * p.H);
  hipLaunchKernelGGL(vsa::scores_kernel, grid, dim3(256), 0, stream, p, r, pooled, scores);
  return hipGetLastError();
}
