// Step 2: pooled tile descriptors (double) and their dot products (float).
//
// Pooling runs one workgroup per (video tile, batch*head, Q|K): the tile is
// read once from the tiled layout into LDS, reduced over its real slots in
// double, and projected (mean gate) or projected-then-reduced (TripPool).
// Scoring is a double-precision GEMM per head on the f64 MFMA, 64x64 outputs
// per workgroup, rounded once to float on the way out.
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

  // Four independent partial sums per channel / output keep the double adds
  // and FMAs from forming one long dependency chain.
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    double part[4] = {0.0, 0.0, 0.0, 0.0};
    int n = 0;
#pragma unroll 4
    for (int sl = 0; sl < kTile; ++sl) {
      if (valid[sl]) {
        part[sl % 4] += (double)xs[sl * LD + c];
        ++n;
      }
    }
    mean[c] = ((part[0] + part[1]) + (part[2] + part[3])) / (double)n;
  }
  __syncthreads();

  if (threadIdx.x < D) {
    const int j = threadIdx.x;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int c = 0; c < D; ++c) acc[c % 4] = fma(mean[c], (double)w[c * D + j], acc[c % 4]);
    pooled[(((int64_t)which * p.B * p.H + bh) * p.max_vt + vt_i) * D + j] =
        (acc[0] + acc[1]) + (acc[2] + acc[3]);
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

// s[bh][i][j] = <Qdesc_i, Kdesc_j>: a double-precision GEMM per head on the
// 16x16x4 f64 MFMA, rounded once to float on the way out. A workgroup owns a
// 64x64 block of scores, each of its four waves a 32x32 quarter (2x2 MFMA
// blocks). Per 16-wide slice of the descriptor, lane l loads four consecutive
// doubles of its row at offset 4*(l/16): MFMA m then contracts channel
// k0 + 4*(l/16) + m of both operands, so the four products cover the slice.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kSB = 64;   // output block edge

__global__ __launch_bounds__(256) void scores_kernel(Plan p, int r,
                                                     const double *__restrict__ pooled,
                                                     float *__restrict__ scores) {
  const int bh = blockIdx.z, h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s];
  const int i0 = blockIdx.y * kSB, j0 = blockIdx.x * kSB;
  if (i0 >= n || j0 >= n) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, g = lane / 16, l16 = lane % 16;
  const int wi = i0 + (wave / 2) * 32, wj = j0 + (wave % 2) * 32;
  const double *Qd = pooled + (int64_t)bh * p.max_vt * r;
  const double *Kd = pooled + ((int64_t)p.B * p.H + bh) * p.max_vt * r;

  int ra[2], rb[2];
  bool va[2], vb[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    ra[a] = wi + a * 16 + l16;
    rb[a] = wj + a * 16 + l16;
    va[a] = ra[a] < n;
    vb[a] = rb[a] < n;
  }
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (f64x4){0.0, 0.0, 0.0, 0.0};

  for (int k0 = 0; k0 < r; k0 += 16) {
    const int kk = k0 + 4 * g;          // r is a multiple of 4: groups are all-in or all-out
    double av[2][4], bv[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const bool oka = va[a] && kk < r, okb = vb[a] && kk < r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        av[a][m] = oka ? Qd[(int64_t)ra[a] * r + kk + m] : 0.0;
        bv[a][m] = okb ? Kd[(int64_t)rb[a] * r + kk + m] : 0.0;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a][m], bv[b][m], acc[a][b], 0, 0, 0);
  }
  // D element e of lane l is row 4*e + l/16, column l % 16 of the block.
  float *out = scores + (int64_t)bh * p.max_vt * p.max_vt;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = wi + a * 16 + 4 * e + g, j = wj + b * 16 + l16;
        if (i < n && j < n) out[(int64_t)i * p.max_vt + j] = (float)acc[a][b][e];
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
