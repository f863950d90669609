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
// The projection X[64 tokens x D] . P[D x R] runs on the 16x16x4 f64 MFMA:
// wave w owns tokens 16w..16w+15 and all R columns (16-column blocks). Lane
// l reads four consecutive channels k0 + 4*(l/16) + m of its token row and of
// its column of P (transposed in LDS), MFMA m contracting channel m of that
// group. Each lane then holds four tokens (rows 4e + l/16) of one column
// (l % 16); the statistics are reduced across lanes, then across waves.
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void pool_trippool_kernel(
    Plan p, const T *__restrict__ qt, const T *__restrict__ kt,
    const int32_t *__restrict__ s2t, const float *__restrict__ wq,
    const float *__restrict__ wk, double *__restrict__ pooled) {
  constexpr int LD = D + 4;                  // float rows, 16-byte aligned
  constexpr int RB = (R + 15) / 16;          // 16-column blocks
  __shared__ __attribute__((aligned(16))) float xs[kTile * LD];
  __shared__ __attribute__((aligned(16))) float pt[RB * 16 * LD];   // P transposed
  __shared__ double red[3][4][RB * 16];      // [stat][wave][column]
  __shared__ int valid[kTile];

  const int vt_i = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int h = bh % p.H, s = h % p.n_shapes;
  if (vt_i >= p.n_vt[s]) return;
  const int tile = p.n_prefix_tiles + vt_i;
  const T *src = (which == 0 ? qt : kt) + ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
  const float *w = (which == 0 ? wq : wk) + (int64_t)h * D * R;

  if (threadIdx.x < kTile)
    valid[threadIdx.x] = s2t[((int64_t)s * p.max_tiles + tile) * kTile + threadIdx.x] >= 0;
  for (int i = threadIdx.x; i < RB * 16 * D; i += blockDim.x) {
    const int c = i % D, j = i / D;          // pt[j][c] = P[c][j], zero past R
    pt[j * LD + c] = j < R ? w[c * R + j] : 0.f;
  }
  load_tile_f32<T, D, LD>(src, xs);
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, g = lane / 16, l16 = lane % 16;
  f64x4 acc[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = (f64x4){0.0, 0.0, 0.0, 0.0};
  const float *xrow = xs + (wave * 16 + l16) * LD;
#pragma unroll 2
  for (int k0 = 0; k0 < D; k0 += 16) {
    const int kk = k0 + 4 * g;
    const float4 xa = *reinterpret_cast<const float4 *>(xrow + kk);
    const double a4[4] = {xa.x, xa.y, xa.z, xa.w};
    double b4[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const float4 pb = *reinterpret_cast<const float4 *>(pt + (b * 16 + l16) * LD + kk);
      b4[b][0] = pb.x; b4[b][1] = pb.y; b4[b][2] = pb.z; b4[b][3] = pb.w;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int b = 0; b < RB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[m], b4[b][m], acc[b], 0, 0, 0);
  }

  // Element e of lane l: token wave*16 + 4e + l/16, column b*16 + l%16.
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    double sum = 0.0, mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (valid[wave * 16 + 4 * e + g]) {
        sum += acc[b][e];
        mx = fmax(mx, acc[b][e]);
        mn = fmin(mn, acc[b][e]);
      }
    }
#pragma unroll
    for (int d = 16; d < 64; d <<= 1) {      // the four lanes of a column
      sum += __shfl_xor(sum, d);
      mx = fmax(mx, __shfl_xor(mx, d));
      mn = fmin(mn, __shfl_xor(mn, d));
    }
    if (g == 0) {
      red[0][wave][b * 16 + l16] = sum;
      red[1][wave][b * 16 + l16] = mx;
      red[2][wave][b * 16 + l16] = mn;
    }
  }
  __syncthreads();

  if (threadIdx.x < R) {
    const int j = threadIdx.x;
    int n = 0;
    for (int sl = 0; sl < kTile; ++sl) n += valid[sl];
    double ts = 0.0, tx = -INFINITY, tn = INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      ts += red[0][ww][j];
      tx = fmax(tx, red[1][ww][j]);
      tn = fmin(tn, red[2][ww][j]);
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

  // Operands of one 16-wide slice: av/bv[buffer][block][m]; the next slice is
  // fetched while the current one is multiplied.
  double av[2][2][4], bv[2][2][4];
  auto fetch = [&](int buf, int k0) {
    const int kk = k0 + 4 * g;          // r is a multiple of 4: groups are all-in or all-out
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const bool oka = va[a] && kk < r, okb = vb[a] && kk < r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        av[buf][a][m] = oka ? Qd[(int64_t)ra[a] * r + kk + m] : 0.0;
        bv[buf][a][m] = okb ? Kd[(int64_t)rb[a] * r + kk + m] : 0.0;
      }
    }
  };
  auto multiply = [&](int buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[buf][a][m], bv[buf][b][m],
                                                           acc[a][b], 0, 0, 0);
  };
  fetch(0, 0);
  for (int k0 = 0; k0 < r; k0 += 32) {
    if (k0 + 16 < r) fetch(1, k0 + 16);
    multiply(0);
    if (k0 + 16 >= r) break;
    if (k0 + 32 < r) fetch(0, k0 + 32);
    multiply(1);
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
