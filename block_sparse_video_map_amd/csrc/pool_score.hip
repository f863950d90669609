// Step 2: pooled tile descriptors (double) and their dot products (float).
//
// Mean gate: one workgroup per 16 video tiles of one (batch*head, Q|K); the
// means are reduced in double and multiplied by the head's gate on the f64
// MFMA. TripPool: one workgroup per (video tile, batch*head, Q|K); the tile's
// tokens are projected on the f64 MFMA, then reduced to [Avg | Max | Min].
// Scoring is a double-precision GEMM per head on the f64 MFMA, 64x64 outputs
// per workgroup with operands staged through LDS, rounded once to float on
// the way out.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

// VSA: desc = mean over real slots, times the head's gate.
//
// One workgroup takes 16 video tiles of one (batch*head, Q|K). Means: every
// thread loads four 16-byte vectors of a tile (two slots x 8 channels of two
// channel groups), adds the two slots in double, and the 32 slot pairs of a
// channel are then summed from LDS; pad slots hold zero in the tiled copy, so
// the sum over all 64 slots divided by the real-slot count is the mean.
// Gate: the 16 x D means times the D x D gate on the 16x16x4 f64 MFMA, wave w
// owning 16-column blocks w, w+4.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kPoolTiles = 16;
constexpr int kTripTiles = 8;                // TripPool: tiles per workgroup (one P load)

template <typename T>
__device__ inline void load8_f32(const T *__restrict__ src, float (&v)[8]);
template <>
__device__ inline void load8_f32<bf16_bits>(const bf16_bits *__restrict__ src, float (&v)[8]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ inline void load8_f32<float>(const float *__restrict__ src, float (&v)[8]) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 a = *reinterpret_cast<const f32x4 *>(src);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Gate product of up to 16 mean rows on the f64 MFMA: mean is [16][D + 1]
// in LDS (rows past nt zero), w the head's D x D gate, dst the first output
// row (D doubles apart). Wave w owns 16-column blocks w, w + 4, ... A: lane l
// holds mean[l%16][k0 + l/16]; B: gate[k0 + l/16][col0 + l%16]; D element e:
// row 4e + l/16, column l%16.
template <int D>
__device__ inline void gate_rows(const double *mean, const float *__restrict__ w, double *dst,
                                 int nt) {
  constexpr int LM = D + 1;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int l16 = lane % 16, g4 = lane / 16;
  for (int cb = wave; cb < D / 16; cb += 4) {
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int k0 = 0; k0 < D; k0 += 4) {
      const double a = mean[l16 * LM + k0 + g4];
      const double b = (double)w[(k0 + g4) * D + cb * 16 + l16];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * e + g4;
      if (row < nt) dst[(int64_t)row * D + cb * 16 + l16] = acc[e];
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_mean_gate_kernel(
    Plan p, PoolJob job, const int32_t *__restrict__ s2t, double *__restrict__ pooled) {
  constexpr int NV = kTile * D / 8;          // 8-element vectors per tile
  constexpr int VPT = NV / 256;              // vectors per thread (4 for D=128)
  static_assert(VPT >= 1 && NV % 256 == 0, "tile must split evenly over 256 threads");
  __shared__ double part[32 * D];            // [slot pair][channel]
  constexpr int LM = D + 1;                  // padded rows: conflict-free MFMA reads
  __shared__ double mean[kPoolTiles * LM];   // [tile][channel]
  __shared__ int count[kPoolTiles];

  const int bh = job.bh0 + blockIdx.y, which = blockIdx.z;
  const int nbh = job.nbh < 0 ? p.B * p.H : job.nbh;
  const int h = bh % p.H, s = h % p.n_shapes;
  const int n = job.ntiles < 0 ? p.n_vt[s] : job.ntiles;
  const int vt0 = blockIdx.x * kPoolTiles;
  if (vt0 >= n) return;
  const int nt = min(kPoolTiles, n - vt0);
  const T *src = (const T *)job.src[which] +
                 ((int64_t)bh * p.max_tiles + job.tile0 + vt0) * (kTile * D);
  const float *w = job.w[which] + (int64_t)h * D * D;
  const int t = threadIdx.x, lane = t % 64, wave = t / 64;

  // Real-slot counts: wave w counts tiles w, w+4, ... (one slot per lane).
  for (int tt = wave; tt < nt; tt += 4) {
    const int tok = s2t[((int64_t)s * p.max_tiles + job.tile0 + vt0 + tt) * kTile + lane];
    const int c = __popcll(__ballot(tok >= 0));
    if (lane == 0) count[tt] = c;
  }
  for (int tt = 0; tt < nt; ++tt) {
    const T *tile = src + (int64_t)tt * kTile * D;
    // Vector v of the tile (row layout): slot (v/64/(D/16))*32 + v%32,
    // channels ((v/64)%(D/16))*16 + ((v%64)/32)*8 + 0..7.
    double acc[VPT / 2][8];
#pragma unroll
    for (int a = 0; a < VPT / 2; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = 0.0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      float v[8];
      load8_f32<T>(tile + (int64_t)(t + 256 * i) * 8, v);
      // i and i + VPT/2 hold the two slot halves of the same channels.
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i % (VPT / 2)][e] += (double)v[e];
    }
#pragma unroll
    for (int a = 0; a < VPT / 2; ++a) {
      const int vec = t + 256 * a;
      const int blk = vec / 64;
      const int c0 = (blk % (D / 16)) * 16 + ((vec % 64) / 32) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) part[(lane % 32) * D + c0 + e] = acc[a][e];
    }
    __syncthreads();
    if (t < D) {
      double sum = 0.0;
#pragma unroll 8
      for (int r = 0; r < 32; ++r) sum += part[r * D + t];
      mean[tt * LM + t] = sum / (double)count[tt];
    }
    __syncthreads();
  }
  for (int tt = nt; tt < kPoolTiles; ++tt)
    if (t < D) mean[tt * LM + t] = 0.0;        // rows past the last tile
  __syncthreads();

  gate_rows<D>(mean, w, pooled + (((int64_t)which * nbh + bh - job.bh0) * job.rows + vt0) * D,
               nt);
}

// Mean gate without the tiles: the gather pass left each video tile's means
// at the tile's own row of `pooled`; a workgroup takes 16 rows of one
// (batch*head, Q|K), reads them into LDS and overwrites them with their gate
// product (the same gate_rows as the pooling kernel, so the same values).
template <int D>
__global__ __launch_bounds__(256) void gate_means_kernel(Plan p, const float *wq,
                                                         const float *wk, double *pooled) {
  constexpr int LM = D + 1;
  __shared__ double mean[kPoolTiles * LM];
  const int bh = blockIdx.y, which = blockIdx.z;
  const int h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s];
  const int vt0 = blockIdx.x * kPoolTiles;
  if (vt0 >= n) return;
  const int nt = min(kPoolTiles, n - vt0);
  double *rows = pooled + (((int64_t)which * p.B * p.H + bh) * p.max_vt + vt0) * D;
  for (int x = threadIdx.x; x < kPoolTiles * D; x += blockDim.x) {
    const int tt = x / D, c = x % D;
    mean[tt * LM + c] = tt < nt ? rows[(int64_t)tt * D + c] : 0.0;
  }
  __syncthreads();
  gate_rows<D>(mean, (which == 0 ? wq : wk) + (int64_t)h * D * D, rows, nt);
}

// Veda TripPool: project every real token (d -> R), then the statistics the
// mode asks for, written in the order [Avg | Max | Min] (bits 1, 2, 4 of stats).
// A workgroup of four waves takes kTripTiles consecutive tiles of one
// (batch*head, Q|K), stages the head's projection in LDS once (transposed,
// float) and gives each wave its own tiles: no barrier inside the tile loop.
// The projection X[64 tokens x D] . P[D x R] runs on the 16x16x4 f64 MFMA,
// 4 x RB blocks of 16 tokens x 16 columns per wave. Lane l reads the four
// consecutive channels k0 + 4*(l/16) + m of its token row straight from the
// tiled copy (8 or 16 contiguous bytes) and of its column of P; MFMA m
// contracts channel m of each lane's group. Element e of block (rb, cb) in
// lane l is token 16 rb + 4e + l/16, column 16 cb + l%16. The statistics
// reduce the four elements of a lane, the four lanes of a column, then the
// four token blocks in order.
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void pool_trippool_kernel(
    Plan p, PoolJob job, int stats, const int32_t *__restrict__ s2t,
    double *__restrict__ pooled) {
  constexpr int LD = D + 4;                  // float rows, 16-byte aligned
  constexpr int RB = (R + 15) / 16;          // 16-column blocks
  __shared__ __attribute__((aligned(16))) float pt[RB * 16 * LD];   // P transposed

  const int bh = job.bh0 + blockIdx.y, which = blockIdx.z;
  const int nbh = job.nbh < 0 ? p.B * p.H : job.nbh;
  const int h = bh % p.H, s = h % p.n_shapes;
  const int n_rows = job.ntiles < 0 ? p.n_vt[s] : job.ntiles;
  const int first = blockIdx.x * kTripTiles;
  if (first >= n_rows) return;
  const int last = min(first + kTripTiles, n_rows);
  const float *w = job.w[which] + (int64_t)h * D * R;

  // The head's projection, once per workgroup: consecutive threads read
  // consecutive columns of a row of P (coalesced), stored transposed.
  for (int i = threadIdx.x; i < RB * 16 * D; i += blockDim.x) {
    const int j = i % (RB * 16), c = i / (RB * 16);   // pt[j][c] = P[c][j], zero past R
    pt[j * LD + c] = j < R ? w[c * R + j] : 0.f;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, g = lane / 16, l16 = lane % 16;
  const int width = __builtin_popcount(stats) * R;

  for (int vt_i = first + wave; vt_i < last; vt_i += 4) {
    const int tile = job.tile0 + vt_i;
    const T *src = (const T *)job.src[which] + ((int64_t)bh * p.max_tiles + tile) * (kTile * D);
    const uint64_t valid = __ballot(s2t[((int64_t)s * p.max_tiles + tile) * kTile + lane] >= 0);
    const int n = __popcll(valid);

    f64x4 acc[4][RB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) acc[rb][cb] = (f64x4){0.0, 0.0, 0.0, 0.0};
    // Token 16 rb + l16, channels k0 + 4g .. +3 in the row layout: slot
    // group (16 rb + l16) / 32, channel block k0 / 16, half g / 2, offset
    // 4 (g % 2) within the 8-channel run.
#pragma unroll 2
    for (int k0 = 0; k0 < D; k0 += 16) {
      double a4[4][4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int sl = 16 * rb + l16;
        const T *x = src + ((sl / 32) * (D / 16) + k0 / 16) * 512 + ((g / 2) * 32 + sl % 32) * 8 +
                     4 * (g % 2);
        if constexpr (sizeof(T) == 2) {
          const uint2 w2 = *reinterpret_cast<const uint2 *>(x);
          a4[rb][0] = __uint_as_float(w2.x << 16);
          a4[rb][1] = __uint_as_float(w2.x & 0xFFFF0000u);
          a4[rb][2] = __uint_as_float(w2.y << 16);
          a4[rb][3] = __uint_as_float(w2.y & 0xFFFF0000u);
        } else {
          const float4 f4 = *reinterpret_cast<const float4 *>(x);
          a4[rb][0] = f4.x;
          a4[rb][1] = f4.y;
          a4[rb][2] = f4.z;
          a4[rb][3] = f4.w;
        }
      }
      double b4[RB][4];
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const float4 pb = *reinterpret_cast<const float4 *>(pt + (cb * 16 + l16) * LD + k0 + 4 * g);
        b4[cb][0] = pb.x;
        b4[cb][1] = pb.y;
        b4[cb][2] = pb.z;
        b4[cb][3] = pb.w;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int cb = 0; cb < RB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[rb][m], b4[cb][m], acc[rb][cb],
                                                              0, 0, 0);
    }

    double *out0 = pooled + (((int64_t)which * nbh + bh - job.bh0) * job.rows + vt_i) * width;
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      double ts = 0.0, tx = -INFINITY, tn = INFINITY;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        double sum = 0.0, mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((valid >> (16 * rb + 4 * e + g)) & 1ull) {
            sum += acc[rb][cb][e];
            mx = fmax(mx, acc[rb][cb][e]);
            mn = fmin(mn, acc[rb][cb][e]);
          }
        }
#pragma unroll
        for (int d = 16; d < 64; d <<= 1) {  // the four lanes of a column
          sum += __shfl_xor(sum, d);
          mx = fmax(mx, __shfl_xor(mx, d));
          mn = fmin(mn, __shfl_xor(mn, d));
        }
        ts += sum;
        tx = fmax(tx, mx);
        tn = fmin(tn, mn);
      }
      const int j = cb * 16 + l16;
      if (g == 0 && j < R) {
        double *out = out0 + j;
        if (stats & 1) {
          *out = ts / (double)n;
          out += R;
        }
        if (stats & 2) {
          *out = tx;
          out += R;
        }
        if (stats & 4) *out = tn;
      }
    }
  }
}

// s[bh][i][j] = <Qdesc_i, Kdesc_j>: a double-precision GEMM per head on the
// 16x16x4 f64 MFMA, rounded once to float on the way out. A workgroup owns a
// 64x64 block of scores, each of its four waves a 32x32 quarter (2x2 MFMA
// blocks). Per 16-wide slice of the descriptor, lane l loads four consecutive
// doubles of its row at offset 4*(l/16): MFMA m then contracts channel
// k0 + 4*(l/16) + m of both operands, so the four products cover the slice.
constexpr int kSB = 64;   // output block edge
constexpr int kKC = 16;   // contraction chunk staged in LDS
constexpr int kLK = kKC + 2;   // padded LDS row (doubles)

// Scores: S = Qd Kd^T per (batch, head), 64x64 outputs per workgroup of four
// waves (each 32x32 = 2x2 blocks of the 16x16x4 f64 MFMA). The 64-row slices
// of Qd and Kd are staged through LDS in chunks of 16 contraction columns,
// double-buffered: every thread fetches 4 doubles of each for the next chunk
// while the current chunk is multiplied.
__global__ __launch_bounds__(256) void scores_kernel(Plan p, int r, ScoreJob job) {
  __shared__ double As[2][kSB * kLK];
  __shared__ double Bs[2][kSB * kLK];
  const int bh = job.bh0 + blockIdx.z, h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s];                                   // query rows
  const int m = job.ncols < 0 ? n : job.ncols;               // key columns
  const int i0 = blockIdx.y * kSB, j0 = blockIdx.x * kSB;
  if (i0 >= n || j0 >= m) return;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / 64);
  const int lane = t % 64, g = lane / 16, l16 = lane % 16;
  const int wr = (wave / 2) * 32, wc = (wave % 2) * 32;    // wave's block inside the 64x64
  const double *Qd = job.q + (int64_t)(bh - job.bh0) * job.q_bh;
  const double *Kd = job.k + (int64_t)(bh - job.bh0) * job.k_bh;

  // Thread t stages row t/4, columns 4*(t%4) .. +3 of the chunk, for A and B.
  const int srow = t / 4, scol = (t % 4) * 4;
  const bool oka = i0 + srow < n, okb = j0 + srow < m;
  const double *qa = Qd + (int64_t)(i0 + srow) * r + scol;
  const double *kb = Kd + (int64_t)(j0 + srow) * r + scol;
  double ra[4], rb[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bool okk = k0 + scol + m < r;
      ra[m] = (oka && okk) ? qa[k0 + m] : 0.0;
      rb[m] = (okb && okk) ? kb[k0 + m] : 0.0;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      As[buf][srow * kLK + scol + m] = ra[m];
      Bs[buf][srow * kLK + scol + m] = rb[m];
    }
  };

  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (f64x4){0.0, 0.0, 0.0, 0.0};

  const int nchunks = (r + kKC - 1) / kKC;
  fetch(0);
  stage(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) fetch((c + 1) * kKC);
    // A: lane l holds row l%16 (of a 16-row block), column k + l/16; B alike.
#pragma unroll
    for (int k = 0; k < kKC; k += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        av[a] = As[buf][(wr + a * 16 + l16) * kLK + k + g];
        bv[a] = Bs[buf][(wc + a * 16 + l16) * kLK + k + g];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (c + 1 < nchunks) stage(buf ^ 1);
    __syncthreads();
  }
  // D element e of lane l is row 4*e + l/16, column l % 16 of the block.
  float *out = job.out + (int64_t)bh * job.out_bh;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + wr + a * 16 + 4 * e + g, j = j0 + wc + b * 16 + l16;
        if (i < n && j < m) out[(int64_t)i * job.out_row + j] = (float)acc[a][b][e];
      }
}

template <typename T, int D>
hipError_t pool_t(const Plan &p, int mode, int R, const PoolJob &job, int nsrc,
                  const int32_t *s2t, double *pooled, hipStream_t st) {
  const int rows = job.ntiles < 0 ? p.max_vt : job.ntiles;
  const int nbh = job.nbh < 0 ? p.B * p.H : job.nbh;
  dim3 grid((rows + kTripTiles - 1) / kTripTiles, nbh, nsrc);
  if (mode == VSA_SCORE_MEAN_GATE) {
    dim3 grid_mg((rows + kPoolTiles - 1) / kPoolTiles, nbh, nsrc);
    hipLaunchKernelGGL((pool_mean_gate_kernel<T, D>), grid_mg, dim3(256), 0, st, p, job, s2t,
                       pooled);
  } else {
    switch (R) {
#define VSA_TRIP(RR)                                                                    \
  case RR:                                                                              \
    hipLaunchKernelGGL((pool_trippool_kernel<T, D, RR>), grid, dim3(256), 0, st, p, job, \
                       trippool_stats(mode), s2t, pooled);                               \
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

hipError_t launch_pool(const Plan &p, int mode, int proj_dim, const PoolJob &job, int nsrc,
                       const int32_t *s2t, double *pooled, hipStream_t stream) {
  if (p.dtype == VSA_BF16) {
    if (p.d == 128)
      return vsa::pool_t<bf16_bits, 128>(p, mode, proj_dim, job, nsrc, s2t, pooled, stream);
    return vsa::pool_t<bf16_bits, 64>(p, mode, proj_dim, job, nsrc, s2t, pooled, stream);
  }
  if (p.d == 128)
    return vsa::pool_t<float, 128>(p, mode, proj_dim, job, nsrc, s2t, pooled, stream);
  return vsa::pool_t<float, 64>(p, mode, proj_dim, job, nsrc, s2t, pooled, stream);
}

hipError_t launch_gate_means(const Plan &p, const float *wq, const float *wk, double *pooled,
                             hipStream_t stream) {
  dim3 grid((p.max_vt + vsa::kPoolTiles - 1) / vsa::kPoolTiles, p.B * p.H, 2);
  if (p.d == 128)
    hipLaunchKernelGGL(vsa::gate_means_kernel<128>, grid, dim3(256), 0, stream, p, wq, wk,
                       pooled);
  else
    hipLaunchKernelGGL(vsa::gate_means_kernel<64>, grid, dim3(256), 0, stream, p, wq, wk,
                       pooled);
  return hipGetLastError();
}

hipError_t launch_scores(const Plan &p, int r, const ScoreJob &job, hipStream_t stream) {
  const int cols = job.ncols < 0 ? p.max_vt : job.ncols;
  const int nbh = job.nbh < 0 ? p.B * p.H : job.nbh;
  dim3 grid((cols + vsa::kSB - 1) / vsa::kSB, (p.max_vt + vsa::kSB - 1) / vsa::kSB, nbh);
  hipLaunchKernelGGL(vsa::scores_kernel, grid, dim3(256), 0, stream, p, r, job);
  return hipGetLastError();
}
