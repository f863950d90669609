// Steps 2-3 fused: tile scores and top-k without the score matrix.
//
// One workgroup of eight waves takes 16 video query tiles (rows) of one
// (batch, head). Their descriptors are staged in LDS in the operand order of
// the 16x16x4 f64 MFMA. Each wave then walks its 16-column blocks of key
// descriptors (blocks wave, wave + 8, ..., two at a time), streaming them
// from global memory one chunk ahead, and accumulates each 16x16 block of
// scores over the descriptor width in the same order as the score-matrix
// kernel: the scores are bit for bit those of vsa_tile_scores. Each score, rounded once
// to float, is kept as an order-preserving 32-bit key in a register (four
// per block and lane, so a row of up to 4096 tiles needs 128 registers).
//
// The select of the 16 rows runs on those registers. A most-significant-
// digit search over each row's own key range finds the k-th largest key T
// and how many keys equal to T are kept (ties keep the lowest indices): each
// pass splits the row's current range into at most 256 power-of-two bins,
// counts them in an LDS histogram per row and keeps the bin holding the k-th
// largest key (at most five passes for 32-bit keys). Wave ballots then give,
// per row and 16-column block, the 16-bit masks of "key > T" and "key == T";
// a scan over a row's masks keeps the first `need` ties and writes the
// ascending index list directly.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kRows = 16;                 // query rows per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 8;                 // contraction steps (4 channels each) per fetch
constexpr int kBins = 256;
constexpr int kMaxBlocks = VSA_FUSED_MAX_TILES / 16;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;                // -0.0 ranks equal to +0.0
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Width (bits) - 8 of a key range, at least 0: (key - lo) >> shift < 256.
__device__ inline int range_shift(uint32_t lo, uint32_t hi) {
  return max(0, 24 - (int)__clz(hi - lo));
}

// Inclusive prefix sum over the lanes of a `width`-lane segment.
__device__ inline int segment_scan(int v, int lane_in_seg, int width) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    if (d >= width) break;
    const int o = __shfl_up(v, d, width);
    if (lane_in_seg >= d) v += o;
  }
  return v;
}

// NB = column blocks per wave: rows of up to NB * 8 * 16 tiles.
template <int NB>
__global__ __launch_bounds__(kThreads) void score_select_kernel(Plan p, int r,
                                                                 FusedSelectJob job) {
  __shared__ double qs[VSA_FUSED_MAX_R / 4 * 64];     // [step][lane]: A operands
  __shared__ int hist[kRows * kBins];
  __shared__ uint16_t gtmap[kRows * kMaxBlocks], eqmap[kRows * kMaxBlocks];
  __shared__ uint32_t row_lo[kRows], row_hi[kRows];
  __shared__ int row_need[kRows];

  const int bh = blockIdx.y, h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s], k = p.k[s];
  const int i0 = blockIdx.x * kRows;
  if (i0 >= n) return;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int steps = r >> 2;
  const int nblk = (n + 15) >> 4;
  const double *Qd = job.q + (int64_t)bh * job.q_bh;
  const double *Kd = job.k + (int64_t)bh * job.k_bh;

  // Query descriptors: element (row i, channel c) at [c / 4][(c % 4) * 16 + i],
  // so lane l of step m reads row l % 16, channel 4m + l / 16.
  for (int x = t; x < kRows * r; x += kThreads) {
    const int i = x / r, c = x - i * r;
    qs[(c >> 2) * 64 + (c & 3) * 16 + i] = (i0 + i < n) ? Qd[(int64_t)(i0 + i) * r + c] : 0.0;
  }
  if (t < kRows) {
    row_lo[t] = 0xFFFFFFFFu;
    row_hi[t] = 0u;
  }
  __syncthreads();

  // ---- scores: key[4b + e] is row 4e + g, column 16 (wave + 8b) + l16, or 0
  // for a column past the row (no finite score has key 0: the smallest,
  // that of -inf, is 0x007FFFFF, so such keys never fall inside a row's key
  // range). Two blocks at a time, their MFMAs interleaved (two independent
  // accumulation chains), key descriptors fetched one chunk ahead.
  uint32_t key[NB * 4];
#pragma unroll
  for (int b = 0; b < NB; b += 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) key[4 * b + e] = 0u;
    const int blk0 = wave + kWaves * b, blk1 = blk0 + kWaves;
    if (blk0 < nblk) {
      const bool two = blk1 < nblk;
      const double *k0 = Kd + (int64_t)min(blk0 * 16 + l16, n - 1) * r + g;
      const double *k1 = Kd + (int64_t)min(blk1 * 16 + l16, n - 1) * r + g;
      f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
      double c0[kChunk], c1[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        c0[c] = k0[4 * c];
        c1[c] = two ? k1[4 * c] : 0.0;
      }
      for (int m0 = 0; m0 < steps; m0 += kChunk) {
        const bool more = m0 + kChunk < steps;
        double n0[kChunk], n1[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          n0[c] = more ? k0[4 * (m0 + kChunk + c)] : 0.0;
          n1[c] = (more && two) ? k1[4 * (m0 + kChunk + c)] : 0.0;
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const double a = qs[(m0 + c) * 64 + lane];
          acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, c0[c], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, c1[c], acc1, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          c0[c] = n0[c];
          c1[c] = n1[c];
        }
      }
      const bool ok0 = blk0 * 16 + l16 < n, ok1 = blk1 * 16 + l16 < n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[4 * b + e] = ok0 ? order_key((float)acc0[e]) : 0u;
        key[4 * b + 4 + e] = ok1 ? order_key((float)acc1[e]) : 0u;
      }
    }
  }

  // ---- each row's key range.
  {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = 0xFFFFFFFFu;
      hi[e] = 0u;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = key[4 * b + e];
        lo[e] = min(lo[e], kk ? kk : 0xFFFFFFFFu);
        hi[e] = max(hi[e], kk);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        lo[e] = min(lo[e], (uint32_t)__shfl_xor((int)lo[e], o));
        hi[e] = max(hi[e], (uint32_t)__shfl_xor((int)hi[e], o));
      }
      if (l16 == 0) {
        atomicMin(&row_lo[4 * e + g], lo[e]);
        atomicMax(&row_hi[4 * e + g], hi[e]);
      }
    }
  }
  __syncthreads();
  if (t < kRows) {
    row_need[t] = k;
    if (i0 + t >= n) row_hi[t] = row_lo[t];   // no such row: nothing to search
  }
  __syncthreads();

  // ---- narrow every row's range to its k-th largest key.
#pragma unroll 1
  for (int pass = 0; pass < 6; ++pass) {
    bool active = false;
#pragma unroll
    for (int i = 0; i < kRows; ++i) active |= row_lo[i] < row_hi[i];
    if (!active) break;                        // same answer in every thread
    uint32_t lo[4], hi[4];
    int sh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = row_lo[4 * e + g];
      hi[e] = row_hi[4 * e + g];
      sh[e] = range_shift(lo[e], hi[e]);
    }
    for (int x = t; x < kRows * kBins; x += kThreads) hist[x] = 0;
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kk = key[4 * b + e];
        if (lo[e] < hi[e] && kk >= lo[e] && kk <= hi[e])
          atomicAdd(&hist[(4 * e + g) * kBins + ((kk - lo[e]) >> sh[e])], 1);
      }
    }
    __syncthreads();
    {
      // Half a wave per row; lane hl holds bins 255 - 8 hl - j, j = 0..7
      // (counting from the top bin down).
      const int row = 2 * wave + (lane >> 5), hl = lane & 31;
      const uint32_t rlo = row_lo[row], rhi = row_hi[row];
      const int need = row_need[row];
      int c[8], tot = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        c[j] = hist[row * kBins + 255 - 8 * hl - j];
        tot += c[j];
      }
      int above = segment_scan(tot, hl, 32) - tot;
      if (rlo < rhi) {
        const int rsh = range_shift(rlo, rhi);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (above < need && need <= above + c[j]) {
            const uint32_t bin = 255 - 8 * hl - j;
            const uint64_t top = (uint64_t)rlo + ((uint64_t)(bin + 1) << rsh) - 1;
            row_lo[row] = rlo + (bin << rsh);
            row_hi[row] = top < rhi ? (uint32_t)top : rhi;
            row_need[row] = need - above;
          }
          above += c[j];
        }
      }
    }
    __syncthreads();
  }

  // ---- masks of kept keys per row and 16-column block.
  {
    uint32_t T[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) T[e] = row_lo[4 * e + g];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int blk = wave + kWaves * b;
      if (blk < nblk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t gt = __ballot(key[4 * b + e] > T[e]);
          const uint64_t eq = __ballot(key[4 * b + e] == T[e]);
          if (l16 == 0) {
            gtmap[(4 * e + g) * kMaxBlocks + blk] = (uint16_t)(gt >> (16 * g));
            eqmap[(4 * e + g) * kMaxBlocks + blk] = (uint16_t)(eq >> (16 * g));
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- ascending lists: wave w writes rows 2w and 2w + 1; lane l scans
  // blocks 4l .. 4l + 3 of the row.
#pragma unroll 1
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 2 * wave + rr;
    if (i0 + row >= n) break;
    int32_t *out = job.out + (int64_t)bh * job.out_bh + (int64_t)(i0 + row) * job.out_row;
    const int need = row_need[row];
    uint32_t gw[4], ew[4];
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = 4 * lane + j;
      gw[j] = w < nblk ? gtmap[row * kMaxBlocks + w] : 0u;
      ew[j] = w < nblk ? eqmap[row * kMaxBlocks + w] : 0u;
      n_eq += __builtin_popcount(ew[j]);
    }
    // Ties ranked by index: this lane keeps the first (need - ties before it).
    int left = need - (segment_scan(n_eq, lane, 64) - n_eq);
    int n_keep = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = ew[j], sel = 0u;
      while (x && left > 0) {
        const uint32_t low = x & (0u - x);
        sel |= low;
        x ^= low;
        --left;
      }
      gw[j] |= sel;
      n_keep += __builtin_popcount(gw[j]);
    }
    int pos = segment_scan(n_keep, lane, 64) - n_keep;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = gw[j];
      while (x) {
        if (pos < k) out[pos] = (4 * lane + j) * 16 + __builtin_ctz(x);   // always: k kept
        ++pos;
        x &= x - 1u;
      }
    }
    for (int c = k + lane; c < job.out_row; c += 64) out[c] = -1;
  }
}

}  // namespace
}  // namespace vsa

hipError_t launch_score_select(const Plan &p, int r, const FusedSelectJob &job,
                               hipStream_t stream) {
  if (p.max_vt > VSA_FUSED_MAX_TILES || r % 32 != 0 || r > VSA_FUSED_MAX_R)
    return hipErrorInvalidValue;
  dim3 grid((p.max_vt + vsa::kRows - 1) / vsa::kRows, p.B * p.H);
  dim3 block(vsa::kThreads);
  if (p.max_vt <= 1024)
    hipLaunchKernelGGL(vsa::score_select_kernel<8>, grid, block, 0, stream, p, r, job);
  else if (p.max_vt <= 2048)
    hipLaunchKernelGGL(vsa::score_select_kernel<16>, grid, block, 0, stream, p, r, job);
  else
    hipLaunchKernelGGL(vsa::score_select_kernel<32>, grid, block, 0, stream, p, r, job);
  return hipGetLastError();
}
