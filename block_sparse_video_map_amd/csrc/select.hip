// Step 3: top-k video key tiles per video query tile.
//
// One workgroup per score row. Scores become order-preserving 32-bit keys
// (larger key = larger score, -0.0 folded into +0.0) held in registers, each
// thread owning a contiguous run of indices. A most-significant-digit select
// over the row's own key range finds the k-th largest key T and how many keys
// equal to T are kept; ties keep the lowest indices. Each pass splits the
// current range [lo, hi] into at most 256 equal power-of-two bins ((key - lo)
// >> sh), counts them in an LDS histogram and keeps the bin holding the k-th
// largest key; starting from the row's min..max (not the top byte of the
// key) spreads the first pass over the bins instead of piling the row into
// the few bins its exponents share. At most five passes. A single ordered
// pass then flags "key > T, or key == T among the first ties" and compacts
// the flagged indices with block prefix sums, which yields the ascending
// block-index list directly. O(n) work per row, exact.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;

__device__ inline uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;                     // -0.0 ranks equal to +0.0
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block scan of one int per thread; also returns the block total.
__device__ inline int block_exclusive_scan(int v, int *wave_tot, int &total) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    if (w < wave) base += wave_tot[w];
    total += wave_tot[w];
  }
  __syncthreads();
  return base + incl - v;
}

// E = keys per thread (n <= E * kSelThreads).
template <int E>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Plan p, SelectJob job) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kSelWaves];
  __shared__ int sel_bin, sel_above;
  __shared__ uint32_t wave_lo[kSelWaves], wave_hi[kSelWaves];

  const int i = blockIdx.x, bh = blockIdx.y, h = bh % p.H, s = h % p.n_shapes;
  if (i >= p.n_vt[s]) return;                   // one row per video query tile
  const int n = job.ncols < 0 ? p.n_vt[s] : job.ncols;
  const int k = job.k < 0 ? p.k[s] : job.k;
  const int t = threadIdx.x;
  const int j0 = t * E;                         // this thread's first index

  const float *row = job.scores + (int64_t)bh * job.in_bh + (int64_t)i * job.in_row;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (j0 + e < n) ? order_key(row[j0 + e]) : 0u;

  // The row's key range.
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (j0 + e < n) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if (t % 64 == 0) {
    wave_lo[t / 64] = lo;
    wave_hi[t / 64] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    lo = min(lo, wave_lo[w]);
    hi = max(hi, wave_hi[w]);
  }

  // Narrow [lo, hi] to the k-th largest key; need = how many keys equal to
  // it are kept. Each pass leaves a range below 2^sh, so sh drops by 8.
  int need = k;
#pragma unroll 1
  for (int pass = 0; pass < 6 && lo < hi; ++pass) {
    const int sh = max(0, 24 - (int)__clz(hi - lo));        // bit length - 8
    hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (j0 + e < n && key[e] >= lo && key[e] <= hi) atomicAdd(&hist[(key[e] - lo) >> sh], 1);
    __syncthreads();
    // Counts from the top bin down: thread t looks at bin 255 - t.
    const int c = hist[255 - t];
    int total;
    const int above = block_exclusive_scan(c, wave_tot, total);   // keys in higher bins
    if (above < need && need <= above + c) {
      sel_bin = 255 - t;
      sel_above = above;
    }
    __syncthreads();
    need -= sel_above;
    const uint64_t top = (uint64_t)lo + ((uint64_t)(sel_bin + 1) << sh) - 1;
    lo += (uint32_t)sel_bin << sh;
    hi = top < hi ? (uint32_t)top : hi;
    __syncthreads();
  }
  const uint32_t T = lo;                        // k-th largest key; keep `need` ties

  // Ordered compaction: ties are ranked by index among themselves.
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) n_eq += (j0 + e < n && key[e] == T);
  int tot_eq;
  int eq_rank = block_exclusive_scan(n_eq, wave_tot, tot_eq);
  int n_keep = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (j0 + e < n) {
      if (key[e] > T) {
        ++n_keep;
      } else if (key[e] == T) {
        n_keep += eq_rank < need;
        ++eq_rank;
      }
    }
  }
  int tot_keep;
  int pos = block_exclusive_scan(n_keep, wave_tot, tot_keep);   // tot_keep == k
  int32_t *out = job.out + (int64_t)bh * job.out_bh + (int64_t)i * job.out_row;
  eq_rank -= n_eq;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (j0 + e < n) {
      bool keep = key[e] > T;
      if (key[e] == T) {
        keep = eq_rank < need;
        ++eq_rank;
      }
      if (keep) out[pos++] = j0 + e;
    }
  }
  for (int c = k + t; c < job.out_row; c += kSelThreads) out[c] = -1;
}

}  // namespace
}  // namespace vsa

hipError_t launch_select(const Plan &p, const SelectJob &job, hipStream_t stream) {
  dim3 grid(p.max_vt, p.B * p.H);
  dim3 block(vsa::kSelThreads);
  const int e = (job.max_cols + vsa::kSelThreads - 1) / vsa::kSelThreads;
  if (e <= 4)
    hipLaunchKernelGGL(vsa::select_kernel<4>, grid, block, 0, stream, p, job);
  else if (e <= 8)
    hipLaunchKernelGGL(vsa::select_kernel<8>, grid, block, 0, stream, p, job);
  else if (e <= 16)
    hipLaunchKernelGGL(vsa::select_kernel<16>, grid, block, 0, stream, p, job);
  else
    hipLaunchKernelGGL(vsa::select_kernel<32>, grid, block, 0, stream, p, job);
  return hipGetLastError();
}
