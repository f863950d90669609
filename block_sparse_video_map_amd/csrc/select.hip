// Step 3: top-k video key tiles per video query tile.
//
// Rows of up to 4096 keys: one wave per score row, four rows per workgroup;
// the waves never wait for one another (longer rows: one workgroup per row,
// below). Scores become order-preserving 32-bit keys (larger key =
// larger score, -0.0 folded into +0.0) held in registers; lane l holds
// indices l, l + 64, l + 128, ..., so every load is one coalesced 256-byte
// segment of the row. A most-significant-digit search over the row's own key
// range finds the k-th largest key T and how many keys equal to T are kept
// (ties keep the lowest indices): each pass splits the current range
// [lo, hi] into at most 256 equal power-of-two bins ((key - lo) >> sh),
// counts them in the wave's LDS histogram and keeps the bin holding the k-th
// largest key. Starting from the row's min..max (not the top byte of the key)
// spreads the first pass over the bins instead of piling the row into the
// few bins its exponents share. At most five passes. The kept indices then
// come out in ascending order, 64 at a time, from two ballots per register:
// "key > T" and "key == T" (ranked among the ties by index). O(n) work per
// row, exact.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSelWaves = 4;
constexpr int kSelThreads = 64 * kSelWaves;

__device__ inline uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;                     // -0.0 ranks equal to +0.0
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Set bits of m below this lane.
__device__ inline int bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// E = keys per lane (n <= 64 E).
template <int E>
__global__ __launch_bounds__(kSelThreads) void select_wave_kernel(Plan p, SelectJob job) {
  __shared__ int hist[kSelWaves][256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * kSelWaves + wave, bh = blockIdx.y, h = bh % p.H,
            s = h % p.n_shapes;
  if (i >= p.n_vt[s]) return;                   // one row per video query tile
  const int n = job.ncols < 0 ? p.n_vt[s] : job.ncols;
  const int k = job.k < 0 ? p.k[s] : job.k;
  int *hw = hist[wave];

  const float *row = job.scores + (int64_t)bh * job.in_bh + (int64_t)i * job.in_row;
  // Indices past the row hold key 0, which no finite score has (the
  // smallest is that of -inf, 0x007FFFFF): the row's range [lo, hi] starts
  // above it, so those keys never enter a histogram or the kept set.
  uint32_t key[E];
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  // Loads from a clamped index, unconditionally: a load under a per-element
  // branch is waited for before the next one is issued.
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = row[min(e * 64 + lane, n - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = e * 64 + lane < n ? order_key(x[e]) : 0u;
    lo = min(lo, key[e] ? key[e] : 0xFFFFFFFFu);
    hi = max(hi, key[e]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }

  // Narrow [lo, hi] to the k-th largest key; need = how many keys equal to
  // it are kept. Each pass leaves a range below 2^sh, so sh drops by 8.
  int need = k;
#pragma unroll 1
  for (int pass = 0; pass < 6 && lo < hi; ++pass) {
    const int sh = max(0, 24 - (int)__clz(hi - lo));        // bit length - 8
#pragma unroll
    for (int j = 0; j < 4; ++j) hw[4 * lane + j] = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] >= lo && key[e] <= hi)
        atomicAdd(&hw[(key[e] - lo) >> sh], 1);
    // Lane l reads bins 255 - 4l - j, j = 0..3: counts from the top bin down.
    int c[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = hw[255 - 4 * lane - j];
      tot += c[j];
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    int above = incl - tot, sel_bin = 0, sel_above = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (above < need && need <= above + c[j]) {
        found = true;
        sel_bin = 255 - 4 * lane - j;
        sel_above = above;
      }
      above += c[j];
    }
    const int src = __builtin_ctzll(__ballot(found));        // exactly one lane
    const int bin = __shfl(sel_bin, src), abv = __shfl(sel_above, src);
    need -= abv;
    const uint64_t top = (uint64_t)lo + ((uint64_t)(bin + 1) << sh) - 1;
    lo += (uint32_t)bin << sh;
    hi = top < hi ? (uint32_t)top : hi;
  }
  const uint32_t T = lo;                        // k-th largest key; keep `need` ties

  int32_t *out = job.out + (int64_t)bh * job.out_bh + (int64_t)i * job.out_row;
  int base = 0, ties = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t eqm = __ballot(key[e] == T);
    const bool keep = key[e] > T || (key[e] == T && ties + bits_below(eqm) < need);
    const uint64_t km = __ballot(keep);
    const int pos = base + bits_below(km);
    if (keep && pos < k) out[pos] = e * 64 + lane;           // always: k kept
    base += __builtin_popcountll(km);
    ties += __builtin_popcountll(eqm);
  }
  for (int c = k + lane; c < job.out_row; c += 64) out[c] = -1;
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

// Rows longer than 4096 keys: one workgroup of four waves per row, each
// thread owning a contiguous run of E indices; the same search, with the
// histogram and the scans shared by the workgroup (one wave would hold 128
// keys per lane).
// E = keys per thread (n <= E * kSelThreads).
template <int E>
__global__ __launch_bounds__(kSelThreads) void select_block_kernel(Plan p, SelectJob job) {
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
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = row[min(j0 + e, n - 1)];   // unconditional: see above
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (j0 + e < n) ? order_key(x[e]) : 0u;

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
      if (keep) {
        if (pos < k) out[pos] = j0 + e;                       // always: k kept
        ++pos;
      }
    }
  }
  for (int c = k + t; c < job.out_row; c += kSelThreads) out[c] = -1;
}

}  // namespace
}  // namespace vsa

hipError_t launch_select(const Plan &p, const SelectJob &job, hipStream_t stream) {
  dim3 block(vsa::kSelThreads);
  if (job.max_cols <= 4096) {
    dim3 grid((p.max_vt + vsa::kSelWaves - 1) / vsa::kSelWaves, p.B * p.H);
    if (job.max_cols <= 512)
      hipLaunchKernelGGL(vsa::select_wave_kernel<8>, grid, block, 0, stream, p, job);
    else if (job.max_cols <= 1024)
      hipLaunchKernelGGL(vsa::select_wave_kernel<16>, grid, block, 0, stream, p, job);
    else if (job.max_cols <= 2048)
      hipLaunchKernelGGL(vsa::select_wave_kernel<32>, grid, block, 0, stream, p, job);
    else
      hipLaunchKernelGGL(vsa::select_wave_kernel<64>, grid, block, 0, stream, p, job);
  } else {
    if (job.max_cols > 8192) return hipErrorInvalidValue;
    dim3 grid(p.max_vt, p.B * p.H);
    if (job.max_cols <= 4096)
      hipLaunchKernelGGL(vsa::select_block_kernel<16>, grid, block, 0, stream, p, job);
    else
      hipLaunchKernelGGL(vsa::select_block_kernel<32>, grid, block, 0, stream, p, job);
  }
  return hipGetLastError();
}
