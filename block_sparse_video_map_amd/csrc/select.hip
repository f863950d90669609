// Step 3: top-k video key tiles per video query tile.
//
// One workgroup per score row. The row is loaded into LDS as 64-bit keys
// (order-preserving float bits << 32 | ~index), bitonic-sorted descending in
// LDS, so the first k keys are the k best tiles with ties going to the lower
// index. The kept tiles are flagged and compacted in index order with wave
// ballots, which gives the ascending block-index list directly.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSelThreads = 256;

__device__ inline uint64_t sort_key(float x, uint32_t idx) {
  if (x == 0.0f) x = 0.0f;                    // -0.0 ranks equal to +0.0
  uint32_t u = __float_as_uint(x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

template <int PMAX>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Plan p,
                                                             const float *__restrict__ scores,
                                                             int32_t *__restrict__ kv_idx) {
  __shared__ uint64_t keys[PMAX];
  __shared__ uint8_t flag[PMAX];
  __shared__ int wave_cnt[kSelThreads / 64];

  const int i = blockIdx.x, bh = blockIdx.y, h = bh % p.H, s = h % p.n_shapes;
  const int n = p.n_vt[s];
  if (i >= n) return;
  const int k = p.k[s];
  int P2 = 1;
  while (P2 < n) P2 <<= 1;

  const float *row = scores + ((int64_t)bh * p.max_vt + i) * p.max_vt;
  for (int j = threadIdx.x; j < P2; j += kSelThreads) {
    keys[j] = j < n ? sort_key(row[j], (uint32_t)j) : 0ull;
    flag[j] = 0;
  }
  __syncthreads();

  // Bitonic sort, descending.
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < P2 / 2; t += kSelThreads) {
        int lo = 2 * stride * (t / stride) + (t % stride);
        int hi = lo + stride;
        uint64_t a = keys[lo], b = keys[hi];
        bool desc = (lo & size) == 0;
        if (desc ? (a < b) : (a > b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  for (int t = threadIdx.x; t < k; t += kSelThreads)
    flag[0xFFFFFFFFu - (uint32_t)(keys[t] & 0xFFFFFFFFull)] = 1;
  __syncthreads();

  // Ordered compaction of the flagged indices.
  int32_t *out = kv_idx + ((int64_t)bh * p.max_vt + i) * p.k_max;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += kSelThreads) {
    int j = c0 + threadIdx.x;
    bool f = j < n && flag[j];
    uint64_t m = __ballot(f);
    int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (f) out[off + before] = j;
    int total = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) total += wave_cnt[w];
    base += total;
    __syncthreads();
  }
  for (int t = k + threadIdx.x; t < p.k_max; t += kSelThreads) out[t] = -1;
}

}  // namespace
}  // namespace vsa

hipError_t launch_select(const Plan &p, const float *scores, int32_t *kv_idx,
                         hipStream_t stream) {
  dim3 grid(p.max_vt, p.B * p.H);
  dim3 block(vsa::kSelThreads);
  if (p.max_vt <= 1024)
    hipLaunchKernelGGL(vsa::select_kernel<1024>, grid, block, 0, stream, p, scores, kv_idx);
  else if (p.max_vt <= 2048)
    hipLaunchKernelGGL(vsa::select_kernel<2048>, grid, block, 0, stream, p, scores, kv_idx);
  else if (p.max_vt <= 4096)
    hipLaunchKernelGGL(vsa::select_kernel<4096>, grid, block, 0, stream, p, scores, kv_idx);
  else
    hipLaunchKernelGGL(vsa::select_kernel<8192>, grid, block, 0, stream, p, scores, kv_idx);
  return hipGetLastError();
}
