// Matrix-core rate probe: a measurement aid for the rooflines, not part of
// the method. Every wave keeps four independent accumulator chains of the
// same MFMA the attention kernels use (bf16 32x32x16, or the scaled E4M3
// 32x32x64), so the launch's rate is what the chip sustains under a pure
// MFMA load at the clock it settles to (the published peaks assume the
// 2.4 GHz maximum engine clock). Kinds 2 to 4 measure how exponentials
// share a SIMD with the fp8 products, in workgroups of eight waves (two on
// every SIMD, whatever else the CU runs): kind 2 the products alone, kind 3
// the products plus 16 exponentials per trip in every wave, kind 4 four
// waves of products beside four waves of exponentials only, so that each
// SIMD holds one wave of each. Every workgroup also records the span of its
// waves' loops (earliest start, latest end) on the shader tick counter and
// on the constant-rate real-time counter, from which the host reads the
// clock the loops ran at and the cycles a CU spends per trip. The span, not
// one wave's loop, is what counts: a SIMD favours its older wave, so with
// two waves on it the first runs at the full rate while the second waits.
#include "device_common.h"
#include "fp8_layout.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kProbeThreads = 256;

typedef int i32x8p __attribute__((ext_vector_type(8)));

template <int KIND, int THREADS>
__global__ __launch_bounds__(THREADS) void mfma_probe_kernel(int iters, uint64_t *ticks,
                                                            float *sink) {
  __shared__ unsigned long long span[4];   // earliest start, latest end: ticks, real time
  if (threadIdx.x == 0) {
    span[0] = span[2] = ~0ull;
    span[1] = span[3] = 0ull;
  }
  __syncthreads();
  uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const bool products = KIND != 4 || wave < 4;
  const bool exps = KIND == 3 || (KIND == 4 && wave >= 4);
  float x[8];                 // eight independent exponential chains in (-1, 0)
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -0.01f * (float)(lane + j);
  if (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)(lane + e));
      b[e] = (__bf16)(0.002f * (float)(lane - e));
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  } else {
    i32x8p a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 ^ (lane & 7);
      b[e] = 0x30303030 ^ (e & 3);
    }
    for (int i = 0; i < iters; ++i) {
      if (products) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0,
                                                                   kFp8ExpBias, 0, kFp8ExpBias);
      }
      if (exps) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e % 8] = -__builtin_amdgcn_exp2f(x[e % 8]);
      }
    }
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[j][r];
#pragma unroll
  for (int j = 0; j < 8; ++j) t += x[j];
  uint64_t t1 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    atomicMin(&span[0], (unsigned long long)t0);
    atomicMax(&span[1], (unsigned long long)t1);
    atomicMin(&span[2], (unsigned long long)r0);
    atomicMax(&span[3], (unsigned long long)r1);
  }
  __syncthreads();
  if (ticks && threadIdx.x == 0) {
    uint64_t *o = ticks + 4 * (size_t)blockIdx.x;
    o[0] = span[0];
    o[1] = span[1];
    o[2] = span[2];
    o[3] = span[3];
  }
  if (t == 1234.5f && sink) sink[0] = t;  // keeps the products live; sink is null
}

}  // namespace
}  // namespace vsa

hipError_t launch_mfma_probe(int kind, int iters, int n_workgroups, uint64_t *ticks,
                             hipStream_t stream) {
  float *sink = nullptr;
  const dim3 grid(n_workgroups), block(vsa::kProbeThreads);
  switch (kind) {
    case 0:
      hipLaunchKernelGGL((vsa::mfma_probe_kernel<0, vsa::kProbeThreads>), grid, block, 0, stream,
                         iters, ticks, sink);
      break;
    case 1:
      hipLaunchKernelGGL((vsa::mfma_probe_kernel<1, vsa::kProbeThreads>), grid, block, 0, stream,
                         iters, ticks, sink);
      break;
    case 2:
      hipLaunchKernelGGL((vsa::mfma_probe_kernel<2, 2 * vsa::kProbeThreads>), grid,
                         dim3(2 * vsa::kProbeThreads), 0, stream, iters, ticks, sink);
      break;
    case 3:
      hipLaunchKernelGGL((vsa::mfma_probe_kernel<3, 2 * vsa::kProbeThreads>), grid,
                         dim3(2 * vsa::kProbeThreads), 0, stream, iters, ticks, sink);
      break;
    default:
      hipLaunchKernelGGL((vsa::mfma_probe_kernel<4, 2 * vsa::kProbeThreads>), grid,
                         dim3(2 * vsa::kProbeThreads), 0, stream, iters, ticks, sink);
      break;
  }
  return hipGetLastError();
}
