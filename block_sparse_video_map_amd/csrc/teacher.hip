// Teacher tile map: full attention max-pooled per (video query tile, video
// key tile) pair, the teacher distribution the tile scorer is measured
// against ("Veda Sparse Attention в ComfyUI", section "Что делает Veda").
//
// Two passes over dense QK^T, one workgroup per (video query tile, batch*head):
//   1. every real query's log-sum-exp over all real keys (prefix and video),
//      online in fp32, base 2, written to a workspace;
//   2. for every video key tile, the largest q.k*scale - lse(q) over the
//      pair's real queries and keys, exponentiated: the largest attention
//      probability of the pair.
// bf16: two waves (one per 32-query half) on the 32x32x16 bf16 MFMA, K
// operands loaded straight from the tiled layout. fp32: one lane per query
// slot with the key tile staged in LDS. A measurement aid, not on the hot
// path.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max over the 64 lanes of a wave.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Real-key bits of a tile (bit = slot).
__device__ inline uint64_t key_mask(const Plan &p, int s, int tile, int lane) {
  return __ballot(slot_token(p, s, tile, lane) >= 0);
}

template <int D, int PASS>
__global__ __launch_bounds__(128) void teacher_bf16_kernel(Plan p, const bf16_bits *qt,
                                                           const bf16_bits *kt,
                                                           const int32_t *s2t, float c2,
                                                           float *lse_ws, float *teacher) {
  constexpr int NC = D / 16;
  constexpr int TB = kTile * D * 2;
  __shared__ float wmax[2];
  const int i = blockIdx.x, bh = blockIdx.y, h = bh % p.H, s = h % p.n_shapes;
  if (i >= p.n_vt[s]) return;
  const int npt = p.n_prefix_tiles, tq = npt + i;
  const int qb = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64, g = lane / 32, l32 = lane % 32;
  const int q = qb * 32 + l32;
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + head_base * (kTile * D), head_bytes);
  const int voff = lane * 16;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;
  const bool qreal = map[(int64_t)tq * kTile + q] >= 0;
  float *lse_row = lse_ws + ((int64_t)bh * p.max_vt + i) * kTile;

  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = buffer_load16(rq, voff, tq * TB + (qb * NC + cc) * 1024);

  // S^T of key half kb of tile t for this wave's queries, pads at -inf, in
  // log2 units. Element r of lane (g, l32) is key (r/4)*8 + g*4 + r%4.
  auto logits = [&](int t, int kb, uint32_t mask32, float (&x)[16]) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      acc = mfma32(buffer_load16(rk, voff, t * TB + (kb * NC + cc) * 1024), qf[cc], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = (r / 4) * 8 + g * 4 + (r % 4);
      x[r] = ((mask32 >> key) & 1u) ? acc[r] * c2 : -INFINITY;
    }
  };

  if (PASS == 1) {
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t < p.n_tiles[s]; ++t) {
      const uint64_t mask = key_mask(p, s, t, lane);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[16];
        logits(t, kb, (uint32_t)(mask >> (32 * kb)), x);
        float mt = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
        const float m_new = fmaxf(m, mt);
        if (m_new == -INFINITY) continue;             // nothing real seen yet
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += exp2f(x[r] - m_new);
        l = l * exp2f(m - m_new) + sum;
        m = m_new;
      }
    }
    // The two lane halves hold different keys of the same query.
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
    const float M = fmaxf(m, mo);
    const float L = (m == -INFINITY ? 0.f : l * exp2f(m - M)) +
                    (mo == -INFINITY ? 0.f : lo * exp2f(mo - M));
    if (g == 0) lse_row[q] = qreal ? M + log2f(L) : INFINITY;
    return;
  }

  const float lq = lse_row[q];                         // +inf for a pad query
  for (int j = 0; j < p.n_vt[s]; ++j) {
    const int t = npt + j;
    const uint64_t mask = key_mask(p, s, t, lane);
    float v = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[16];
      logits(t, kb, (uint32_t)(mask >> (32 * kb)), x);
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, x[r] - lq);
    }
    v = wave_max(v);
    if (lane == 0) wmax[qb] = v;
    __syncthreads();
    if (threadIdx.x == 0)
      teacher[((int64_t)bh * p.max_vt + i) * p.max_vt + j] = exp2f(fmaxf(wmax[0], wmax[1]));
    __syncthreads();
  }
}

template <int D, int PASS>
__global__ __launch_bounds__(64) void teacher_f32_kernel(Plan p, const float *qt,
                                                         const float *kt, const int32_t *s2t,
                                                         float c2, float *lse_ws,
                                                         float *teacher) {
  constexpr int LD = D + 1;
  __shared__ float ks[kTile * LD];
  __shared__ int valid[kTile];
  const int i = blockIdx.x, bh = blockIdx.y, h = bh % p.H, s = h % p.n_shapes;
  if (i >= p.n_vt[s]) return;
  const int npt = p.n_prefix_tiles, tq = npt + i;
  const int lane = threadIdx.x;
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;
  const bool qreal = map[(int64_t)tq * kTile + lane] >= 0;
  float *lse_row = lse_ws + ((int64_t)bh * p.max_vt + i) * kTile;
  float qv[D];
  const float *Q = qt + (head_base + tq) * (kTile * D);
#pragma unroll
  for (int c = 0; c < D; ++c) qv[c] = Q[row_layout_offset(lane, c, D)];

  auto stage = [&](int t) {
    const float *K = kt + (head_base + t) * (kTile * D);
    __syncthreads();
    for (int vec = lane; vec < kTile * D / 8; vec += 64) {
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        int sl, c;
        row_layout_decode(vec, e8, D, sl, c);
        ks[sl * LD + c] = K[vec * 8 + e8];
      }
    }
    valid[lane] = map[(int64_t)t * kTile + lane] >= 0;
    __syncthreads();
  };
  auto logit = [&](int j) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) acc = fmaf(qv[c], ks[j * LD + c], acc);
    return valid[j] ? acc * c2 : -INFINITY;
  };

  if (PASS == 1) {
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t < p.n_tiles[s]; ++t) {
      stage(t);
      for (int j = 0; j < kTile; ++j) {
        const float x = logit(j);
        if (x == -INFINITY) continue;
        const float m_new = fmaxf(m, x);
        l = l * exp2f(m - m_new) + exp2f(x - m_new);
        m = m_new;
      }
    }
    lse_row[lane] = qreal ? m + log2f(l) : INFINITY;
    return;
  }
  const float lq = lse_row[lane];
  for (int jt = 0; jt < p.n_vt[s]; ++jt) {
    stage(npt + jt);
    float v = -INFINITY;
    for (int j = 0; j < kTile; ++j) v = fmaxf(v, logit(j) - lq);
    v = wave_max(v);
    if (lane == 0) teacher[((int64_t)bh * p.max_vt + i) * p.max_vt + jt] = exp2f(v);
  }
}

}  // namespace
}  // namespace vsa

hipError_t launch_teacher(const Plan &p, const void *qt, const void *kt, const int32_t *s2t,
                          float scale, float *lse_ws, float *teacher, hipStream_t stream) {
  const float c2 = scale * vsa::kLog2e;
  dim3 grid(p.max_vt, p.B * p.H);
  if (p.dtype == VSA_BF16) {
    const bf16_bits *q = (const bf16_bits *)qt, *k = (const bf16_bits *)kt;
    if (p.d == 128) {
      hipLaunchKernelGGL((vsa::teacher_bf16_kernel<128, 1>), grid, dim3(128), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
      hipLaunchKernelGGL((vsa::teacher_bf16_kernel<128, 2>), grid, dim3(128), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
    } else {
      hipLaunchKernelGGL((vsa::teacher_bf16_kernel<64, 1>), grid, dim3(128), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
      hipLaunchKernelGGL((vsa::teacher_bf16_kernel<64, 2>), grid, dim3(128), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
    }
  } else {
    const float *q = (const float *)qt, *k = (const float *)kt;
    if (p.d == 128) {
      hipLaunchKernelGGL((vsa::teacher_f32_kernel<128, 1>), grid, dim3(64), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
      hipLaunchKernelGGL((vsa::teacher_f32_kernel<128, 2>), grid, dim3(64), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
    } else {
      hipLaunchKernelGGL((vsa::teacher_f32_kernel<64, 1>), grid, dim3(64), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
      hipLaunchKernelGGL((vsa::teacher_f32_kernel<64, 2>), grid, dim3(64), 0, stream, p, q, k,
                         s2t, c2, lse_ws, teacher);
    }
  }
  return hipGetLastError();
}
