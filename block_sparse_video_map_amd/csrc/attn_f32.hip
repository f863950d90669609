// Step 4 (fp32): tile-skipping attention in fp32 throughout.
//
// The precise path: one wave per query tile, one lane per query slot. Each
// allowed key tile is staged in LDS (unpacked from the tiled layouts), the
// lane computes its 64 logits with fp32 FMAs and folds them into a running
// max/sum/output with the exact expf. Same key-tile lists as the bf16 path.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(Plan p, const float *__restrict__ qt,
                                                      const float *__restrict__ kt,
                                                      const float *__restrict__ vt,
                                                      const int32_t *__restrict__ s2t,
                                                      const int32_t *__restrict__ kv_idx,
                                                      const int32_t *__restrict__ ref_idx,
                                                      float scale, float *__restrict__ out,
                                                      float *__restrict__ lse) {
  constexpr int LD = D + 1;
  __shared__ float ks[kTile * LD], vs[kTile * LD];
  __shared__ int valid[kTile];

  // Work item: blockIdx.x enumerates (b, h, query tile) in head order.
  const int64_t L = blockIdx.x;
  const int b = (int)(L / p.tiles_per_batch);
  int64_t rem = L % p.tiles_per_batch;
  const int cyc = (int)(rem / p.tiles_per_cycle);
  int rem2 = (int)(rem % p.tiles_per_cycle);
  int s = 0;
  while (rem2 >= p.n_tiles[s]) {
    rem2 -= p.n_tiles[s];
    ++s;
  }
  const int h = cyc * p.n_shapes + s, tq = rem2, bh = b * p.H + h;
  const int lane = threadIdx.x;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : video_row_len(p, s);
  const int32_t *kv_row =
      full_row ? nullptr : kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max;
  const int32_t *ref_row = (full_row || p.n_ref == 0)
                               ? nullptr
                               : ref_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_ref;
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;

  float q[D], o[D];
  const float *Q = qt + (head_base + tq) * (kTile * D);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = Q[row_layout_offset(lane, c, D)];
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int e = 0; e < n_kv; ++e) {
    int tk = e;
    if (!full_row) {
      tk = video_row_tile(p, s, e, kv_row, ref_row);
      if (tk < 0) continue;                              // not a tile index: ignored
    }
    const float *K = kt + (head_base + tk) * (kTile * D);
    const float *V = vt + (head_base + tk) * (kTile * D);
    __syncthreads();
    for (int vec = lane; vec < kTile * D / 8; vec += 64) {
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        int sl, c;
        row_layout_decode(vec, e8, D, sl, c);
        ks[sl * LD + c] = K[vec * 8 + e8];
        col_layout_decode(vec, e8, D, sl, c);
        vs[sl * LD + c] = V[vec * 8 + e8];
      }
    }
    valid[lane] = map[tk * kTile + lane] >= 0;
    __syncthreads();

    float sc[kTile];
    float mt = -INFINITY;
    for (int j = 0; j < kTile; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(q[c], ks[j * LD + c], acc);
      sc[j] = valid[j] ? acc * scale : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
    for (int j = 0; j < kTile; ++j) {
      if (!valid[j]) continue;
      const float pj = expf(sc[j] - m_new);
      l += pj;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(pj, vs[j * LD + c], o[c]);
    }
    m = m_new;
  }

  const int32_t tok = map[(int64_t)tq * kTile + lane];
  if (tok >= 0) {
    float *orow = out + ((int64_t)bh * p.N + tok) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
    if (lse) lse[(int64_t)bh * p.N + tok] = m + logf(l);
  }
}

}  // namespace

hipError_t launch_attn_f32(const Plan &p, const void *qt, const void *kt, const void *vt,
                           const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                           float scale,
                           void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  if (p.d == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(total), dim3(64), 0, stream, p,
                       (const float *)qt, (const float *)kt, (const float *)vt, s2t, kv_idx, ref_idx,
                       scale, (float *)out, lse);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(total), dim3(64), 0, stream, p,
                       (const float *)qt, (const float *)kt, (const float *)vt, s2t, kv_idx, ref_idx,
                       scale, (float *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
