// Step 4 (bf16): tile-skipping flash attention on the 32x32x16 bf16 MFMA.
//
// Work unit: one 64-token query tile per workgroup of four waves. The query
// tile's key-tile list (all prefix tiles, then its kept video tiles; every
// tile for a prefix query tile) is split round-robin over the four waves;
// each wave keeps its own running max, sum and output for all 64 queries and
// the four partial results are merged in LDS at the end.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// every lane owns one query column: the softmax max/sum needs a single
// exchange with lane^32, the rescale of O is one scalar per lane, and the
// accumulator of S^T is already the B operand of the PV product once
// converted to bf16. Q/K tiles are stored in the MFMA operand order and V
// tiles in the matching column order (see the tiled layouts), so every
// operand fetch is a contiguous 1 KB wave load straight into registers.
//
// Workgroups are renumbered so that each of the eight XCDs (which receive
// workgroup ids round-robin) walks a contiguous run of query tiles of the
// same head: neighbouring query tiles keep overlapping key tiles, which then
// hit in that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 load8(const bf16_bits *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// Maps a workgroup id to (b, h, query tile) with XCD-contiguous runs.
__device__ inline void work_item(const Plan &p, int total, int &b, int &h, int &tq) {
  int i = blockIdx.x;
  int q8 = total / 8;
  int L = i < 8 * q8 ? (i % 8) * q8 + i / 8 : i;
  b = (int)(L / p.tiles_per_batch);
  int64_t rem = L % p.tiles_per_batch;
  int cyc = (int)(rem / p.tiles_per_cycle);
  int rem2 = (int)(rem % p.tiles_per_cycle);
  int s = 0;
  while (rem2 >= p.n_tiles[s]) {
    rem2 -= p.n_tiles[s];
    ++s;
  }
  h = cyc * p.n_shapes + s;
  tq = rem2;
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(Plan p, int total, const bf16_bits *__restrict__ qt,
                      const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                      const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                      float scale_log2, bf16_bits *__restrict__ out,
                      float *__restrict__ lse) {
  constexpr int NC = D / 16;   // 16-channel chunks (QK^T reduction steps)
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int LDO = D + 1;
  __shared__ float sm_m[kWaves][kTile], sm_l[kWaves][kTile];
  __shared__ float osum[kTile * LDO];

  int b, h, tq;
  work_item(p, total, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : npt + p.k[s];
  const int32_t *kv_row =
      full_row ? nullptr : kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max;
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;

  // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.
  bf16x8 qf[2][NC];
  {
    const bf16_bits *Q = qt + (head_base + tq) * (kTile * D);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qf[qb][cc] = load8(Q + ((qb * NC + cc) * 64 + lane) * 8);
  }

  float m_run[2] = {kNegBig, kNegBig};
  float l_run[2] = {0.f, 0.f};
  f32x16 o[2][NDB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;

  for (int e = wave; e < n_kv; e += kWaves) {
    int tk = e;
    if (!full_row && e >= npt) {
      const int j = kv_row[e - npt];
      if ((unsigned)j >= (unsigned)p.n_vt[s]) continue;  // not a tile index: ignored
      tk = npt + j;
    }
    const bf16_bits *K = kt + (head_base + tk) * (kTile * D);
    const bf16_bits *V = vt + (head_base + tk) * (kTile * D);
    const uint64_t valid = __ballot(map[tk * kTile + lane] >= 0);

    bf16x8 kf[2][NC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kb][cc] = load8(K + ((kb * NC + cc) * 64 + lane) * 8);
    // S^T[key][query] for key block kb, query block qb.
    f32x16 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc = mfma32(kf[kb][cc], qf[qb][cc], acc);
        sacc[kb][qb] = acc;
      }

    // V is fetched after the QK^T products so that it can reuse K's registers;
    // its latency hides behind the softmax below.
    bf16x8 vf[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) vf[db][j] = load8(V + ((db * 4 + j) * 64 + lane) * 8);

    // Accumulator element r of lane (g, l32) is key kb*32 + (r/4)*8 + g*4 + r%4.
    if (valid != ~0ull) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int key = kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          if (!((valid >> key) & 1ull)) {
            sacc[kb][0][r] = -INFINITY;
            sacc[kb][1][r] = -INFINITY;
          }
        }
    }

    bf16x8 pf[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qb], mx * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][r], scale_log2, -m_new));
          psum += pv;
          sacc[kb][qb][r] = pv;
        }
      l_run[qb] = l_run[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
      // P^T fragment j covers keys 16j..16j+15: accumulator kb = j/2, r = (j%2)*8 + e.
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) pf[qb][j][e8] = (__bf16)sacc[j / 2][qb][(j % 2) * 8 + e8];
    }

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[qb][db] = mfma32(vf[db][j], pf[qb][j], o[qb][db]);
  }

  // Merge the four waves' partial softmax states.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (g == 0) {
      sm_m[wave][qb * 32 + l32] = m_run[qb];
      sm_l[wave][qb * 32 + l32] = lt;
    }
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qb * 32 + l32;
    float M = sm_m[0][q];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][q]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += sm_l[w][q] * __builtin_amdgcn_exp2f(sm_m[w][q] - M);
    const float f = __builtin_amdgcn_exp2f(m_run[qb] - M) / L;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] *= f;
  }
  for (int turn = 0; turn < kWaves; ++turn) {
    if (wave == turn) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qb * 32 + l32;
            const int c = db * 32 + (r / 4) * 8 + g * 4 + (r % 4);
            if (turn == 0)
              osum[q * LDO + c] = o[qb][db][r];
            else
              osum[q * LDO + c] += o[qb][db][r];
          }
    }
    __syncthreads();
  }

  const int32_t *qmap = map + (int64_t)tq * kTile;
  bf16_bits *out_bh = out + (int64_t)bh * p.N * D;
  for (int idx = threadIdx.x; idx < kTile * D / 8; idx += blockDim.x) {
    const int row = idx / (D / 8), ch = idx % (D / 8);
    const int32_t tok = qmap[row];
    if (tok < 0) continue;
    bf16x8 v8;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) v8[e8] = (__bf16)osum[row * LDO + ch * 8 + e8];
    *reinterpret_cast<bf16x8 *>(out_bh + (int64_t)tok * D + ch * 8) = v8;
  }
  if (lse && threadIdx.x < kTile) {
    const int q = threadIdx.x;
    const int32_t tok = qmap[q];
    if (tok >= 0) {
      float M = sm_m[0][q];
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][q]);
      float L = 0.f;
      for (int w = 0; w < kWaves; ++w) L += sm_l[w][q] * __builtin_amdgcn_exp2f(sm_m[w][q] - M);
      lse[(int64_t)bh * p.N + tok] = M * kLn2 + logf(L);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, float scale,
                            void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  const float sl2 = scale * kLog2e;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(total), dim3(256), 0, stream, p, total,
                       (const bf16_bits *)qt, (const bf16_bits *)kt, (const bf16_bits *)vt,
                       s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(total), dim3(256), 0, stream, p, total,
                       (const bf16_bits *)qt, (const bf16_bits *)kt, (const bf16_bits *)vt,
                       s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
