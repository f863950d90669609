// Step 4 (bf16): tile-skipping flash attention on the 32x32x16 bf16 MFMA.
//
// Work unit: one 64-token query tile per workgroup of four waves, one wave
// per SIMD. The query tile's key-tile list (all prefix tiles, then its kept
// video tiles; every tile for a prefix query tile) is dealt round-robin to
// the four waves ("key splits"); every wave holds all 64 queries, so each
// K/V byte it fetches serves 64 queries (no wave fetches what another one
// fetches). Each wave keeps its own running max, sum and output; the four
// splits are merged in LDS at the end.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// every lane owns one query column: the softmax max needs a single exchange
// between the two 32-lane halves (v_permlane32_swap), the rescale of O is one
// scalar per lane, and the accumulator of S^T is already the B operand of the
// PV product once converted to bf16. Q/K tiles are stored in the MFMA operand
// order and V tiles in the matching column order (see the tiled layouts), so
// every operand fetch is a contiguous 1 KB wave load straight into registers
// through a buffer resource whose tile offset stays in scalar registers.
//
// A wave walks its key tiles in 32-key halves ("units"); K and V of a unit
// are fetched two units ahead into double buffers, and S of unit u+1 is
// computed before the softmax of unit u. The running max is an integer in
// log2 units and is only raised when a row max exceeds it by more than 2^8
// (then O and the sum are rescaled); the stale max is exact because O and
// the sum share it.
//
// Workgroups are renumbered so that each of the eight XCDs (which receive
// workgroup ids round-robin) walks a contiguous run of query tiles of the
// same head: neighbouring query tiles keep overlapping key tiles, which then
// hit in that XCD's L2.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 4;
constexpr int kThreads = 64 * kSplits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(Plan p, int total, const bf16_bits *__restrict__ qt,
                      const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                      const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                      float scale_log2, bf16_bits *__restrict__ out,
                      float *__restrict__ lse) {
  constexpr int NC = D / 16, NDB = D / 32, LDO = D + 1;
  __shared__ float sm_m[kSplits][kTile], sm_l[kSplits][kTile];
  __shared__ float osum[kTile * LDO];

  int b, h, tq;
  work_item(p, total, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : npt + p.k[s];
  typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
  const const_i32_ptr kv_row =
      full_row ? nullptr
               : (const_i32_ptr)(kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max);
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;
  const int n_mine = n_kv > ks ? (n_kv - ks + kSplits - 1) / kSplits : 0;

  constexpr int TB = kTile * D * 2;
  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt + head_base * (kTile * D), head_bytes);
  const int voff = lane * 16;

bf16x8 qf[2][NC];           // Q^T fragments (B operand of S^T = K Q^T)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      qf[qb][cc] = buffer_load16(rq, voff, tq * TB + (qb * NC + cc) * 1024);
  bf16x8 kbuf[2][NC], vbuf[2][NDB][2];
  f32x16 sbuf[2][2];          // [unit parity][qb]
  f32x16 o[2][NDB];
  float m_use[2] = {kNegBig, kNegBig}, l_run[2] = {0.f, 0.f};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;

  auto tile_of = [&](int i, bool &ok) -> int {
    const int e = ks + kSplits * i;
    ok = true;
    if (full_row || e < npt) return e;
    const int j = kv_row[e - npt];
    if ((unsigned)j >= (unsigned)p.n_vt[s]) {
      ok = false;
      return 0;
    }
    return npt + j;
  };
  auto tile_mask = [&](int tile, bool ok) -> uint64_t {
    const uint64_t m = __ballot(slot_token(p, s, tile, lane) >= 0);
    return ok ? m : 0ull;
  };
  auto load_k = [&](int buf, int tile, int kb) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kbuf[buf][cc] = buffer_load16(rk, voff, tile * TB + (kb * NC + cc) * 1024);
  };
  auto load_v = [&](int buf, int tile, int kb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        vbuf[buf][db][jj] = buffer_load16(rv, voff, tile * TB + (db * 4 + 2 * kb + jj) * 1024);
  };
  auto qk = [&](int buf, f32x16 (&acc)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) acc[qb] = mfma32(kbuf[buf][cc], qf[qb][cc], acc[qb]);
    }
  };
  auto apply_mask = [&](f32x16 (&sc)[2], uint32_t mask32) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k0 = (r / 4) * 8 + (r % 4);
      const bool keep = g ? ((mask32 >> (k0 + 4)) & 1u) : ((mask32 >> k0) & 1u);
      sc[0][r] = keep ? sc[0][r] : -INFINITY;
      sc[1][r] = keep ? sc[1][r] : -INFINITY;
    }
  };
  auto exp_unit = [&](const f32x16 &sc, float mref, bf16x8 (&pf)[2], float &psum, float &mx) {
    float m4[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      m4[a] = fmaxf(fmaxf(sc[4 * a], sc[4 * a + 1]), fmaxf(sc[4 * a + 2], sc[4 * a + 3]));
    mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), mx) * scale_log2;
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -mref));
    float s8[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) s8[a] = pv[2 * a] + pv[2 * a + 1];
    psum = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r / 8][r % 8] = (__bf16)pv[r];
  };
  // Softmax of one unit (S^T in sc) and its PV product with V buffer vb.
  auto step = [&](f32x16 (&sc)[2], int vb) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      bf16x8 pf[2];
      float psum, mx;
      exp_unit(sc[qb], m_use[qb], pf, psum, mx);
      if (__any(mx > m_use[qb] + kRescaleSlack)) {
        const float m_new = ceilf(fmaxf(m_use[qb], mx));
        const float alpha = __builtin_amdgcn_exp2f(m_use[qb] - m_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        m_use[qb] = m_new;
        float unused;
        exp_unit(sc[qb], m_new, pf, psum, unused);
      }
      l_run[qb] += psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) o[qb][db] = mfma32(vbuf[vb][db][jj], pf[jj], o[qb][db]);
    }
  };

  if (n_mine > 0) {
    // Unit u = 2i + kb: key half kb of the wave's i-th tile, K in kbuf[u%2]
    // and V in vbuf[u%2], both fetched two units ahead.
    bool ok0, ok1 = false;
    int t0 = tile_of(0, ok0), t1 = 0;
    if (n_mine > 1) t1 = tile_of(1, ok1);
    uint64_t mask0 = tile_mask(t0, ok0), mask1 = 0;
    load_k(0, t0, 0);
    load_v(0, t0, 0);
    load_k(1, t0, 1);
    load_v(1, t0, 1);
    qk(0, sbuf[0]);
    if (n_mine > 1) load_k(0, t1, 0);
    for (int i = 0; i < n_mine; ++i) {
      const bool more = i + 1 < n_mine;
      if (more) mask1 = tile_mask(t1, ok1);
      // unit 2i
      qk(1, sbuf[1]);                                 // S of unit 2i+1
      if (more) load_k(1, t1, 1);                     // K of unit 2i+3
      if ((uint32_t)mask0 != 0xFFFFFFFFu) apply_mask(sbuf[0], (uint32_t)mask0);
      step(sbuf[0], 0);
      if (more) load_v(0, t1, 0);                     // V of unit 2i+2
      // unit 2i+1
      if (more) qk(0, sbuf[0]);                       // S of unit 2i+2
      bool ok2 = false;
      int t2 = 0;
      if (i + 2 < n_mine) {
        t2 = tile_of(i + 2, ok2);
        load_k(0, t2, 0);                             // K of unit 2i+4
      }
      if ((uint32_t)(mask0 >> 32) != 0xFFFFFFFFu) apply_mask(sbuf[1], (uint32_t)(mask0 >> 32));
      step(sbuf[1], 1);
      if (more) load_v(1, t1, 1);                     // V of unit 2i+3
      t0 = t1;
      mask0 = mask1;
      t1 = t2;
      ok1 = ok2;
    }
  }

  // Merge the four key splits.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    if (g == 0) {
      sm_m[ks][qb * 32 + l32] = m_use[qb];
      sm_l[ks][qb * 32 + l32] = lt;
    }
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = qb * 32 + l32;
    float M = sm_m[0][q];
#pragma unroll
    for (int w = 1; w < kSplits; ++w) M = fmaxf(M, sm_m[w][q]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kSplits; ++w) L += sm_l[w][q] * __builtin_amdgcn_exp2f(sm_m[w][q] - M);
    const float f = __builtin_amdgcn_exp2f(m_use[qb] - M) / L;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] *= f;
  }
  for (int turn = 0; turn < kSplits; ++turn) {
    if (ks == turn) {
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
      for (int w = 1; w < kSplits; ++w) M = fmaxf(M, sm_m[w][q]);
      float L = 0.f;
      for (int w = 0; w < kSplits; ++w) L += sm_l[w][q] * __builtin_amdgcn_exp2f(sm_m[w][q] - M);
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
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
