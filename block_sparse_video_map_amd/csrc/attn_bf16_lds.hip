// Step 4 (bf16), LDS-staged variant: the two query-half waves of a key split
// share each 32-key unit of K and V through LDS.
//
// Same work decomposition and math as attn_bf16.hip (one query tile per
// workgroup, eight waves = two query halves x four key splits, transposed
// products, lazy rescale). Difference: a unit's K and V blocks are copied
// from HBM straight into an LDS ring (direct-to-LDS buffer loads, no VGPRs),
// wave qb=0 fetching the K blocks and wave qb=1 the V blocks of their split,
// so every byte crosses L2 once per workgroup instead of once per wave. The
// ring has two slots per split: unit u+1 is in flight while unit u is
// multiplied. One workgroup barrier per unit orders "slot filled" before the
// reads and "slot drained" before it is refilled.
#include <cstdlib>

#include "device_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 4;
constexpr int kThreads = 64 * 2 * kSplits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

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

// s_waitcnt with only the vector-memory counter constrained to zero.
__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_lds_kernel(Plan p, int total, const bf16_bits *__restrict__ qt,
                          const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                          const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                          float scale_log2, bf16_bits *__restrict__ out,
                          float *__restrict__ lse) {
  constexpr int NC = D / 16, NDB = D / 32, LDO = D + 1;
  constexpr int UNIT = 32 * D;                 // elements of K (or V) in a unit
  constexpr int SLOT = 2 * UNIT;               // K then V
  constexpr int RING = kSplits * SLOT;        // one stage: a slot per key split
  static_assert(RING >= kTile * LDO * 2, "epilogue reuses a ring stage");
  // Two stages as separate arrays: a stage is only read while the other one
  // is being filled, and distinct objects let the compiler see that the reads
  // never alias the in-flight copies (so it does not wait for them).
  __shared__ __attribute__((aligned(1024))) bf16_bits ring0[RING];
  __shared__ __attribute__((aligned(1024))) bf16_bits ring1[RING];
  __shared__ float sm_m[kSplits][kTile], sm_l[kSplits][kTile];
  float *osum = reinterpret_cast<float *>(ring0);

  int b, h, tq;
  work_item(p, total, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int qb = wave % 2, ks = wave / 2;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : npt + p.k[s];
  // The key-tile list is read through the constant address space, i.e. with
  // scalar loads that do not share the vector-memory counter with the copies.
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

  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = buffer_load16(rq, voff, tq * TB + (qb * NC + cc) * 1024);
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_use = kNegBig, l_run = 0.f;

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

  // Starts the copy of one unit (tile, key half kb) into `slot` (this wave's
  // half of it: K blocks for qb = 0, V blocks for qb = 1).
  auto issue = [&](bf16_bits *slot, int tile, int kb) {
    if (qb == 0) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (lds_ptr_t)(slot + cc * 512), 16, voff, tile * TB + (kb * NC + cc) * 1024, 0, 0);
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rv, (lds_ptr_t)(slot + UNIT + (db * 2 + jj) * 512), 16, voff,
              tile * TB + (db * 4 + 2 * kb + jj) * 1024, 0, 0);
    }
  };

  // Multiplies the unit held in `slot` (key half kb of the current tile).
  auto compute = [&](const bf16_bits *slot, uint32_t mask32) {
    bf16x8 kf[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kf[cc] = *reinterpret_cast<const bf16x8 *>(slot + cc * 512 + lane * 8);
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) sc = mfma32(kf[cc], qf[cc], sc);
    if (mask32 != 0xFFFFFFFFu) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r / 4) * 8 + g * 4 + (r % 4);
        if (!((mask32 >> key) & 1u)) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    if (__any(mx > m_use + kRescaleSlack)) {
      const float m_new = fmaxf(m_use, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    const float mneg = -m_use;
    bf16x8 pf[2];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, mneg));
      psum += pv;
      pf[r / 8][r % 8] = (__bf16)pv;
    }
    l_run += psum;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8 *>(slot + UNIT + (db * 2 + jj) * 512 + lane * 8);
        o[db] = mfma32(vf, pf[jj], o[db]);
      }
  };

  // Key half 0 of every tile goes through ring0, key half 1 through ring1.
  bf16_bits *slot0 = ring0 + ks * SLOT;
  bf16_bits *slot1 = ring1 + ks * SLOT;
  const int n_pairs = (n_kv + kSplits - 1) / kSplits;   // key split 0 has the most
  // Real-key mask of a tile, from the geometry (no memory access).
  auto tile_mask = [&](int tile, bool ok) -> uint64_t {
    const uint64_t m = __ballot(slot_token(p, s, tile, lane) >= 0);
    return ok ? m : 0ull;
  };
  bool ok_cur = false;
  int tile_cur = 0;
  uint64_t mask_cur = 0;
  if (n_mine > 0) {
    tile_cur = tile_of(0, ok_cur);
    issue(slot0, tile_cur, 0);
    mask_cur = tile_mask(tile_cur, ok_cur);
  }
  for (int i = 0; i < n_pairs; ++i) {
    const bool mine = i < n_mine;
    // Unit 2i: tile i, keys 0..31, in ring0; fill ring1 with keys 32..63.
    wait_vmem_all();
    __syncthreads();
    if (mine) issue(slot1, tile_cur, 1);
    if (mine) compute(slot0, (uint32_t)mask_cur);
    // Unit 2i+1: tile i, keys 32..63, in ring1; fill ring0 with tile i+1.
    bool ok_nxt = false;
    int tile_nxt = 0;
    uint64_t mask_nxt = 0;
    wait_vmem_all();
    __syncthreads();
    if (i + 1 < n_mine) {
      tile_nxt = tile_of(i + 1, ok_nxt);
      issue(slot0, tile_nxt, 0);
      mask_nxt = tile_mask(tile_nxt, ok_nxt);
    }
    if (mine) compute(slot1, (uint32_t)(mask_cur >> 32));
    tile_cur = tile_nxt;
    mask_cur = mask_nxt;
  }
  __syncthreads();

  // Merge the four key splits of each query half (the ring becomes osum).
  {
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (g == 0) {
      sm_m[ks][qb * 32 + l32] = m_use;
      sm_l[ks][qb * 32 + l32] = lt;
    }
  }
  __syncthreads();
  {
    const int q = qb * 32 + l32;
    float M = sm_m[0][q];
#pragma unroll
    for (int w = 1; w < kSplits; ++w) M = fmaxf(M, sm_m[w][q]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kSplits; ++w) L += sm_l[w][q] * __builtin_amdgcn_exp2f(sm_m[w][q] - M);
    const float f = __builtin_amdgcn_exp2f(m_use - M) / L;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= f;
  }
  for (int turn = 0; turn < kSplits; ++turn) {
    if (ks == turn) {
      const int q = qb * 32 + l32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = db * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          if (turn == 0)
            osum[q * LDO + c] = o[db][r];
          else
            osum[q * LDO + c] += o[db][r];
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

hipError_t launch_attn_bf16_lds(const Plan &p, const void *qt, const void *kt, const void *vt,
                                const int32_t *s2t, const int32_t *kv_idx, float scale,
                                void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  const float sl2 = scale * kLog2e;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_bf16_lds_kernel<128>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_lds_kernel<64>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
