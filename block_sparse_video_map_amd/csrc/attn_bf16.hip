// Step 4 (bf16): tile-skipping flash attention on the 32x32x16 bf16 MFMA.
//
// Work unit: one 64-token query tile per workgroup of eight waves, two per
// SIMD. The tile's key-tile list (all prefix tiles, then its kept video
// tiles; every tile for a prefix query tile) is dealt round-robin to four
// key splits; each split is served by two waves, one per 32-query half.
// Every split keeps its own running max, sum and output; the four are merged
// in LDS at the end. One query tile per CU keeps the key tiles that
// neighbouring query tiles share close together in time, so that they hit
// in the XCD's L2.
//
// The two waves of a split share each K/V tile through LDS: a 32-key half
// ("unit") of a tile is copied from HBM straight into a two-slot LDS ring of
// the split by direct-to-LDS buffer loads (wave 0 copies the K blocks, wave
// 1 the V blocks; no registers held while in flight), one unit ahead of its
// use. Only the two waves of a split wait for each other, once per unit,
// through a pair of LDS counters ("next slot landed", "this slot read by
// both"); the four splits drift freely, so on each SIMD one split's softmax
// (VALU) tends to overlap another split's products (MFMA). A workgroup-wide
// barrier per unit instead keeps all eight waves in step and measured 3.7%
// slower.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// every lane owns one query column: the S^T accumulator is already the B
// operand of the PV product once converted to bf16, and a rescale of O is
// one scalar per lane. Q/K tiles are stored in the MFMA operand order and V
// tiles in the matching column order, so every operand block is a
// contiguous 1 KB wave access.
//
// The running max is an integer in log2 units, raised only when needed: a
// unit's probabilities are formed against the current max, and only when
// some lane's sum over the unit exceeds 2^8 (which any logit more than 8
// above the max causes) is the true row max taken, O and the sum rescaled and
// the unit redone. Row sums are taken over the bf16-rounded probabilities
// that enter the PV product, so numerator and denominator use the same
// weights.
//
// Workgroups are renumbered so that each of the eight XCDs (which receive
// workgroup ids round-robin) walks a contiguous run of query tiles of the
// same head.
#include <cstdlib>

#include "attn_common.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 4;                   // key splits per query tile
constexpr int kWaves = 2 * kSplits;          // two query halves per split
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSumLimit = 256.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(Plan p, int total, const bf16_bits *__restrict__ qt,
                      const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                      const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                      const int32_t *__restrict__ ref_idx, float scale_log2,
                      bf16_bits *__restrict__ out, float *__restrict__ lse) {
  constexpr int NC = D / 16, NDB = D / 32;
  constexpr int UNIT = 32 * D;                 // elements of one unit's K (or V)
  // Two slots, each K then V of one unit. Distinct objects: a slot is only
  // read while the other one is being filled.
  __shared__ __attribute__((aligned(1024))) bf16_bits ring0_all[kSplits * 2 * UNIT];
  __shared__ __attribute__((aligned(1024))) bf16_bits ring1_all[kSplits * 2 * UNIT];
  __shared__ int pair_count[kSplits * 2];      // units finished, per (split, wave)

  int b, h, tq;
  work_item(p, total, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int qb = wave % 2, ks = wave / 2;
  bf16_bits *const ring0 = ring0_all + ks * 2 * UNIT;
  bf16_bits *const ring1 = ring1_all + ks * 2 * UNIT;
  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : video_row_len(p, s);
  // The kept-tile list is read through the constant address space (scalar
  // loads), which keeps it off the vector-memory counter of the copies.
  typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
  const const_i32_ptr kv_row =
      full_row ? nullptr
               : (const_i32_ptr)(kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max);
  const const_i32_ptr ref_row =
      (full_row || p.n_ref == 0)
          ? nullptr
          : (const_i32_ptr)(ref_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_ref);
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;

  constexpr int TB = kTile * D * 2;
  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt + head_base * (kTile * D), head_bytes);
  const int voff = lane * 16;

  bf16x8 qf[NC];              // this wave's Q^T fragments (B operand of S^T = K Q^T)
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = buffer_load16(rq, voff, tq * TB + (qb * NC + cc) * 1024);
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_use = kNegBig, l_run = 0.f;

  // Global tile of the i-th key tile of the row; ok = false for an index
  // outside the head's video tiles (then the tile is fully masked).
  const int n_mine = n_kv > ks ? (n_kv - ks + kSplits - 1) / kSplits : 0;
  auto tile_of = [&](int i, bool &ok) -> int {
    ok = true;
    i = ks + kSplits * i;
    if (full_row) return i;
    const int tile = video_row_tile(p, s, i, kv_row, ref_row);
    if (tile < 0) {
      ok = false;
      return 0;
    }
    return tile;
  };
  // Real-key mask of a tile (bit = slot), ~0 for a full tile.
  auto tile_mask = [&](int tile, bool ok) -> uint64_t {
    if (!ok) return 0ull;
    if (tile_full(p, s, tile)) return ~0ull;
    return __ballot(slot_token(p, s, tile, lane) >= 0);
  };
  // Copy of unit (tile, key half kb) into a slot: wave 0 the K blocks, wave 1
  // the V blocks.
  auto issue = [&](bf16_bits *slot, int tile, int kb) {
    if (qb == 0) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(slot + cc * 512), 16, voff,
                                                 tile * TB + (kb * NC + cc) * 1024, 0, 0);
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
  auto frag = [&](const bf16_bits *slot, int blk) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(slot + blk * 512 + lane * 8);
  };
  // P^T of a unit (bf16) against the running max, and the lane's sum of the
  // rounded probabilities.
  auto probs = [&](const f32x16 &sc, bf16x8 (&pf)[2]) -> float {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[j][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[8 * j + e], scale_log2, -m_use));
      const bf16x8 v = pf[j];
      a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, a1, false);
      a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, a1, false);
    }
    return a0 + a1;
  };
  // One unit from a slot: S^T, the mask of a partly filled tile, softmax
  // (with the rare raise of the max), PV.
  auto unit = [&](const bf16_bits *slot, uint32_t mask32) {
    bf16x8 kf[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) kf[cc] = frag(slot, cc);
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) sc = mfma32(kf[cc], qf[cc], sc);
    __builtin_amdgcn_sched_group_barrier(0x100, NC, 0);   // the NC K fragment reads,
    __builtin_amdgcn_sched_group_barrier(0x008, NC, 0);   // then the NC S^T products
    // The V fragments are read now, so their LDS latency hides behind the
    // softmax instead of stalling each PV product.
    bf16x8 vf[2 * NDB];
#pragma unroll
    for (int j = 0; j < 2 * NDB; ++j) vf[j] = frag(slot + UNIT, j);
    if (mask32 != 0xFFFFFFFFu) {
      // Element r of lane (g, l32) is key (r/4)*8 + g*4 + r%4 of the unit.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k0i = (r / 4) * 8 + g * 4 + (r % 4);
        sc[r] = ((mask32 >> k0i) & 1u) ? sc[r] : -INFINITY;
      }
    }
    bf16x8 pf[2];
    float ps = probs(sc, pf);
    if (__builtin_expect(__any(ps > kSumLimit), 0)) {
      // A logit exceeded the running max by more than the slack: take the
      // unit's true row max (both lane halves), move the max there, redo.
      float m = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, sc[r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                       false, false);
      m = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), m) * scale_log2;
      const float m_new = fmaxf(ceilf(fmaxf(m_use, m)), kNegBig);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_use = m_new;
      ps = probs(sc, pf);
    }
    l_run += ps;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      o[db] = mfma32(vf[db * 2], pf[0], o[db]);
      o[db] = mfma32(vf[db * 2 + 1], pf[1], o[db]);
    }
  };

  // Wait for the other wave of this split to finish its n-th unit, after
  // posting our own: own copies landed and own reads of the old slot done
  // (all counters drained) before the post. The wait is bounded, so it ends
  // even if the partner never posts (which the schedule below rules out).
  typedef volatile __attribute__((address_space(3))) int *lds_iptr;
  const lds_iptr count = (lds_iptr)pair_count;
  auto pair_sync = [&](int n) {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) count[ks * 2 + qb] = n;
    for (int guard = 0; count[ks * 2 + 1 - qb] < n && guard < (1 << 24); ++guard)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  // Unit 2i + kb is key half kb of the split's i-th tile; even units use slot
  // ring0, odd units ring1. The copy of the next unit is issued before the
  // current one is computed. Both waves of a split run the same n_mine steps.
  bool ok = false;
  int t = 0;
  uint64_t mask = 0;
  if (threadIdx.x < kSplits * 2) pair_count[threadIdx.x] = 0;
  if (n_mine > 0) {
    t = tile_of(0, ok);
    mask = tile_mask(t, ok);
    issue(ring0, t, 0);
  }
  sync_slots();
  for (int i = 0; i < n_mine; ++i) {
    issue(ring1, t, 1);
    unit(ring0, (uint32_t)mask);
    pair_sync(2 * i + 1);
    const bool more = i + 1 < n_mine;
    bool ok1 = false;
    int t1 = 0;
    if (more) {
      t1 = tile_of(i + 1, ok1);
      issue(ring0, t1, 0);
    }
    unit(ring1, (uint32_t)(mask >> 32));
    pair_sync(2 * i + 2);
    t = t1;
    mask = more ? tile_mask(t1, ok1) : 0ull;
  }
  __syncthreads();                             // every split done with its rings

  // Merge the four key splits of each query half (the rings are free now).
  float *osum = reinterpret_cast<float *>(ring0_all);       // [64][D], swizzled
  float *sm_m = reinterpret_cast<float *>(ring1_all);       // [kSplits][64]
  float *sm_l = sm_m + kSplits * kTile;
  const int q = qb * 32 + l32;
  {
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (g == 0) {
      sm_m[ks * kTile + q] = m_use;
      sm_l[ks * kTile + q] = lt;
    }
  }
  __syncthreads();
  float M = sm_m[q];
#pragma unroll
  for (int w = 1; w < kSplits; ++w) M = fmaxf(M, sm_m[w * kTile + q]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSplits; ++w) L += sm_l[w * kTile + q] * __builtin_amdgcn_exp2f(sm_m[w * kTile + q] - M);
  const float f = __builtin_amdgcn_exp2f(m_use - M) / L;
  // Element (q, c) of the merged tile sits at q*D + (c ^ (q % 32)).
  for (int turn = 0; turn < kSplits; ++turn) {
    if (ks == turn) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = db * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          float &dst = osum[q * D + (c ^ l32)];
          if (turn == 0)
            dst = o[db][r] * f;
          else
            dst += o[db][r] * f;
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
    for (int e8 = 0; e8 < 8; ++e8) v8[e8] = (__bf16)osum[row * D + ((ch * 8 + e8) ^ (row % 32))];
    *reinterpret_cast<bf16x8 *>(out_bh + (int64_t)tok * D + ch * 8) = v8;
  }
  if (lse && threadIdx.x < kTile) {
    const int qq = threadIdx.x;
    const int32_t tok = qmap[qq];
    if (tok >= 0) {
      float MM = sm_m[qq];
      for (int w = 1; w < kSplits; ++w) MM = fmaxf(MM, sm_m[w * kTile + qq]);
      float LL = 0.f;
      for (int w = 0; w < kSplits; ++w) LL += sm_l[w * kTile + qq] * __builtin_amdgcn_exp2f(sm_m[w * kTile + qq] - MM);
      lse[(int64_t)bh * p.N + tok] = MM * kLn2 + logf(LL);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                            float scale, void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  const float sl2 = scale * kLog2e;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
