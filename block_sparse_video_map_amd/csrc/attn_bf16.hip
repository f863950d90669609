// Step 4 (bf16): tile-skipping flash attention on the 32x32x16 bf16 MFMA.
//
// Work unit: a workgroup of eight waves takes two neighbouring query tiles
// of one head, with their key lists cut into 32-key units and merged into
// shared and paired steps (attn_pairs.h). Every wave therefore has work in
// every step, and each K/V byte a shared step copies serves both tiles
// (neighbouring tiles share most of their kept tiles). Steps are dealt
// round-robin to two key splits; a split is four waves (two tiles x two
// 32-query halves), one per SIMD, and the two splits put different query
// halves on each SIMD.
//
// A split's K and V go through two-slot LDS rings filled by direct-to-LDS
// buffer loads (each of the four waves copies its share; no registers held
// while in flight): K two steps ahead of use, V one. The four waves wait for
// each other once per step through LDS counters; the wait is bounded, and a
// wave that gives up makes the workgroup write NaN. The step lists are built
// once per workgroup in LDS, so the loop reads one entry per step.
//
// Each wave owns 32 query columns: S^T = K Q^T and O^T = V^T P^T, so the S^T
// accumulator is already the B operand of the PV product once converted to
// bf16, and a rescale of O is one scalar per lane. A step issues its sixteen
// MFMAs in a fixed order (the PV product of the previous step interleaved
// with the S^T product of the next) with the softmax of the current step
// spread between them, so one wave keeps the matrix pipe busy while it
// computes exponentials.
//
// The running max is an integer in log2 units, raised only when needed: a
// unit's probabilities are formed against the current max, and only when
// some lane's sum over the unit exceeds 2^8 (which any logit more than 8
// above the max causes) is the true column max taken, O and the sum rescaled
// and the unit redone. Row sums are taken over the bf16-rounded
// probabilities that enter the PV product.
//
// Workgroups are renumbered so that each of the eight XCDs (which receive
// workgroup ids round-robin) walks a contiguous run of query-tile pairs.
#include <cstdlib>

#include "attn_common.h"
#include "attn_pairs.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 2;                       // key splits per workgroup
constexpr int kWaves = 8;                        // splits x two tiles x two query halves
constexpr int kThreads = 64 * kWaves;
using pairs::kNone;
using pairs::kRowCap;
using pairs::PairGrid;
constexpr int kStepCap = 4 * kRowCap;            // steps per chunk
constexpr int kStepStride = kStepCap / kSplits;  // steps per split
constexpr int kChunkTiles = kStepCap / 2;        // key tiles per chunk of a shared list
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSumLimit = 256.0f;
constexpr int kGuard = 1 << 20;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Four consecutive 1 KiB blocks to LDS; one LDS base (M0) and one global
// offset, the instruction offset moving both alike.
__device__ inline void copy4k(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 1024, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 2048, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 3072, 0);
}
__device__ inline void copy2k(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 1024, 0);
}

// Softmax probabilities of one unit against the running max m (log2 units),
// rounded to bf16 (the B operand of the PV product), and this lane's sum of
// the rounded values.
__device__ __forceinline__ float unit_probs(const f32x16 &sc, float scale_log2, float m,
                                            bf16x8 &p0, bf16x8 &p1) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; ++e) p0[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[e], scale_log2, -m));
#pragma unroll
  for (int e = 0; e < 8; ++e)
    p1[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[8 + e], scale_log2, -m));
  float a0 = 0.f, a1 = 0.f;
  a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 0, 1), ones, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 2, 3), ones, a1, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 4, 5), ones, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p0, p0, 6, 7), ones, a1, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 0, 1), ones, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 2, 3), ones, a1, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 4, 5), ones, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p1, p1, 6, 7), ones, a1, false);
  return a0 + a1;
}

// Largest element of a query column over the unit's 32 keys (both lane halves).
__device__ __forceinline__ float column_max(const f32x16 &sc) {
  float m = sc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, sc[r]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                   false, false);
  return fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), m);
}

// Real-key mask (bit = slot within the unit) of unit entry e; 0 for no unit.
__device__ __forceinline__ uint32_t unit_mask(const Plan &p, int s, uint32_t e, int l32) {
  if (e == kNone) return 0u;
  const int tile = (int)((e & 0x7FFF) >> 1), kb = (int)(e & 1);
  return (uint32_t)__ballot(slot_token(p, s, tile, kb * 32 + l32) >= 0);
}

// Element r of lane (g, l32) of an S^T block is key (r/4)*8 + g*4 + r%4.
__device__ __forceinline__ void mask_keys(f32x16 &sc, uint32_t m32, int g) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int k0i = (r / 4) * 8 + g * 4 + (r % 4);
    sc[r] = ((m32 >> k0i) & 1u) ? sc[r] : -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(Plan p, PairGrid gd, const bf16_bits *__restrict__ qt,
                      const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                      const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                      const int32_t *__restrict__ ref_idx, float scale_log2,
                      bf16_bits *__restrict__ out, float *__restrict__ lse) {
  constexpr int NC = D / 16, NDB = D / 32;
  constexpr int UNIT = 32 * D;                 // elements of one unit's K (or V)
  constexpr int UB = UNIT * 2;                 // its bytes
  constexpr int TB = kTile * D * 2;            // bytes of one tile
  constexpr int SLOT = 2 * UNIT;               // a split's slot: two units (tile A, tile B)
  // Issue slots of a step: its 2*NDB + NC MFMAs, at least one per softmax
  // chunk (sixteen chunks: one element pair every two slots).
  constexpr int kSlots = 2 * NDB + NC > 16 ? 2 * NDB + NC : 16;
  // Four distinct slot arrays (K and V, two slots each), so that reads of one
  // slot never wait for copies landing in another.
  __shared__ __attribute__((aligned(1024))) bf16_bits kslot0[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) bf16_bits kslot1[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) bf16_bits vslot0[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) bf16_bits vslot1[kSplits * SLOT];
  __shared__ uint32_t steps[kStepCap];
  __shared__ uint32_t ulA[2 * kRowCap];
  __shared__ uint16_t bx[2 * kRowCap];
  __shared__ __attribute__((aligned(16))) int grp_count[kSplits * 4];
  __shared__ int scan[2 * kWaves];
  __shared__ int fault;

  int b, h, tA, tB;
  pairs::pair_item(p, gd, b, h, tA, tB);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  // Split 1 takes the roles with the query halves swapped, so that the two
  // waves of each SIMD (w and w + 4) hold different halves: where a tile's
  // second half is all pads (its waves skip their products), every SIMD
  // still has a computing wave.
  const int sp = wave / 4, role = (wave % 4) ^ sp;   // split; role = tile*2 + query half
  const int tb = role / 2, qb = role % 2;
  const int myT = tb ? tB : tA;
  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool fullA = p.dense || tA < npt;
  const bool merge = tB >= 0 && !fullA;         // two video rows with their own lists
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;
  auto kv_row_of = [&](int t) {
    return kv_idx + ((int64_t)bh * p.max_vt + (t - npt)) * p.k_max;
  };
  auto ref_row_of = [&](int t) -> const int32_t * {
    return p.n_ref == 0 ? nullptr : ref_idx + ((int64_t)bh * p.max_vt + (t - npt)) * p.k_ref;
  };

  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt + head_base * (kTile * D), head_bytes);
  const int voff = lane * 16;

  if (threadIdx.x < kSplits * 4) grp_count[threadIdx.x] = 0;
  if (threadIdx.x == 0) fault = 0;
  // A wave whose tile has no unit in a paired step (entry kNone) still runs
  // its PV products, with every probability zero, on its tile's half of the
  // V slot, which this kernel may not have written yet. LDS keeps what an
  // earlier kernel left there, possibly NaN or Inf bit patterns, and
  // 0 * NaN = NaN; so the V rings start zeroed (whatever the kernel writes
  // there later is a finite V row). The barriers of the list building order
  // these stores before the first copy into the rings.
  {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 *v0 = reinterpret_cast<u32x4 *>(vslot0), *v1 = reinterpret_cast<u32x4 *>(vslot1);
    for (int x = threadIdx.x; x < kSplits * SLOT / 8; x += kThreads) {
      v0[x] = z;
      v1[x] = z;
    }
  }

  bf16x8 qf[NC];
  const int qtile = myT >= 0 ? myT : tA;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    qf[cc] = buffer_load16(rq, voff, qtile * TB + (qb * NC + cc) * 1024);
  const bool q_live = myT >= 0 && __any(map[(int64_t)myT * kTile + qb * 32 + l32] >= 0);
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_use = kNegBig, l_run = 0.f;
  bool stalled = false;
  int sync_n = 0;

  // The four waves of a split wait for each other once per step (LDS
  // counters); bounded, and a wave that gives up poisons the outputs.
  typedef volatile __attribute__((address_space(3))) int *lds_iptr;
  typedef volatile __attribute__((address_space(3))) i32x4 *lds_i4ptr;
  const lds_iptr count = (lds_iptr)grp_count;
  const lds_i4ptr count4 = (lds_i4ptr)(grp_count + sp * 4);
  auto grp_sync = [&]() {
    ++sync_n;
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (lane == 0) count[sp * 4 + role] = sync_n;
    if (stalled) return;
    int guard = 0;
    for (;;) {
      const i32x4 c = *count4;
      if (min(min(c.x, c.y), min(c.z, c.w)) >= sync_n) break;
      if (++guard > kGuard) {
        stalled = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
  };

  // ---- step lists (attn_pairs.h): 32-key units, step j to split j % 2.
  // The merged build keeps its tile bitmaps in the K slots before any copy.
  const pairs::ListSmem lsm{steps, ulA, bx, scan, reinterpret_cast<uint32_t *>(kslot0)};

  const uint32_t *mysteps = steps + sp * kStepStride;
  auto step_at = [&](int j) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(mysteps[j]);
  };
  auto my_unit = [&](uint32_t st) -> uint32_t { return tb ? (st >> 16) : (st & 0xFFFFu); };
  auto is_shared = [&](uint32_t st) -> bool { return (st & 0xFFFFu) == (st >> 16); };
  // This wave's share of the copies of a step. Shared unit: roles 0 and 1
  // copy the two halves of K, roles 2 and 3 the two halves of V. Separate
  // units: role 0 copies A's K, role 1 A's V, role 2 B's K, role 3 B's V
  // (A's unit at offset 0 of the slot, B's at UNIT).
  // The split's offset into the slot arrays goes through an empty asm, so
  // that each copy's LDS base is one scalar add per step. Otherwise the
  // compiler keeps one base per slot, role and block live across the loop;
  // they spill, and every step reads them back with VALU instructions.
  auto issue_k = [&](uint32_t st, bf16_bits *slot_all) __attribute__((always_inline)) {
    int sbase = sp * SLOT;
    asm volatile("" : "+s"(sbase));
    bf16_bits *dst = slot_all + sbase;
    const uint32_t eA = st & 0xFFFFu, eB = st >> 16;
    if (eA == eB) {
      if (role < 2 && eA != kNone) {
        const int tile = (int)((eA & 0x7FFF) >> 1), kb = (int)(eA & 1);
#pragma unroll
        for (int g4 = 0; g4 < NC / 8; ++g4)
          copy4k(rk, (lds_ptr_t)(dst + (role * (NC / 8) + g4) * 2048), voff,
                 tile * TB + kb * UB + (role * (NC / 8) + g4) * 4096);
        if (NC / 8 == 0 && role == 0)            // d = 64: one 4 KiB half
          copy4k(rk, (lds_ptr_t)dst, voff, tile * TB + kb * UB);
      }
    } else if (role == 0 || role == 2) {
      const uint32_t e = (st >> (8 * role)) & 0xFFFFu;
      if (e != kNone) {
        const int tile = (int)((e & 0x7FFF) >> 1), kb = (int)(e & 1);
        bf16_bits *d2 = dst + (role / 2) * UNIT;
#pragma unroll
        for (int g4 = 0; g4 < NC / 4; ++g4)
          copy4k(rk, (lds_ptr_t)(d2 + g4 * 2048), voff, tile * TB + kb * UB + g4 * 4096);
      }
    }
  };
  auto issue_v = [&](uint32_t st, bf16_bits *slot_all) __attribute__((always_inline)) {
    int sbase = sp * SLOT;
    asm volatile("" : "+s"(sbase));
    bf16_bits *dst = slot_all + sbase;
    const uint32_t eA = st & 0xFFFFu, eB = st >> 16;
    if (eA == eB) {
      if (role >= 2 && eA != kNone) {
        const int tile = (int)((eA & 0x7FFF) >> 1), kb = (int)(eA & 1);
#pragma unroll
        for (int dd = 0; dd < NDB / 2; ++dd) {
          const int db = (role - 2) * (NDB / 2) + dd;
          copy2k(rv, (lds_ptr_t)(dst + db * 1024), voff, tile * TB + db * 4096 + kb * 2048);
        }
      }
    } else if (role == 1 || role == 3) {
      const uint32_t e = (st >> (8 * (role - 1))) & 0xFFFFu;
      if (e != kNone) {
        const int tile = (int)((e & 0x7FFF) >> 1), kb = (int)(e & 1);
        bf16_bits *d2 = dst + (role / 2) * UNIT;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          copy2k(rv, (lds_ptr_t)(d2 + db * 1024), voff, tile * TB + db * 4096 + kb * 2048);
      }
    }
  };
  auto frag = [&](const bf16_bits *slot_all, int off, int blk) __attribute__((always_inline))
      -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(slot_all + sp * SLOT + off + blk * 512 + lane * 8);
  };
  // Offset of this wave's unit in a step's slot.
  auto unit_off = [&](uint32_t st) -> int { return is_shared(st) ? 0 : tb * UNIT; };

  const int n_rows = merge ? 1 : (fullA ? p.n_tiles[s] : video_row_len(p, s));
  const int chunk = merge ? n_rows : kChunkTiles;
  for (int e0 = 0; e0 < n_rows; e0 += chunk) {
    const int nS =
        merge ? pairs::build_merged<2, kWaves, kSplits, kStepStride>(
                    p, s, kv_row_of(tA), ref_row_of(tA), kv_row_of(tB), ref_row_of(tB), lsm)
              : pairs::build_shared<2, kWaves, kSplits, kStepStride>(
                    p, s, fullA, fullA ? nullptr : kv_row_of(tA), fullA ? nullptr : ref_row_of(tA),
                    e0, min(n_rows, e0 + chunk), lsm);
    const int n_u = nS > sp ? (nS - sp + kSplits - 1) / kSplits : 0;
    if (n_u > 0) {
      // Step u: K in slot u%2 of the K slots, V in slot u%2 of the V slots.
      // Step u issues K of step u+2 and V of step u+1, reads K of step u+1
      // and V of step u, takes the PV product of step u-1, S of step u+1
      // with the softmax of step u, and ends with the group wait.
      uint32_t st0 = step_at(0);
      uint32_t st1 = n_u > 1 ? step_at(1) : kNone | (kNone << 16);
      uint32_t st2 = n_u > 2 ? step_at(2) : kNone | (kNone << 16);
      issue_k(st0, kslot0);
      if (n_u > 1) issue_k(st1, kslot1);
      issue_v(st0, vslot0);
      grp_sync();
      bf16x8 p0, p1;
      f32x16 sc;
      const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
      bf16x8 vf[2 * NDB];
      if (q_live) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int off = unit_off(st0);
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc = mfma32(frag(kslot0, off, cc), qf[cc], acc);
        sc = acc;
        const uint32_t me = my_unit(st0);
        if (me & 0x8000) mask_keys(sc, unit_mask(p, s, me, l32), g);
        if (m_use == kNegBig) m_use = fmaxf(ceilf(column_max(sc) * scale_log2), kNegBig);
#pragma unroll
        for (int j = 0; j < 2 * NDB; ++j)
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) vf[j][e8] = (__bf16)0.f;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) p0[e8] = p1[e8] = (__bf16)0.f;
      }
      grp_sync();
// One step with a next step: KR/VR the slots read (K of step u+1, V of step
// u), KW/VW the slots refilled (K of step u+2, V of step u+1). st0/st1/st2:
// the entries of steps u, u+1, u+2.
#define VSA_STEP(KR, VR, KW, VW)                                                          \
  {                                                                                       \
    if (u + 2 < n_u) issue_k(st2, KW);                                                    \
    issue_v(st1, VW);                                                                     \
    const uint32_t pend = mysteps[min(u + 3, n_u - 1)];                                   \
    if (q_live) {                                                                         \
      const int koff = unit_off(st1), voff2 = unit_off(st0);                              \
      bf16x8 kf[NC];                                                                      \
      _Pragma("unroll") for (int cc = 0; cc < NC; ++cc) kf[cc] = frag(KR, koff, cc);      \
      f32x16 sn;                                                                          \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) sn[r] = 0.f;                         \
      float tt[16];                                                                       \
      bf16x2 pk[8];                                                                       \
      float a0 = 0.f, a1 = 0.f;                                                           \
      __builtin_amdgcn_sched_barrier(0);                                                  \
      _Pragma("unroll") for (int i = 0; i < kSlots; ++i) {                                \
        const int n_pv = 2 * NDB;                                                         \
        const bool is_s = (i < 2) ? false : (i >= n_pv + NC - 2) ? true : (i % 2 == 0);  \
        const int idx = (i < 2) ? i : (i >= n_pv + NC - 2) ? (i - n_pv)                   \
                        : (i % 2 == 0) ? (i / 2 - 1) : ((i + 1) / 2);                     \
        if (i >= n_pv + NC) {                                                             \
        } else if (!is_s) {                                                               \
          o[idx / 2] = mfma32(vf[idx], (idx % 2) ? p1 : p0, o[idx / 2]);                  \
          vf[idx] = frag(VR, voff2, idx);                                                 \
        } else {                                                                          \
          sn = mfma32(kf[idx], qf[idx], sn);                                              \
        }                                                                                 \
        if (i < 16) {                                                                     \
          const int k = i / 2;                                                            \
          if (i % 2 == 0) {                                                               \
            tt[2 * k] = fmaf(sc[2 * k], scale_log2, -m_use);                              \
            tt[2 * k + 1] = fmaf(sc[2 * k + 1], scale_log2, -m_use);                      \
            tt[2 * k] = __builtin_amdgcn_exp2f(tt[2 * k]);                                \
          } else {                                                                        \
            tt[2 * k + 1] = __builtin_amdgcn_exp2f(tt[2 * k + 1]);                        \
            pk[k] = bf16x2{(__bf16)tt[2 * k], (__bf16)tt[2 * k + 1]};                     \
            if (k % 2 == 0)                                                               \
              a0 = __builtin_amdgcn_fdot2_f32_bf16(pk[k], ones2, a0, false);              \
            else                                                                          \
              a1 = __builtin_amdgcn_fdot2_f32_bf16(pk[k], ones2, a1, false);              \
          }                                                                               \
        }                                                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                \
      }                                                                                   \
      p0 = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),     \
                                   __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3),     \
                                   0, 1, 2, 3, 4, 5, 6, 7);                               \
      p1 = __builtin_shufflevector(__builtin_shufflevector(pk[4], pk[5], 0, 1, 2, 3),     \
                                   __builtin_shufflevector(pk[6], pk[7], 0, 1, 2, 3),     \
                                   0, 1, 2, 3, 4, 5, 6, 7);                               \
      float ps = a0 + a1;                                                                 \
      if (__builtin_expect(__any(ps > kSumLimit), 0)) {                                   \
        const float m_new =                                                               \
            fmaxf(ceilf(fmaxf(m_use, column_max(sc) * scale_log2)), kNegBig);             \
        const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);                        \
        l_run *= alpha;                                                                   \
        _Pragma("unroll") for (int db = 0; db < NDB; ++db)                                \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) o[db][r] *= alpha;               \
        m_use = m_new;                                                                    \
        ps = unit_probs(sc, scale_log2, m_use, p0, p1);                                   \
      }                                                                                   \
      l_run += ps;                                                                        \
      sc = sn;                                                                            \
      const uint32_t me = my_unit(st1);                                                   \
      if (me & 0x8000) mask_keys(sc, unit_mask(p, s, me, l32), g);                        \
    }                                                                                     \
    grp_sync();                                                                           \
    st0 = st1;                                                                            \
    st1 = st2;                                                                            \
    st2 = __builtin_amdgcn_readfirstlane(pend);                                           \
  }
      int u = 0;
      for (; u + 2 < n_u; u += 2) {
        VSA_STEP(kslot1, vslot0, kslot0, vslot1)
        ++u;
        VSA_STEP(kslot0, vslot1, kslot1, vslot0)
        --u;
      }
      if (u + 1 < n_u) {
        VSA_STEP(kslot1, vslot0, kslot0, vslot1)
        ++u;
      }
#undef VSA_STEP
      // Last step (V in slot u%2), after the PV product of step u-1.
      if (q_live) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          o[db] = mfma32(vf[db * 2], p0, o[db]);
          o[db] = mfma32(vf[db * 2 + 1], p1, o[db]);
        }
        float ps = unit_probs(sc, scale_log2, m_use, p0, p1);
        if (__builtin_expect(__any(ps > kSumLimit), 0)) {
          const float m_new = fmaxf(ceilf(fmaxf(m_use, column_max(sc) * scale_log2)), kNegBig);
          const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
          m_use = m_new;
          ps = unit_probs(sc, scale_log2, m_use, p0, p1);
        }
        l_run += ps;
        const int voff2 = unit_off(st0);
        const bf16_bits *vl = (u % 2 == 0) ? vslot0 : vslot1;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          o[db] = mfma32(frag(vl, voff2, db * 2), p0, o[db]);
          o[db] = mfma32(frag(vl, voff2, db * 2 + 1), p1, o[db]);
        }
      }
    }
    __syncthreads();                           // lists and slots free for the next chunk
  }
  if (stalled) fault = 1;

  // Merge the two key splits of each (tile, query half); the slots are free.
  float *osum = reinterpret_cast<float *>(tb ? kslot1 : kslot0);   // [64][D], swizzled
  float *sm_m = reinterpret_cast<float *>(vslot0);                 // [split][tile][64]
  float *sm_l = sm_m + kSplits * 2 * kTile;
  const int q = qb * 32 + l32;
  {
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (g == 0) {
      sm_m[(sp * 2 + tb) * kTile + q] = m_use;
      sm_l[(sp * 2 + tb) * kTile + q] = lt;
    }
  }
  __syncthreads();
  float M = kNegBig;
#pragma unroll
  for (int w = 0; w < kSplits; ++w) M = fmaxf(M, sm_m[(w * 2 + tb) * kTile + q]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSplits; ++w)
    L += sm_l[(w * 2 + tb) * kTile + q] * __builtin_amdgcn_exp2f(sm_m[(w * 2 + tb) * kTile + q] - M);
  const float f = __builtin_amdgcn_exp2f(m_use - M) / L;
  // Element (q, c) of the merged tile sits at q*D + (c ^ (q % 32)).
  for (int turn = 0; turn < kSplits; ++turn) {
    if (sp == turn) {
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
  const bool bad = fault != 0;
  bf16_bits *out_bh = out + (int64_t)bh * p.N * D;
  for (int t2 = 0; t2 < 2; ++t2) {
    const int tq = t2 ? tB : tA;
    if (tq < 0) continue;
    const int32_t *qmap = map + (int64_t)tq * kTile;
    const float *os = reinterpret_cast<const float *>(t2 ? kslot1 : kslot0);
    for (int idx = threadIdx.x; idx < kTile * D / 8; idx += blockDim.x) {
      const int row = idx / (D / 8), ch = idx % (D / 8);
      const int32_t tok = qmap[row];
      if (tok < 0) continue;
      bf16x8 v8;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8)
        v8[e8] = bad ? (__bf16)NAN : (__bf16)os[row * D + ((ch * 8 + e8) ^ (row % 32))];
      *reinterpret_cast<bf16x8 *>(out_bh + (int64_t)tok * D + ch * 8) = v8;
    }
    if (lse && threadIdx.x < kTile) {
      const int qq = threadIdx.x;
      const int32_t tok = qmap[qq];
      if (tok >= 0) {
        float MM = kNegBig;
        for (int w = 0; w < kSplits; ++w) MM = fmaxf(MM, sm_m[(w * 2 + t2) * kTile + qq]);
        float LL = 0.f;
        for (int w = 0; w < kSplits; ++w)
          LL += sm_l[(w * 2 + t2) * kTile + qq] *
                __builtin_amdgcn_exp2f(sm_m[(w * 2 + t2) * kTile + qq] - MM);
        lse[(int64_t)bh * p.N + tok] = bad ? NAN : MM * kLn2 + logf(LL);
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                            float scale, void *out, float *lse, hipStream_t stream) {
  const PairGrid gd = pairs::make_grid(p);
  const float sl2 = scale * kLog2e;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(gd.total), dim3(kThreads), 0, stream, p, gd,
                       (const bf16_bits *)qt, (const bf16_bits *)kt, (const bf16_bits *)vt, s2t,
                       kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(gd.total), dim3(kThreads), 0, stream, p, gd,
                       (const bf16_bits *)qt, (const bf16_bits *)kt, (const bf16_bits *)vt, s2t,
                       kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
