// Step 4 (fp8): tile-skipping flash attention on the 32x32x64 f8 MFMA.
//
// The low-precision variant of the bf16 kernel: the node runs its attention
// as a quantized kernel ("Veda Sparse Attention в ComfyUI", section "Узел
// ComfyUI"), and on MI355X the 8-bit matrix core format, OCP E4M3, runs at
// twice the bf16 rate. Inputs are the per-tile scaled E4M3 tiles written by
// the quantizer; each tile's power-of-two scale is applied inside the MFMA
// through its scale operand (an exact 2^(e) factor), so S = Q K^T and the
// PV product see the dequantized values.
//
// Work split as in the bf16 kernel: a workgroup of eight waves takes two
// neighbouring query tiles whose key lists are merged into shared and
// paired steps (attn_pairs.h), dealt to two key splits of four waves (two
// tiles x two 32-query halves). A unit is a whole 64-key tile here, because
// the PV product sums over 64 keys per instruction; its K and its V are
// 8 KiB each at d = 128, the size of a bf16 half-tile unit. K is copied into
// a two-slot LDS ring two steps ahead of use and V one step ahead, by
// direct-to-LDS buffer loads; the four waves of a split wait for each other
// once per step (bounded; a wave that gives up makes the workgroup write
// NaN).
//
// Products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so a lane
// owns one query column. The probabilities are packed to E4M3 in the order
// the S^T accumulator holds them, which is the order the V tile layout
// stores keys in, so P^T is the B operand of the PV product as it stands.
// Row sums are taken over the same rounded probabilities, by one more MFMA
// against an all-ones A operand, so numerator and denominator use the same
// weights. A step issues its nine MFMAs (the PV product and row sum of the
// previous unit alternating with the S^T product of the next) with the
// current unit's softmax spread between them.
//
// The running max m is an integer in log2 units, set 8 below the row max, so
// that probabilities lie in (0, 2^8] and use the whole E4M3 range (largest
// value 448; normal down to 2^-6). It is raised only when a unit holds a
// logit more than 8 above it. The test runs at the end of the step that
// computes the unit's S^T, outside the MFMA sequence: O and the row sums
// are rescaled there by the exact power of two, and the probabilities still
// waiting for their PV product (formed against the old max) take the same
// factor through the product's per-column B scale.
#include <cstdlib>

#include "attn_common.h"
#include "attn_pairs.h"
#include "fp8_layout.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 2;                       // key splits per workgroup
constexpr int kWaves = 8;                        // splits x two tiles x two query halves
constexpr int kThreads = 64 * kWaves;
using pairs::kNone;
using pairs::kRowCap;
using pairs::PairGrid;
constexpr int kStepCap = 2 * kRowCap;            // steps per chunk (one unit per key tile)
constexpr int kStepStride = kStepCap / kSplits;  // steps per split
constexpr int kChunkTiles = kStepCap;            // key tiles per chunk of a shared list
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;                   // probabilities <= 2^kSlack
constexpr int kOne = kFp8ExpBias;                // scale byte of 2^0
constexpr int kGuard = 1 << 20;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// D += A B over 64 E4M3 products per output, A scaled by 2^(sa - 127) and B
// by 2^(sb - 127) (scale bytes in bits 0..7).
__device__ inline f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ inline i32x8 join(i32x4 lo, i32x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The 32-byte operand of this lane in a 2 KiB block (two halves 1 KiB apart).
__device__ inline i32x8 lds_operand(const uint8_t *blk, int lane) {
  return join(*reinterpret_cast<const i32x4 *>(blk + lane * 16),
              *reinterpret_cast<const i32x4 *>(blk + 1024 + lane * 16));
}

// N consecutive 1 KiB blocks to LDS (N <= 4: one LDS base, instruction
// offsets move source and destination alike).
template <int N>
__device__ inline void copy_kib(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, int voff, int soff) {
  static_assert(N == 2 || N == 4, "two or four blocks");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 1024, 0);
  if (N == 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 3072, 0);
  }
}

// Counts as a use of x (in VGPRs) at this point, so that its computation
// stays before it. (The host pass, which never runs kernel code, sees an
// empty body: "v" is a GPU register constraint.)
template <typename T>
__host__ __device__ __forceinline__ void keep_here(const T &x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#else
  (void)x;
#endif
}

// Real-key mask of unit entry e (bit = key slot 0..63); 0 for no unit.
__device__ __forceinline__ uint64_t unit_mask(const Plan &p, int s, uint32_t e, int lane) {
  if (e == kNone) return 0ull;
  return __ballot(slot_token(p, s, (int)(e & 0x7FFF), lane) >= 0);
}

// Element r of block kb of lane (g, l32) of S^T is key kb*32 + (r/4)*8 + g*4 + r%4:
// after one shift by 4g, a fixed bit per element.
__device__ __forceinline__ void mask_keys(f32x16 (&sc)[2], uint64_t m, int g) {
  const uint64_t mg = m >> (4 * g);
  const uint32_t lo = (uint32_t)mg, hi = (uint32_t)(mg >> 32);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bit = (r / 4) * 8 + (r % 4);
      sc[kb][r] = (((kb ? hi : lo) >> bit) & 1u) ? sc[kb][r] : -INFINITY;
    }
}

// Four probabilities of elements r0..r0+3 of block kb against the max m,
// packed to E4M3: byte e = 4j + t of the P^T operand is element 4*(j%4) + t
// of block j/4.
__device__ __forceinline__ int probs4(const f32x16 &blk, int r0, float scale_log2, float m) {
  float pv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pv[t] = __builtin_amdgcn_exp2f(fmaf(blk[r0 + t], scale_log2, -m));
  return (int)fp8_pack4(pv[0], pv[1], pv[2], pv[3]);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fp8_kernel(Plan p, PairGrid gd, const uint8_t *__restrict__ q8,
                     const uint8_t *__restrict__ k8, const uint8_t *__restrict__ v8,
                     const uint32_t *__restrict__ scales, const int32_t *__restrict__ s2t,
                     const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ ref_idx,
                     float scale_log2, bf16_bits *__restrict__ out, float *__restrict__ lse) {
  constexpr int NCH = D / 64, NDB = D / 32;
  constexpr int TB = kTile * D;                // bytes of one fp8 tile (the unit)
  constexpr int SLOT = 2 * TB;                 // a split's slot: two units (tile A, tile B)
  constexpr int NS = 2 * NCH;                  // S^T products per unit
  constexpr int NP = NDB + 1;                  // PV products and the row sum
  constexpr int NSLOT = NS + NP;               // MFMA issue slots of a step
  __shared__ __attribute__((aligned(1024))) uint8_t kslot0[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot1[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot0[kSplits * SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot1[kSplits * SLOT];
  __shared__ uint32_t steps[kStepCap];
  __shared__ uint32_t ulA[kRowCap];
  __shared__ uint16_t bx[kRowCap];
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
  // Scale words are read through the constant address space (scalar loads).
  typedef const __attribute__((address_space(4))) uint32_t *const_u32_ptr;
  const const_u32_ptr sc_row = (const_u32_ptr)(scales + head_base);

  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q8 + head_base * TB, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k8 + head_base * TB, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8 + head_base * TB, head_bytes);
  const int voff = lane * 16;

  if (threadIdx.x < kSplits * 4) grp_count[threadIdx.x] = 0;
  if (threadIdx.x == 0) fault = 0;
  // A wave whose tile has no unit in a paired step (entry kNone) still runs
  // its PV products, with every probability zero, on its tile's half of the
  // V slot, which this kernel may not have written yet. LDS keeps what an
  // earlier kernel left there, possibly E4M3 NaN codes, and 0 * NaN = NaN; so
  // the V rings start zeroed. The barriers of the list building order these
  // stores before the first copy into the rings.
  {
    const i32x4 z = {0, 0, 0, 0};
    i32x4 *v0 = reinterpret_cast<i32x4 *>(vslot0), *v1 = reinterpret_cast<i32x4 *>(vslot1);
    for (int x = threadIdx.x; x < kSplits * SLOT / 16; x += kThreads) {
      v0[x] = z;
      v1[x] = z;
    }
  }

  i32x8 qf[NCH];              // this wave's Q^T operands (B of S^T = K Q^T)
  const int qtile = myT >= 0 ? myT : tA;
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int base = qtile * TB + (qb * NCH + cc) * 2048;
    qf[cc] = join(__builtin_amdgcn_raw_buffer_load_b128(rq, voff, base, 0),
                  __builtin_amdgcn_raw_buffer_load_b128(rq, voff, base + 1024, 0));
  }
  const int sq = (int)(sc_row[qtile] & 0xFFu);
  const bool q_live = myT >= 0 && __any(map[(int64_t)myT * kTile + qb * 32 + l32] >= 0);
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  f32x16 o[NDB], lsum;
#pragma unroll
  for (int r = 0; r < 16; ++r) lsum[r] = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_use = kNegBig;
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

  // Step lists: one unit per key tile; the merged build keeps its tile
  // bitmaps in the K slots before any copy.
  const pairs::ListSmem lsm{steps, ulA, bx, scan, reinterpret_cast<uint32_t *>(kslot0)};
  const uint32_t *mysteps = steps + sp * kStepStride;
  auto step_at = [&](int j) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(mysteps[j]);
  };
  auto my_unit = [&](uint32_t st) -> uint32_t { return tb ? (st >> 16) : (st & 0xFFFFu); };
  auto is_shared = [&](uint32_t st) -> bool { return (st & 0xFFFFu) == (st >> 16); };
  // Scale word of this wave's unit in a step (0 for none: the unit is masked).
  auto unit_word = [&](uint32_t st) -> uint32_t {
    const uint32_t e = my_unit(st);
    const uint32_t w = sc_row[min((int)(e & 0x7FFF), p.max_tiles - 1)];
    return e == kNone ? 0u : w;
  };
  // This wave's share of the copies of a step. Shared unit: roles 0 and 1
  // copy the two halves of K, roles 2 and 3 the two halves of V. Separate
  // units: role 0 copies A's K, role 1 A's V, role 2 B's K, role 3 B's V
  // (A's unit at offset 0 of the slot, B's at TB).
  auto issue_k = [&](uint32_t st, uint8_t *slot_all) __attribute__((always_inline)) {
    uint8_t *dst = slot_all + sp * SLOT;
    const uint32_t eA = st & 0xFFFFu, eB = st >> 16;
    if (eA == eB) {
      if (role < 2 && eA != kNone) {
        const int tile = (int)(eA & 0x7FFF);
        copy_kib<TB / 2048>(rk, (lds_ptr_t)(dst + role * (TB / 2)), voff,
                            tile * TB + role * (TB / 2));
      }
    } else if (role == 0 || role == 2) {
      const uint32_t e = (st >> (8 * role)) & 0xFFFFu;
      if (e != kNone) {
        const int tile = (int)(e & 0x7FFF);
        uint8_t *d2 = dst + (role / 2) * TB;
#pragma unroll
        for (int g4 = 0; g4 < TB / 4096; ++g4)
          copy_kib<4>(rk, (lds_ptr_t)(d2 + g4 * 4096), voff, tile * TB + g4 * 4096);
      }
    }
  };
  auto issue_v = [&](uint32_t st, uint8_t *slot_all) __attribute__((always_inline)) {
    uint8_t *dst = slot_all + sp * SLOT;
    const uint32_t eA = st & 0xFFFFu, eB = st >> 16;
    if (eA == eB) {
      if (role >= 2 && eA != kNone) {
        const int tile = (int)(eA & 0x7FFF);
        copy_kib<TB / 2048>(rv, (lds_ptr_t)(dst + (role - 2) * (TB / 2)), voff,
                            tile * TB + (role - 2) * (TB / 2));
      }
    } else if (role == 1 || role == 3) {
      const uint32_t e = (st >> (8 * (role - 1))) & 0xFFFFu;
      if (e != kNone) {
        const int tile = (int)(e & 0x7FFF);
        uint8_t *d2 = dst + (role / 2) * TB;
#pragma unroll
        for (int g4 = 0; g4 < TB / 4096; ++g4)
          copy_kib<4>(rv, (lds_ptr_t)(d2 + g4 * 4096), voff, tile * TB + g4 * 4096);
      }
    }
  };
  // Operand block blk of this wave's unit in a step's slot.
  auto unit_off = [&](uint32_t st) -> int { return is_shared(st) ? 0 : tb * TB; };
  auto frag = [&](const uint8_t *slot_all, int off, int blk) __attribute__((always_inline))
      -> i32x8 { return lds_operand(slot_all + sp * SLOT + off + blk * 2048, lane); };
  // Before a unit's softmax: raises the max when some column's logits reach
  // more than kSlack above it, rescaling O and the row sums (which hold every
  // unit whose PV product has been issued) and returning in ps the B scale
  // byte for the probabilities still waiting for theirs (kOne otherwise).
  auto check_max = [&](const f32x16 (&sc)[2], int &ps) __attribute__((always_inline)) {
    float mt = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = fmaxf(mt, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[1][r]);
    ps = kOne;
    if (__builtin_expect(__any(fmaf(mt, scale_log2, -m_use) > kSlack), 0)) {
      // Both lane halves hold the same query column.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      const float rm = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), mt);
      const float m_new = fmaxf(m_use, ceilf(rm * scale_log2) - kSlack);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      ps = kOne - (int)fminf(m_new - m_use, (float)kOne);
      m_use = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum[r] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  };

  const int n_rows = merge ? 1 : (fullA ? p.n_tiles[s] : video_row_len(p, s));
  const int chunk = merge ? n_rows : kChunkTiles;
  for (int e0 = 0; e0 < n_rows; e0 += chunk) {
    const int nS =
        merge ? pairs::build_merged<1, kWaves, kSplits, kStepStride>(
                    p, s, kv_row_of(tA), ref_row_of(tA), kv_row_of(tB), ref_row_of(tB), lsm)
              : pairs::build_shared<1, kWaves, kSplits, kStepStride>(
                    p, s, fullA, fullA ? nullptr : kv_row_of(tA), fullA ? nullptr : ref_row_of(tA),
                    e0, min(n_rows, e0 + chunk), lsm);
    const int n_u = nS > sp ? (nS - sp + kSplits - 1) / kSplits : 0;
    if (n_u > 0) {
      // Step u: K in slot u%2 of the K slots, V in slot u%2 of the V slots.
      // Step u issues K of step u+2 and V of step u+1, reads K of step u+1
      // and V of step u, takes the PV product and row sum of step u-1, S of
      // step u+1 with the softmax of step u, and ends with the group wait.
      uint32_t st0 = step_at(0);
      uint32_t st1 = n_u > 1 ? step_at(1) : kNone | (kNone << 16);
      uint32_t st2 = n_u > 2 ? step_at(2) : kNone | (kNone << 16);
      issue_k(st0, kslot0);
      if (n_u > 1) issue_k(st1, kslot1);
      issue_v(st0, vslot0);
      grp_sync();
      f32x16 sc[2];
      i32x8 vf[NDB], pprev;
      int sv_prev = kOne, sv_cur = kOne, ps = kOne;
      if (q_live) {
        const uint32_t w0 = unit_word(st0);
        const int sk = (int)((w0 >> 8) & 0xFFu);
        sv_cur = (int)((w0 >> 16) & 0xFFu);
        const int off = unit_off(st0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc)
            sc[kb] = mfma8(frag(kslot0, off, kb * NCH + cc), qf[cc], sc[kb], sk, sq);
        }
        const uint32_t me = my_unit(st0);
        if (me & 0x8000) mask_keys(sc, unit_mask(p, s, me, lane), g);
        check_max(sc, ps);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 8; ++j) vf[db][j] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) pprev[j] = 0;
      }
      grp_sync();
      // One step with a next step: KR/VR the slots read (K of step u+1, V of
      // step u), KW/VW the slots refilled (K of step u+2, V of step u+1).
      auto step = [&](int u, const uint8_t *KR, const uint8_t *VR, uint8_t *KW, uint8_t *VW)
          __attribute__((always_inline)) {
        if (u + 2 < n_u) issue_k(st2, KW);
        issue_v(st1, VW);
        const uint32_t pend = mysteps[min(u + 3, n_u - 1)];
        if (q_live) {
          const uint32_t w1 = unit_word(st1);
          const int sk1 = (int)((w1 >> 8) & 0xFFu);
          const int koff = unit_off(st1), voff2 = unit_off(st0);
          f32x16 sn[2];
          i32x8 kf[2];
          i32x8 pf;
          kf[0] = frag(KR, koff, 0);
          kf[1] = frag(KR, koff, 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NSLOT; ++i) {
            // Slots alternate PV (even) and S (odd) while both last.
            const int pairs_n = NS < NP ? NS : NP;
            const bool is_s = i < 2 * pairs_n ? (i % 2 == 1) : (NS > NP);
            const int idx = i < 2 * pairs_n ? i / 2 : i - pairs_n;
            if (is_s) {
              const int kb = idx / NCH, cc = idx % NCH;
              sn[kb] = mfma8(kf[idx % 2], qf[cc], cc == 0 ? f32x16{} : sn[kb], sk1, sq);
              if (idx + 2 < NS) kf[idx % 2] = frag(KR, koff, idx + 2);
            } else if (idx < NDB) {
              o[idx] = mfma8(vf[idx], pprev, o[idx], sv_prev, ps);
              vf[idx] = frag(VR, voff2, idx);
            } else {
              lsum = mfma8(ones, pprev, lsum, kOne, ps);
            }
#pragma unroll
            for (int c = (i * 8 + NSLOT - 1) / NSLOT; c < ((i + 1) * 8 + NSLOT - 1) / NSLOT; ++c)
              pf[c] = probs4(sc[c / 4], 4 * (c % 4), scale_log2, m_use);
            __builtin_amdgcn_sched_barrier(0);
          }
          // Keeps the probabilities and the PV products in the sequence above:
          // their next uses lie past the branches below, where the compiler
          // would otherwise move them.
          keep_here(pf);
          keep_here(lsum);
#pragma unroll
          for (int db = 0; db < NDB; ++db) keep_here(o[db]);
          pprev = pf;
          sc[0] = sn[0];
          sc[1] = sn[1];
          const uint32_t me = my_unit(st1);
          if (me & 0x8000) mask_keys(sc, unit_mask(p, s, me, lane), g);
          check_max(sc, ps);
          sv_prev = sv_cur;
          sv_cur = (int)((w1 >> 16) & 0xFFu);
        }
        grp_sync();
        st0 = st1;
        st1 = st2;
        st2 = __builtin_amdgcn_readfirstlane(pend);
      };
      int u = 0;
      for (; u + 2 < n_u; u += 2) {
        step(u, kslot1, vslot0, kslot0, vslot1);
        step(u + 1, kslot0, vslot1, kslot1, vslot0);
      }
      if (u + 1 < n_u) {
        step(u, kslot1, vslot0, kslot0, vslot1);
        ++u;
      }
      // Last step (V in slot u%2): the PV product of step u-1, then the
      // softmax and PV product of step u.
      if (q_live) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mfma8(vf[db], pprev, o[db], sv_prev, ps);
        lsum = mfma8(ones, pprev, lsum, kOne, ps);
        i32x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = probs4(sc[j / 4], 4 * (j % 4), scale_log2, m_use);
        const int voff2 = unit_off(st0);
        const uint8_t *vl = (u % 2 == 0) ? vslot0 : vslot1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = mfma8(frag(vl, voff2, db), pf, o[db], sv_cur, kOne);
        lsum = mfma8(ones, pf, lsum, kOne, kOne);
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
  if (g == 0) {
    sm_m[(sp * 2 + tb) * kTile + q] = m_use;
    sm_l[(sp * 2 + tb) * kTile + q] = lsum[0];                     // every row holds the sum
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
      bf16x8 v8o;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8)
        v8o[e8] = bad ? (__bf16)NAN : (__bf16)os[row * D + ((ch * 8 + e8) ^ (row % 32))];
      *reinterpret_cast<bf16x8 *>(out_bh + (int64_t)tok * D + ch * 8) = v8o;
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

hipError_t launch_attn_fp8(const Plan &p, const uint8_t *q8, const uint8_t *k8,
                           const uint8_t *v8, const uint8_t *scales, const int32_t *s2t,
                           const int32_t *kv_idx, const int32_t *ref_idx, float scale,
                           void *out, float *lse, hipStream_t stream) {
  const PairGrid gd = pairs::make_grid(p);
  const float sl2 = scale * kLog2e;
  const uint32_t *sw = (const uint32_t *)scales;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_fp8_kernel<128>, dim3(gd.total), dim3(kThreads), 0, stream, p, gd,
                       q8, k8, v8, sw, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<64>, dim3(gd.total), dim3(kThreads), 0, stream, p, gd,
                       q8, k8, v8, sw, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
