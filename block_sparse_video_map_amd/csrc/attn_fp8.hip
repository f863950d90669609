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
// The bf16 kernel's work split with two key splits instead of four: one
// 64-token query tile per workgroup of four waves, two key splits of two
// waves (one per 32-query half), two workgroups per CU. Each split has a
// two-slot LDS ring filled by direct-to-LDS buffer loads (wave 0 the K tile,
// wave 1 the V tile) and one barrier per key tile. A whole 64-key tile is one
// unit here: K and V of a tile are 8 KB each at d = 128. With half the bytes
// per key tile of the bf16 path, fewer splits per workgroup (less coupling at
// the barrier) measured faster than four, while the bf16 kernel keeps four
// (its L2 reuse across neighbouring query tiles matters more there).
//
// Products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so a lane
// owns one query column. The probabilities are packed to E4M3 in the order
// the S^T accumulator holds them, which is the order the V tile layout
// stores keys in, so P^T is the B operand of the PV product as it stands.
// Row sums are taken over the same rounded probabilities, by one more MFMA
// against an all-ones A operand, so numerator and denominator use the same
// weights.
//
// The running max m is an integer in log2 units, set 8 below the row max, so
// that probabilities lie in (0, 2^8] and use the whole E4M3 range (largest
// value 448; normal down to 2^-6). It is raised only when a unit holds a
// logit more than 8 above it; then O and the row sum are rescaled first.
#include <cstdlib>

#include "attn_common.h"
#include "fp8_layout.h"
#include "kernels.h"

namespace vsa {
namespace {

constexpr int kSplits = 2;                   // key splits per query tile
constexpr int kWaves = 2 * kSplits;          // two query halves per split
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kSlack = 8.0f;               // probabilities <= 2^kSlack
constexpr int kOne = kFp8ExpBias;            // scale byte of 2^0

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

// The 32-byte operand of this lane in a 2 KB block (two halves 1 KB apart).
__device__ inline i32x8 lds_operand(const uint8_t *blk, int lane) {
  return join(*reinterpret_cast<const i32x4 *>(blk + lane * 16),
              *reinterpret_cast<const i32x4 *>(blk + 1024 + lane * 16));
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fp8_kernel(Plan p, int total, const uint8_t *__restrict__ q8,
                     const uint8_t *__restrict__ k8, const uint8_t *__restrict__ v8,
                     const uint32_t *__restrict__ scales, const int32_t *__restrict__ s2t,
                     const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ ref_idx,
                     float scale_log2, bf16_bits *__restrict__ out, float *__restrict__ lse) {
  constexpr int NCH = D / 64, NDB = D / 32;
  constexpr int TB = kTile * D;                // bytes of one fp8 tile
  // Two slots per split, each K then V of one key tile. Distinct objects: a
  // slot is only read while the other one is being filled.
  __shared__ __attribute__((aligned(1024))) uint8_t ring0_all[kSplits * 2 * TB];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1_all[kSplits * 2 * TB];

  int b, h, tq;
  work_item(p, total, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int qb = wave % 2, ks = wave / 2;
  uint8_t *const ring0 = ring0_all + ks * 2 * TB;
  uint8_t *const ring1 = ring1_all + ks * 2 * TB;
  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : video_row_len(p, s);
  // Key lists and scale words are read through the constant address space
  // (scalar loads), off the vector-memory counter of the copies.
  typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
  typedef const __attribute__((address_space(4))) uint32_t *const_u32_ptr;
  const const_i32_ptr kv_row =
      full_row ? nullptr
               : (const_i32_ptr)(kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max);
  const const_i32_ptr ref_row =
      (full_row || p.n_ref == 0)
          ? nullptr
          : (const_i32_ptr)(ref_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_ref);
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const const_u32_ptr sc_row = (const_u32_ptr)(scales + head_base);
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;

  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q8 + head_base * TB, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k8 + head_base * TB, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8 + head_base * TB, head_bytes);
  const int voff = lane * 16;

  i32x8 qf[NCH];              // this wave's Q^T operands (B of S^T = K Q^T)
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int base = tq * TB + (qb * NCH + cc) * 2048;
    qf[cc] = join(__builtin_amdgcn_raw_buffer_load_b128(rq, voff, base, 0),
                  __builtin_amdgcn_raw_buffer_load_b128(rq, voff, base + 1024, 0));
  }
  const int sq = (int)(sc_row[tq] & 0xFFu);
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

  // Global tile of this split's i-th key tile; ok = false for an index
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
  auto tile_mask = [&](int tile, bool ok) -> uint64_t {
    if (!ok) return 0ull;
    if (tile_full(p, s, tile)) return ~0ull;
    return __ballot(slot_token(p, s, tile, lane) >= 0);
  };
  // Copy of key tile `tile` into a slot: wave 0 the K tile, wave 1 the V tile.
  auto issue = [&](uint8_t *slot, int tile) {
    const __amdgpu_buffer_rsrc_t r = qb == 0 ? rk : rv;
    uint8_t *dst = slot + qb * TB;
#pragma unroll
    for (int j = 0; j < TB / 1024; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + j * 1024), 16, voff,
                                               tile * TB + j * 1024, 0, 0);
  };
  // One key tile from a slot: S^T, the mask of a partly filled tile, the
  // rare raise of the max, E4M3 probabilities, row sums and PV.
  auto unit = [&](const uint8_t *slot, uint64_t mask, uint32_t word) {
    const int sk = (int)((word >> 8) & 0xFFu), sv = (int)((word >> 16) & 0xFFu);
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
        sc[kb] = mfma8(lds_operand(slot + (kb * NCH + cc) * 2048, lane), qf[cc], sc[kb], sk, sq);
    }
    if (mask != ~0ull) {
      // Element r of block kb of lane (g, l32) is key kb*32 + (r/4)*8 + g*4 + r%4.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          sc[kb][r] = ((mask >> key) & 1ull) ? sc[kb][r] : -INFINITY;
        }
    }
    float mt = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[1][r]);
    if (__builtin_expect(__any(fmaf(mt, scale_log2, -m_use) > kSlack), 0)) {
      // Move the max to 8 below the unit's row max (both lane halves hold
      // the same query), rescaling what has been summed so far.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      const float rm = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), mt);
      const float m_new = fmaxf(m_use, ceilf(rm * scale_log2) - kSlack);
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum[r] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_use = m_new;
    }
    // Byte e = 4j + t of the P^T operand is element 4*(j%4) + t of block j/4.
    i32x8 pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kb = j / 4, r0 = 4 * (j % 4);
      float pv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        pv[t] = __builtin_amdgcn_exp2f(fmaf(sc[kb][r0 + t], scale_log2, -m_use));
      pf[j] = (int)fp8_pack4(pv[0], pv[1], pv[2], pv[3]);
    }
    lsum = mfma8(ones, pf, lsum, kOne, kOne);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      o[db] = mfma8(lds_operand(slot + TB + db * 2048, lane), pf, o[db], sv, kOne);
  };

  // Unit i (this split's i-th key tile) uses ring0 for even i, ring1 for
  // odd i; the copy of unit i + 1 is issued before unit i is computed. Every
  // wave runs the same number of barriers; a split with fewer tiles idles.
  const int n_steps = (n_kv + kSplits - 1) / kSplits;
  bool ok = false;
  int t = 0;
  uint64_t mask = 0;
  uint32_t word = 0;
  if (n_mine > 0) {
    t = tile_of(0, ok);
    word = sc_row[t];
    mask = tile_mask(t, ok);
    issue(ring0, t);
  }
  sync_slots();
  for (int i = 0; i < n_steps; i += 2) {
    bool ok1 = false;
    int t1 = 0;
    uint32_t word1 = 0;
    if (i + 1 < n_mine) {
      t1 = tile_of(i + 1, ok1);
      word1 = sc_row[t1];
      issue(ring1, t1);
    }
    if (i < n_mine) unit(ring0, mask, word);
    const uint64_t mask1 = i + 1 < n_mine ? tile_mask(t1, ok1) : 0ull;
    sync_slots();
    bool ok2 = false;
    int t2 = 0;
    uint32_t word2 = 0;
    if (i + 2 < n_mine) {
      t2 = tile_of(i + 2, ok2);
      word2 = sc_row[t2];
      issue(ring0, t2);
    }
    if (i + 1 < n_mine) unit(ring1, mask1, word1);
    sync_slots();
    t = t2;
    word = word2;
    mask = i + 2 < n_mine ? tile_mask(t2, ok2) : 0ull;
  }

  // Merge the key splits of each query half (the rings are free now:
  // the last step ended with a barrier).
  float *osum = reinterpret_cast<float *>(ring0_all);       // [64][D], swizzled
  float *sm_m = reinterpret_cast<float *>(ring1_all);       // [kSplits][64]
  float *sm_l = sm_m + kSplits * kTile;
  const int q = qb * 32 + l32;
  if (g == 0) {
    sm_m[ks * kTile + q] = m_use;
    sm_l[ks * kTile + q] = lsum[0];                         // every row holds the sum
  }
  __syncthreads();
  float M = sm_m[q];
#pragma unroll
  for (int w = 1; w < kSplits; ++w) M = fmaxf(M, sm_m[w * kTile + q]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSplits; ++w)
    L += sm_l[w * kTile + q] * __builtin_amdgcn_exp2f(sm_m[w * kTile + q] - M);
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
    bf16x8 v8o;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8)
      v8o[e8] = (__bf16)osum[row * D + ((ch * 8 + e8) ^ (row % 32))];
    *reinterpret_cast<bf16x8 *>(out_bh + (int64_t)tok * D + ch * 8) = v8o;
  }
  if (lse && threadIdx.x < kTile) {
    const int qq = threadIdx.x;
    const int32_t tok = qmap[qq];
    if (tok >= 0) {
      float MM = sm_m[qq];
      for (int w = 1; w < kSplits; ++w) MM = fmaxf(MM, sm_m[w * kTile + qq]);
      float LL = 0.f;
      for (int w = 0; w < kSplits; ++w)
        LL += sm_l[w * kTile + qq] * __builtin_amdgcn_exp2f(sm_m[w * kTile + qq] - MM);
      lse[(int64_t)bh * p.N + tok] = MM * kLn2 + logf(LL);
    }
  }
}

}  // namespace

hipError_t launch_attn_fp8(const Plan &p, const uint8_t *q8, const uint8_t *k8,
                           const uint8_t *v8, const uint8_t *scales, const int32_t *s2t,
                           const int32_t *kv_idx, const int32_t *ref_idx, float scale,
                           void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  const float sl2 = scale * kLog2e;
  const uint32_t *sw = (const uint32_t *)scales;
  if (p.d == 128)
    hipLaunchKernelGGL(attn_fp8_kernel<128>, dim3(total), dim3(kThreads), 0, stream, p, total,
                       q8, k8, v8, sw, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<64>, dim3(total), dim3(kThreads), 0, stream, p, total,
                       q8, k8, v8, sw, s2t, kv_idx, ref_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
