// Step 4 (bf16): tile-skipping flash attention on the 32x32x16 bf16 MFMA.
//
// Work unit: one 64-token query tile per workgroup of eight waves, two waves
// per SIMD. Wave w owns query half qb = w % 2 (32 queries) and key split
// ks = w / 2: the query tile's key-tile list (all prefix tiles, then its kept
// video tiles; every tile for a prefix query tile) is dealt round-robin to the
// four key splits. Each wave keeps its own running max, sum and output; the
// four key splits of each query half are merged in LDS at the end. The two
// waves sharing a SIMD interleave in hardware, so one wave's softmax (VALU)
// runs under the other wave's matrix products.
//
// The products are taken transposed, S^T = K Q^T and O^T = V^T P^T, so that
// every lane owns one query column: the softmax max/sum needs a single
// exchange with lane^32, the rescale of O is one scalar per lane, and the
// accumulator of S^T is already the B operand of the PV product once
// converted to bf16. Q/K tiles are stored in the MFMA operand order and V
// tiles in the matching column order (see the tiled layouts), so every
// operand fetch is a contiguous 1 KB wave load straight into registers.
//
// Each wave walks its key tiles in 32-key halves ("units") through a
// software pipeline: S of unit u+1 is computed before the softmax of unit u,
// K of unit u+2 is fetched right after that, and V of unit u+1 right after
// the PV product of unit u. The output is rescaled only when a row maximum
// grows by more than 2^8 (exact: O and the sum share the stale maximum).
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

constexpr int kSplits = 4;              // key splits per query tile
constexpr int kThreads = 64 * 2 * kSplits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: stale max may lag by 2^8

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Maps a workgroup id to (b, h, query tile). Workgroup ids reach the eight
// XCDs round-robin. map_mode 0: each XCD walks one contiguous eighth of all
// query tiles; 1: identity (the XCDs share the same head, interleaved tiles);
// 2: runs of 32 consecutive query tiles are dealt to the XCDs in turn, so all
// XCDs work on the same stretch of one head, each on a contiguous run.
__device__ inline void work_item(const Plan &p, int total, int map_mode, int &b, int &h,
                                 int &tq) {
  int i = blockIdx.x;
  int L = i;
  if (map_mode == 0) {
    int q8 = total / 8;
    L = i < 8 * q8 ? (i % 8) * q8 + i / 8 : i;
  } else if (map_mode == 2) {
    // Runs of 32 consecutive query tiles, dealt to the XCDs in turn.
    constexpr int run = 32;
    const int grp = i / (8 * run), w = i % (8 * run);
    if (grp < total / (8 * run)) L = grp * 8 * run + (w % 8) * run + w / 8;
  }
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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(Plan p, int total, int map_mode, const bf16_bits *__restrict__ qt,
                      const bf16_bits *__restrict__ kt, const bf16_bits *__restrict__ vt,
                      const int32_t *__restrict__ s2t, const int32_t *__restrict__ kv_idx,
                      float scale_log2, bf16_bits *__restrict__ out,
                      float *__restrict__ lse) {
  constexpr int NC = D / 16;   // 16-channel chunks (QK^T reduction steps)
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int LDO = D + 1;
  __shared__ float sm_m[kSplits][kTile], sm_l[kSplits][kTile];
  __shared__ float osum[kTile * LDO];

  int b, h, tq;
  work_item(p, total, map_mode, b, h, tq);
  const int s = h % p.n_shapes;
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform
  const int lane = threadIdx.x % 64;
  const int qb = wave % 2, ks = wave / 2;
  const int g = lane / 32, l32 = lane % 32;
  const int npt = p.n_prefix_tiles;
  const bool full_row = p.dense || tq < npt;
  const int n_kv = full_row ? p.n_tiles[s] : npt + p.k[s];
  const int32_t *kv_row =
      full_row ? nullptr : kv_idx + ((int64_t)bh * p.max_vt + (tq - npt)) * p.k_max;
  const int64_t head_base = (int64_t)bh * p.max_tiles;
  const int32_t *map = s2t + (int64_t)s * p.max_tiles * kTile;
  const int n_mine = n_kv > ks ? (n_kv - ks + kSplits - 1) / kSplits : 0;

  // Buffer resources over this head's tiles: tile t, block j of a tile is at
  // byte t*TB + j*1024, lane l reads 16 bytes at +16*l.
  constexpr int TB = kTile * D * 2;      // bytes per tile
  const uint32_t head_bytes = (uint32_t)p.max_tiles * TB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + head_base * (kTile * D), head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt + head_base * (kTile * D), head_bytes);
  const int voff = lane * 16;

  bf16x8 qf[NC];              // Q^T fragments of this query half
  bf16x8 kf[NC];              // K of one 32-key unit
  bf16x8 vf[NDB][2];          // V of one 32-key unit
  f32x16 sbuf[2];             // S^T of two consecutive units
  f32x16 o[NDB];              // O^T accumulators
  float m_use = kNegBig, l_run = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = buffer_load16(rq, voff, tq * TB + (qb * NC + cc) * 1024);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // Tile of the wave's i-th key-tile entry; an entry that is not a tile index
  // is served by tile 0 with every key masked out.
  // (Every value here is wave-uniform; readfirstlane states that to the
  // compiler so tile offsets stay in scalar registers.)
  auto tile_of = [&](int i, bool &ok) -> int {
    const int e = ks + kSplits * i;
    ok = true;
    if (full_row || e < npt) return e;
    const int j = __builtin_amdgcn_readfirstlane(kv_row[e - npt]);
    if ((unsigned)j >= (unsigned)p.n_vt[s]) {
      ok = false;
      return 0;
    }
    return npt + j;
  };
  auto tile_mask = [&](int tile, bool ok) -> uint64_t {
    const uint64_t m = __ballot(map[tile * kTile + lane] >= 0);
    return ok ? m : 0ull;
  };
  auto load_k = [&](int tile, int kb) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      kf[cc] = buffer_load16(rk, voff, tile * TB + (kb * NC + cc) * 1024);
  };
  auto load_v = [&](int tile, int kb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        vf[db][jj] = buffer_load16(rv, voff, tile * TB + (db * 4 + 2 * kb + jj) * 1024);
  };
  auto qk = [&](f32x16 &acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc = mfma32(kf[cc], qf[cc], acc);
  };
  // Softmax of one unit (S^T in sc, keys masked by mask32) and its PV product.
  auto softmax_pv = [&](f32x16 &sc, uint32_t mask32) {
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
      for (int jj = 0; jj < 2; ++jj) o[db] = mfma32(vf[db][jj], pf[jj], o[db]);
  };

  if (n_mine > 0) {
    // Prologue: S of unit 0, K of unit 1 and V of unit 0 in flight.
    bool ok_cur, ok_nxt = false;
    int tile_cur = tile_of(0, ok_cur);
    int tile_nxt = 0;
    uint64_t mask_cur = tile_mask(tile_cur, ok_cur), mask_nxt = 0;
    load_k(tile_cur, 0);
    load_v(tile_cur, 0);
    qk(sbuf[0]);
    load_k(tile_cur, 1);

    for (int i = 0; i < n_mine; ++i) {
      const bool more = i + 1 < n_mine;
      if (more) {
        tile_nxt = tile_of(i + 1, ok_nxt);
        mask_nxt = tile_mask(tile_nxt, ok_nxt);
      }
      // Unit 2i = tile i, keys 0..31 (S in sbuf[0]); K holds unit 2i+1.
      qk(sbuf[1]);                           // S of unit 2i+1
      if (more) load_k(tile_nxt, 0);         // K of unit 2i+2
      softmax_pv(sbuf[0], (uint32_t)mask_cur);
      load_v(tile_cur, 1);                   // V of unit 2i+1
      // Unit 2i+1 = tile i, keys 32..63 (S in sbuf[1]); K holds unit 2i+2.
      if (more) {
        qk(sbuf[0]);                         // S of unit 2i+2
        load_k(tile_nxt, 1);                 // K of unit 2i+3
      }
      softmax_pv(sbuf[1], (uint32_t)(mask_cur >> 32));
      if (more) load_v(tile_nxt, 0);         // V of unit 2i+2
      ok_cur = ok_nxt;
      tile_cur = tile_nxt;
      mask_cur = mask_nxt;
    }
  }

  // Merge the four key splits of each query half.
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

hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, float scale,
                            void *out, float *lse, hipStream_t stream) {
  const int total = (int)(p.tiles_per_batch * p.B);
  const float sl2 = scale * kLog2e;
  static const int map_mode = [] {
    const char *e = getenv("VSA_ATTN_MAP");   // tuning knob, read once
    return e ? atoi(e) : 0;
  }();
  if (p.d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, map_mode, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(total), dim3(kThreads), 0, stream, p,
                       total, map_mode, (const bf16_bits *)qt, (const bf16_bits *)kt,
                       (const bf16_bits *)vt, s2t, kv_idx, sl2, (bf16_bits *)out, lse);
  return hipGetLastError();
}

}  // namespace vsa
