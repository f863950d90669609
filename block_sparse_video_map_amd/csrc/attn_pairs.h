// Query-tile pairs and their step lists, shared by the bf16 and fp8
// tile-skipping attention kernels.
//
// A workgroup takes two neighbouring query tiles of one head, A and B
// (prefix query tiles pair with prefix query tiles and video with video; an
// odd one out goes alone). A query tile's key list (all prefix tiles, then
// its kept video tiles; every tile for a prefix query tile) is cut into
// units of U per key tile: U = 2 gives 32-key halves (the bf16 kernel),
// U = 1 whole 64-key tiles (the fp8 kernel, whose matrix instruction sums
// over 64 keys). Units without a real key are dropped. A unit both tiles
// keep is one shared step; the i-th unit only A keeps and the i-th unit only
// B keeps form one paired step. Membership comes from a bitmap of each row's
// tiles, so the order of the indices does not matter. Step j goes to key
// split j % kSplits.
//
// Entry of a unit: tile * U + half, bit 15 set when the unit holds a pad
// slot; kNone for no unit. A step word holds A's entry in bits 0..15 and
// B's in bits 16..31 (equal for a shared step).
#pragma once

#include <algorithm>

#include "attn_common.h"

namespace vsa {
namespace pairs {

constexpr int kRowCap = 1024;                    // key tiles per row of a merged pair list
constexpr uint32_t kNone = 0xFFFF;               // no unit for this tile in a step

// Workgroups per head and shape for the pairing of query tiles.
struct PairGrid {
  int32_t n_wg[VSA_MAX_SHAPES];   // workgroups per head of each shape
  int64_t wg_per_cycle;           // over one cycle of shapes
  int64_t wg_per_batch;
  int32_t total;
  int32_t pair_video;             // video query rows are paired (their lists fit)
};

inline PairGrid make_grid(const Plan &p) {
  PairGrid g{};
  int longest = 0;
  for (int s = 0; s < p.n_shapes; ++s)
    longest = std::max(longest, p.n_prefix_tiles - p.n_ref + p.k_ref + p.k[s]);
  g.pair_video = !p.dense && longest <= kRowCap;
  for (int s = 0; s < p.n_shapes; ++s) {
    if (p.dense) {
      g.n_wg[s] = (p.n_tiles[s] + 1) / 2;
    } else {
      g.n_wg[s] = (p.n_prefix_tiles + 1) / 2 + (g.pair_video ? (p.n_vt[s] + 1) / 2 : p.n_vt[s]);
    }
  }
  g.wg_per_cycle = 0;
  for (int s = 0; s < p.n_shapes; ++s) g.wg_per_cycle += g.n_wg[s];
  g.wg_per_batch = 0;
  for (int h = 0; h < p.H; ++h) g.wg_per_batch += g.n_wg[h % p.n_shapes];
  g.total = (int32_t)(g.wg_per_batch * p.B);
  return g;
}

__device__ inline int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Real keys among the 32 slots of key half kb of `tile` (shape s).
__device__ inline int unit_real(const Plan &p, int s, int tile, int kb) {
  if (tile < p.n_prefix_tiles) {
    int seg = 0;
    while (seg + 1 < p.n_prefix && tile >= p.prefix_tile0[seg + 1]) ++seg;
    const int r = p.prefix_len[seg] - (tile - p.prefix_tile0[seg]) * kTile - 32 * kb;
    return r < 0 ? 0 : (r > 32 ? 32 : r);
  }
  if (p.video_full[s]) return 32;
  const int v = tile - p.n_prefix_tiles;
  const int gw = p.grid_w[s], gh = p.grid_h[s];
  const int wi = v % gw, hi = (v / gw) % gh, ti = v / (gw * gh);
  const int pt = p.shape[s][0], ph = p.shape[s][1], pw = p.shape[s][2];
  const int rt = min(pt, p.T - ti * pt), rh = min(ph, p.Hv - hi * ph), rw = min(pw, p.Wv - wi * pw);
  if (rt == pt && rh == ph && rw == pw) return 32;
  // Slot (a*ph + b)*pw + c is real when a < rt, b < rh and c < rw. The
  // extents are powers of two (their product is 64), so a half of the tile
  // is a whole range along one axis: the a-planes [kb*pt/2, (kb+1)*pt/2)
  // when a plane holds at most 32 slots, else (pt = 1) the b-rows
  // [kb*ph/2, (kb+1)*ph/2) when a row holds at most 32, else (ph = 1) the
  // columns [kb*32, kb*32 + 32).
  auto overlap = [](int lo, int len, int r) { return max(0, min(lo + len, r) - lo); };
  if (ph * pw <= 32) return overlap(kb * (pt / 2), pt / 2, rt) * rh * rw;
  if (pw <= 32) return overlap(kb * (ph / 2), ph / 2, rh) * rw;
  return overlap(kb * 32, 32, rw);
}

// Query tiles tA, tB (tB < 0: none) of workgroup blockIdx.x. Workgroups
// reach the eight XCDs round-robin; the renumbering gives each XCD a
// contiguous run of pairs (head order), so the key tiles that neighbouring
// query tiles share meet in one L2.
__device__ inline void pair_item(const Plan &p, const PairGrid &gd, int &b, int &h, int &tA,
                                 int &tB) {
  const int i = blockIdx.x;
  const int q8 = gd.total / 8;
  const int L = i < 8 * q8 ? (i % 8) * q8 + i / 8 : i;
  b = (int)(L / gd.wg_per_batch);
  const int64_t rem = L % gd.wg_per_batch;
  const int cyc = (int)(rem / gd.wg_per_cycle);
  int r = (int)(rem % gd.wg_per_cycle);
  int s = 0;
  while (r >= gd.n_wg[s]) {
    r -= gd.n_wg[s];
    ++s;
  }
  h = cyc * p.n_shapes + s;
  const int npt = p.n_prefix_tiles;
  if (p.dense) {
    tA = 2 * r;
    tB = tA + 1 < p.n_tiles[s] ? tA + 1 : -1;
    return;
  }
  const int npw = (npt + 1) / 2;
  if (r < npw) {
    tA = 2 * r;
    tB = tA + 1 < npt ? tA + 1 : -1;
    return;
  }
  const int v = r - npw;
  if (gd.pair_video) {
    tA = npt + 2 * v;
    tB = 2 * v + 1 < p.n_vt[s] ? tA + 1 : -1;
  } else {
    tA = npt + v;
    tB = -1;
  }
}

// The LDS arrays of the list building. steps: kSplits rows of `stride`
// words; ulA and bx: U * kRowCap entries; scan: 2 * (waves of the
// workgroup) ints; bitmap: 2 * ceil(max_tiles / 32) words, free to reuse
// once the lists are built.
struct ListSmem {
  uint32_t *steps;
  uint32_t *ulA;
  uint16_t *bx;
  int *scan;
  uint32_t *bitmap;
};

// Real-key counts of the U units of `tile` (n1 = 0 for U = 1).
template <int U>
__device__ __forceinline__ void tile_units(const Plan &p, int s, int tile, int &n0, int &n1) {
  if (U == 2) {
    n0 = unit_real(p, s, tile, 0);
    n1 = unit_real(p, s, tile, 1);
  } else {
    n0 = unit_real(p, s, tile, 0) + unit_real(p, s, tile, 1);
    n1 = 0;
  }
}

template <int U>
__device__ __forceinline__ uint32_t unit_entry(int tile, int half, int real) {
  return (uint32_t)(tile * U + half) | (real < 32 * (3 - U) ? 0x8000u : 0u);
}

template <int kSplits, int kStride>
__device__ __forceinline__ void put_step(const ListSmem &sm, int j, uint32_t eA, uint32_t eB) {
  sm.steps[(j % kSplits) * kStride + j / kSplits] = eA | (eB << 16);
}

// Units of the row entries [e0, e1) (kv_row/ref_row: the row's kept video
// tiles; full rows take every tile) as shared steps; returns their count.
template <int U, int kWaves, int kSplits, int kStride>
__device__ __forceinline__ int build_shared(const Plan &p, int s, bool full, const int32_t *kv_row,
                                            const int32_t *ref_row, int e0, int e1,
                                            const ListSmem &sm) {
  constexpr int kThreads = 64 * kWaves;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  int base = 0;
  for (int r0 = e0; r0 < e1; r0 += kThreads) {
    const int e = r0 + (int)threadIdx.x;
    int tile = -1, n0 = 0, n1 = 0;
    if (e < e1) {
      tile = full ? e : video_row_tile(p, s, e, kv_row, ref_row);
      if (tile >= 0) tile_units<U>(p, s, tile, n0, n1);
    }
    const uint64_t b1 = __ballot(n0 > 0 || n1 > 0);
    const uint64_t b2 = U == 2 ? __ballot(n0 > 0 && n1 > 0) : 0ull;
    const int pre = lanes_below(b1) + (U == 2 ? lanes_below(b2) : 0);
    if (lane == 0)
      sm.scan[wave] = __builtin_popcountll(b1) + (U == 2 ? __builtin_popcountll(b2) : 0);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = sm.scan[w];
      woff += w < wave ? c : 0;
      tot += c;
    }
    int pos = base + woff + pre;
    if (n0 > 0) {
      const uint32_t u = unit_entry<U>(tile, 0, n0);
      put_step<kSplits, kStride>(sm, pos++, u, u);
    }
    if (U == 2 && n1 > 0) {
      const uint32_t u = unit_entry<U>(tile, 1, n1);
      put_step<kSplits, kStride>(sm, pos, u, u);
    }
    base += tot;
    __syncthreads();
  }
  return base;
}

// Two video rows A and B: units both rows keep are shared steps; the i-th
// unit only A keeps and the i-th unit only B keeps make one step (kNone for
// the shorter side). Returns the step count.
template <int U, int kWaves, int kSplits, int kStride>
__device__ __forceinline__ int build_merged(const Plan &p, int s, const int32_t *kvA,
                                            const int32_t *rfA, const int32_t *kvB,
                                            const int32_t *rfB, const ListSmem &sm) {
  constexpr int kThreads = 64 * kWaves;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  uint32_t *bmA = sm.bitmap;
  uint32_t *bmB = bmA + (p.max_tiles + 31) / 32;
  const int words = (p.max_tiles + 31) / 32;
  for (int i = threadIdx.x; i < 2 * words; i += kThreads) bmA[i] = 0u;
  __syncthreads();
  const int n_kv = video_row_len(p, s);
  for (int e = threadIdx.x; e < n_kv; e += kThreads) {
    const int ta = video_row_tile(p, s, e, kvA, rfA), tbb = video_row_tile(p, s, e, kvB, rfB);
    if (ta >= 0) atomicOr(&bmA[ta >> 5], 1u << (ta & 31));
    if (tbb >= 0) atomicOr(&bmB[tbb >> 5], 1u << (tbb & 31));
  }
  __syncthreads();
  int nA = 0, nxA = 0;
  for (int r0 = 0; r0 < n_kv; r0 += kThreads) {
    const int e = r0 + (int)threadIdx.x;
    int tile = -1, n0 = 0, n1 = 0;
    bool shared = false;
    if (e < n_kv) {
      tile = video_row_tile(p, s, e, kvA, rfA);
      if (tile >= 0) {
        tile_units<U>(p, s, tile, n0, n1);
        shared = (bmB[tile >> 5] >> (tile & 31)) & 1u;
      }
    }
    const int cnt = (n0 > 0) + (n1 > 0), xc = shared ? 0 : cnt;
    const uint64_t b1 = __ballot(cnt >= 1), b2 = U == 2 ? __ballot(cnt >= 2) : 0ull;
    const uint64_t x1 = __ballot(xc >= 1), x2 = U == 2 ? __ballot(xc >= 2) : 0ull;
    const int pre = lanes_below(b1) + (U == 2 ? lanes_below(b2) : 0);
    const int xpre = lanes_below(x1) + (U == 2 ? lanes_below(x2) : 0);
    if (lane == 0) {
      sm.scan[wave] = __builtin_popcountll(b1) + (U == 2 ? __builtin_popcountll(b2) : 0);
      sm.scan[kWaves + wave] = __builtin_popcountll(x1) + (U == 2 ? __builtin_popcountll(x2) : 0);
    }
    __syncthreads();
    int woff = 0, tot = 0, xoff = 0, xtot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = sm.scan[w], x = sm.scan[kWaves + w];
      woff += w < wave ? c : 0;
      tot += c;
      xoff += w < wave ? x : 0;
      xtot += x;
    }
    int pos = nA + woff + pre, xr = nxA + xoff + xpre;
    if (n0 > 0) {
      const uint32_t u = unit_entry<U>(tile, 0, n0);
      sm.ulA[pos++] = u | (shared ? 0u : (uint32_t)(xr++ + 1) << 16);
    }
    if (U == 2 && n1 > 0) {
      const uint32_t u = unit_entry<U>(tile, 1, n1);
      sm.ulA[pos] = u | (shared ? 0u : (uint32_t)(xr + 1) << 16);
    }
    nA += tot;
    nxA += xtot;
    __syncthreads();
  }
  int nxB = 0;
  for (int r0 = 0; r0 < n_kv; r0 += kThreads) {
    const int e = r0 + (int)threadIdx.x;
    int tile = -1, n0 = 0, n1 = 0;
    if (e < n_kv) {
      tile = video_row_tile(p, s, e, kvB, rfB);
      if (tile >= 0 && !((bmA[tile >> 5] >> (tile & 31)) & 1u)) tile_units<U>(p, s, tile, n0, n1);
    }
    const uint64_t b1 = __ballot(n0 > 0 || n1 > 0);
    const uint64_t b2 = U == 2 ? __ballot(n0 > 0 && n1 > 0) : 0ull;
    const int pre = lanes_below(b1) + (U == 2 ? lanes_below(b2) : 0);
    if (lane == 0)
      sm.scan[wave] = __builtin_popcountll(b1) + (U == 2 ? __builtin_popcountll(b2) : 0);
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = sm.scan[w];
      woff += w < wave ? c : 0;
      tot += c;
    }
    int pos = nxB + woff + pre;
    if (n0 > 0) sm.bx[pos++] = (uint16_t)unit_entry<U>(tile, 0, n0);
    if (U == 2 && n1 > 0) sm.bx[pos] = (uint16_t)unit_entry<U>(tile, 1, n1);
    nxB += tot;
    __syncthreads();
  }
  const int nS = nA + max(0, nxB - nxA);
  for (int i = threadIdx.x; i < nS; i += kThreads) {
    uint32_t eA, eB;
    if (i < nA) {
      const uint32_t a = sm.ulA[i];
      eA = a & 0xFFFFu;
      const uint32_t x = a >> 16;
      eB = x == 0 ? eA : (x - 1 < (uint32_t)nxB ? (uint32_t)sm.bx[x - 1] : kNone);
    } else {
      eA = kNone;
      eB = sm.bx[nxA + (i - nA)];
    }
    put_step<kSplits, kStride>(sm, i, eA, eB);
  }
  __syncthreads();
  return nS;
}

}  // namespace pairs
}  // namespace vsa
