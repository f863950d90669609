// Pieces shared by the bf16 and fp8 tile-skipping attention kernels: the
// XCD-aware work-item numbering, the "tile holds no pad" test and the slot
// barrier of the LDS ring.
#pragma once

#include "device_common.h"

namespace vsa {

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Query tile of workgroup blockIdx.x. Workgroups reach the eight XCDs
// round-robin; the renumbering gives each XCD a contiguous run of query
// tiles (head order), so the key tiles that neighbouring query tiles share
// meet in one L2.
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

// True when every slot of `tile` holds a real token (wave-uniform inputs,
// so this compiles to scalar code).
__device__ inline bool tile_full(const Plan &p, int s, int tile) {
  if (tile < p.n_prefix_tiles) {
    int seg = 0;
    while (seg + 1 < p.n_prefix && tile >= p.prefix_tile0[seg + 1]) ++seg;
    return (tile - p.prefix_tile0[seg] + 1) * kTile <= p.prefix_len[seg];
  }
  if (p.video_full[s]) return true;
  const int v = tile - p.n_prefix_tiles;
  const int gw = p.grid_w[s], gh = p.grid_h[s];
  const int wi = v % gw, hi = (v / gw) % gh, ti = v / (gw * gh);
  return (ti + 1) * p.shape[s][0] <= p.T && (hi + 1) * p.shape[s][1] <= p.Hv &&
         (wi + 1) * p.shape[s][2] <= p.Wv;
}

// Both waves' copies have landed and both waves are done reading the slot
// they just used: own copies drained (vector-memory counter), then the
// workgroup barrier.
__device__ inline void sync_slots() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

}  // namespace vsa
