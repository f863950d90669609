// Device-side helpers shared by the kernels: element types, the two tiled
// layouts and the slot -> token map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace vsa {

constexpr int kTile = VSA_TILE;

// Row-operand layout of a tile (Q and K): 512-element blocks of 32 slots x 16
// channels; inside a block lane (0..63) holds 8 consecutive channels of one
// slot: lane = ((c%16)/8)*32 + s%32. This is the A/B operand order of the
// 32x32x16 bf16 MFMA, so one wave loads a block as 1 KB contiguous.
__host__ __device__ inline int row_layout_offset(int s, int c, int D) {
  return ((s / 32) * (D / 16) + c / 16) * 512 + (((c % 16) / 8) * 32 + s % 32) * 8 + c % 8;
}

// Inverse of row_layout_offset for element e of lane vector `vec` (8 elements).
__host__ __device__ inline void row_layout_decode(int vec, int e, int D, int &s, int &c) {
  int blk = vec / 64, lane = vec % 64;
  s = (blk / (D / 16)) * 32 + lane % 32;
  c = (blk % (D / 16)) * 16 + (lane / 32) * 8 + e;
}

// Column-operand layout (V): 512-element blocks of 16 slots x 32 channels;
// lane = ((s%8)/4)*32 + c%32 holds 8 slots of one channel, in the slot order
// the 32x32 MFMA accumulator leaves the softmax probabilities in, so that
// P^T from the first product feeds the second product without a shuffle.
__host__ __device__ inline int col_layout_offset(int s, int c, int D) {
  (void)D;
  return ((c / 32) * 4 + s / 16) * 512 + (((s % 8) / 4) * 32 + c % 32) * 8 +
         ((s % 16) / 8) * 4 + s % 4;
}

__host__ __device__ inline void col_layout_decode(int vec, int e, int D, int &s, int &c) {
  (void)D;
  int blk = vec / 64, lane = vec % 64;
  int j = blk % 4, db = blk / 4;
  s = j * 16 + (e / 4) * 8 + (lane / 32) * 4 + e % 4;
  c = db * 32 + lane % 32;
}

// Token held by slot `slot` of tile `tile` under shape `s`, or -1 for a pad.
__device__ inline int32_t slot_token(const Plan &p, int s, int tile, int slot) {
  if (tile < p.n_prefix_tiles) {
    int seg = 0;
    while (seg + 1 < p.n_prefix && tile >= p.prefix_tile0[seg + 1]) ++seg;
    int j = (tile - p.prefix_tile0[seg]) * kTile + slot;
    return j < p.prefix_len[seg] ? p.prefix_off[seg] + j : -1;
  }
  if (tile >= p.n_tiles[s]) return -1;
  int v = tile - p.n_prefix_tiles;
  int gw = p.grid_w[s], gh = p.grid_h[s];
  int wi = v % gw, hi = (v / gw) % gh, ti = v / (gw * gh);
  int pt = p.shape[s][0], ph = p.shape[s][1], pw = p.shape[s][2];
  int a = slot / (ph * pw), b = (slot / pw) % ph, c = slot % pw;
  int t = ti * pt + a, y = hi * ph + b, x = wi * pw + c;
  if (t >= p.T || y >= p.Hv || x >= p.Wv) return -1;
  return p.P + (t * p.Hv + y) * p.Wv + x;
}

// Key tile of entry e of a video query tile's key list: the dense prefix
// tiles (every prefix tile except those of the reference stream), then the
// kept reference tiles (ref_row), then the kept video tiles (kv_row). -1 when
// the stored index is not a tile of its stream (the entry is skipped). With
// no reference stream (n_ref == 0) the list is all prefix tiles, then kv_row.
template <typename Ptr>
__device__ inline int video_row_tile(const Plan &p, int s, int e, Ptr kv_row, Ptr ref_row) {
  const int n_dense = p.n_prefix_tiles - p.n_ref;
  if (e < n_dense) return e < p.ref_t0 ? e : e + p.n_ref;
  e -= n_dense;
  if (e < p.k_ref) {
    const int j = ref_row[e];
    return (unsigned)j < (unsigned)p.n_ref ? p.ref_t0 + j : -1;
  }
  const int j = kv_row[e - p.k_ref];
  return (unsigned)j < (unsigned)p.n_vt[s] ? p.n_prefix_tiles + j : -1;
}

// Length of a video query tile's key list.
__device__ inline int video_row_len(const Plan &p, int s) {
  return p.n_prefix_tiles - p.n_ref + p.k_ref + p.k[s];
}

// Buffer resource over `bytes` bytes at `base` (raw, untyped loads; reads past
// the end return zero instead of faulting). The varying part of an address
// then lives in SGPRs (soffset) plus one per-lane VGPR offset.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ inline bf16x8 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ inline float bf16_to_float(bf16_bits u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

template <typename T>
__device__ inline float to_float(T v);
template <>
__device__ inline float to_float<float>(float v) { return v; }
template <>
__device__ inline float to_float<bf16_bits>(bf16_bits v) { return bf16_to_float(v); }

}  // namespace vsa
