// Host planner: the validated problem with every derived count. The struct is
// trivially copyable and is handed to every kernel by value.
#pragma once

#include <stdint.h>

#include "vsa.h"

struct Plan {
  int32_t B, H, N, d, T, Hv, Wv;
  int32_t dtype;
  int32_t n_prefix;
  int32_t prefix_len[VSA_MAX_SEGMENTS];
  int32_t prefix_off[VSA_MAX_SEGMENTS];        // first token of the segment
  int32_t prefix_tile0[VSA_MAX_SEGMENTS + 1];  // first tile of the segment
  int32_t P;                                   // prefix tokens
  int32_t n_shapes;
  int32_t shape[VSA_MAX_SHAPES][3];            // (pt, ph, pw)
  int32_t grid_t[VSA_MAX_SHAPES], grid_h[VSA_MAX_SHAPES], grid_w[VSA_MAX_SHAPES];
  int32_t video_full[VSA_MAX_SHAPES];          // every video tile of the shape is full
  int32_t n_prefix_tiles;
  int32_t n_tiles[VSA_MAX_SHAPES];
  int32_t n_vt[VSA_MAX_SHAPES];
  int32_t k[VSA_MAX_SHAPES];
  int32_t max_tiles, max_vt, k_max, keep_bp;
  int32_t dense;                               // sparsity == 0
  // Two-stream budget: prefix tiles [ref_t0, ref_t0 + n_ref) form the
  // reference stream, of which every video query tile keeps k_ref
  // (n_ref == 0: off, every prefix tile is a dense key).
  int32_t ref_t0, n_ref, k_ref;
  int64_t tiles_per_batch;                     // sum over heads of n_tiles
  int64_t tiles_per_cycle;                     // sum over one shape cycle
};

// Validates `prob` and fills `plan`. Returns a vsa_status. Host only.
int make_plan(const vsa_problem *prob, double sparsity, Plan *plan);

// Validates `prob` ignoring sparsity (steps that do not depend on it).
int make_plan_geometry(const vsa_problem *prob, Plan *plan);

// Validates a two-stream budget against the plan and records it there.
int apply_ref_budget(const vsa_ref_budget *budget, Plan *plan);

// Width r (doubles) of one tile descriptor for a score mode. Returns a
// vsa_status: mean gate needs proj_dim == d; the TripPool modes a power of
// two in 8..VSA_MAX_PROJ, r = proj_dim times the number of statistics.
int descriptor_width(int mode, int proj_dim, int d, int *r);

// TripPool statistics a mode writes, as bits: 1 Avg, 2 Max, 4 Min (blocks
// in that order); 0 for the mean gate.
inline int trippool_stats(int mode) {
  switch (mode) {
    case VSA_SCORE_TRIPPOOL: return 7;
    case VSA_SCORE_TRIPPOOL_MAXMIN: return 6;
    case VSA_SCORE_TRIPPOOL_AVG: return 1;
    default: return 0;
  }
}
