// Launchers of the HIP kernels (host side). Each enqueues on `stream` and
// returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

hipError_t launch_build_map(const Plan &p, int32_t *s2t, hipStream_t stream);
// q8/k8/v8/scales non-null (bf16 only): also the E4M3 copies and scale bytes
// that launch_quant_fp8 would write, from the same pass. means non-null: also
// the channel means of the Q and K video tiles, double, at row
// (which * B*H + bh) * max_vt + video tile (the pooling workspace's layout).
hipError_t launch_gather(const Plan &p, const void *q, const void *k, const void *v,
                         const int32_t *s2t, void *qt, void *kt, void *vt, uint8_t *q8,
                         uint8_t *k8, uint8_t *v8, uint8_t *scales, hipStream_t stream,
                         double *means = nullptr);
// Mean gate from the tile means launch_gather wrote into `pooled`: each row
// is replaced, in place, by its product with the head's gate (wq for Q rows,
// wk for K rows), as the mean-gate pooling kernel computes it.
hipError_t launch_gate_means(const Plan &p, const float *wq, const float *wk, double *pooled,
                             hipStream_t stream);
// Tiles to pool: per (batch*head), tiles tile0 .. tile0+ntiles-1 of the tiled
// copies (ntiles < 0: the head's video tiles); source z of the launch reads
// src[z] with weights w[z] and writes rows ((z*nbh + bh - bh0)*rows + i) of
// the output. The launch covers (batch*head) bh0 .. bh0+nbh-1 (nbh < 0: all).
struct PoolJob {
  int32_t tile0;
  int32_t ntiles;
  int32_t rows;
  const void *src[2];
  const float *w[2];
  int32_t bh0 = 0;
  int32_t nbh = -1;
};

// Descriptor dot products: rows = the head's video query tiles of q, columns
// = ncols key descriptors of k (ncols < 0: the head's video tiles), output
// out[bh*out_bh + i*out_row + j]. q_bh / k_bh: doubles per (batch*head), q and
// k pointing at (batch*head) bh0; the launch covers bh0 .. bh0+nbh-1 (nbh < 0:
// all).
struct ScoreJob {
  const double *q;
  int64_t q_bh;
  const double *k;
  int64_t k_bh;
  int32_t ncols;
  float *out;
  int64_t out_row;
  int64_t out_bh;
  int32_t bh0 = 0;
  int32_t nbh = -1;
};

// Top-k per row: row i of (batch*head) bh is scores[bh*in_bh + i*in_row],
// ncols long (< 0: the head's video tiles), keeping k (< 0: the head's k);
// the ascending list goes to out[bh*out_bh + i*out_row], padded with -1 up
// to out_row.
struct SelectJob {
  const float *scores;
  int64_t in_row;
  int64_t in_bh;
  int32_t ncols;
  int32_t max_cols;
  int32_t k;
  int32_t *out;
  int32_t out_row;
  int64_t out_bh;
};

// Fused scores and top-k: descriptors q (rows) and k (columns) per
// (batch*head), q_bh / k_bh doubles apart; the ascending lists go to
// out[bh*out_bh + i*out_row], padded with -1 up to out_row.
struct FusedSelectJob {
  const double *q;
  int64_t q_bh;
  const double *k;
  int64_t k_bh;
  int32_t *out;
  int32_t out_row;
  int64_t out_bh;
};

hipError_t launch_pool(const Plan &p, int mode, int proj_dim, const PoolJob &job, int nsrc,
                       const int32_t *s2t, double *pooled, hipStream_t stream);
hipError_t launch_scores(const Plan &p, int r, const ScoreJob &job, hipStream_t stream);
hipError_t launch_select(const Plan &p, const SelectJob &job, hipStream_t stream);
// Needs p.max_vt <= VSA_FUSED_MAX_TILES and r % 32 == 0, r <= VSA_FUSED_MAX_R.
hipError_t launch_score_select(const Plan &p, int r, const FusedSelectJob &job,
                               hipStream_t stream);
// ref_idx: the reference stream's kept tiles when p.n_ref > 0, else unused.
hipError_t launch_attention(const Plan &p, const void *qt, const void *kt,
                            const void *vt, const int32_t *s2t, const int32_t *kv_idx,
                            const int32_t *ref_idx, float scale, void *out, float *lse,
                            hipStream_t stream);
// Teacher tile map: two dense passes (per-query log-sum-exp into lse_ws, then
// the largest attention probability per video tile pair into teacher).
hipError_t launch_teacher(const Plan &p, const void *qt, const void *kt, const int32_t *s2t,
                          float scale, float *lse_ws, float *teacher, hipStream_t stream);
// fp8 path: per-tile power-of-two scaled E4M3 copies of the bf16 tiles (and
// their scale bytes, 4 per (batch*head, tile)), then attention over them.
hipError_t launch_quant_fp8(const Plan &p, const void *qt, const void *kt, const void *vt,
                            uint8_t *q8, uint8_t *k8, uint8_t *v8, uint8_t *scales,
                            hipStream_t stream);
// Matrix-core rate probe (kind 0 bf16, 1 fp8): 256-thread workgroups, each
// wave `iters` trips of four MFMAs; ticks (or null) gets 4 counters per
// workgroup.
hipError_t launch_mfma_probe(int kind, int iters, int n_workgroups, uint64_t *ticks,
                             hipStream_t stream);
namespace vsa {
hipError_t launch_attn_fp8(const Plan &p, const uint8_t *q8, const uint8_t *k8,
                           const uint8_t *v8, const uint8_t *scales, const int32_t *s2t,
                           const int32_t *kv_idx, const int32_t *ref_idx, float scale,
                           void *out, float *lse, hipStream_t stream);
}  // namespace vsa
