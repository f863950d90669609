// Host planner: validation, tile grids, kept counts and buffer sizes.
// Plain C++ with no HIP call, so every error path runs without a GPU.
#include "plan.h"

#include <cmath>
#include <cstring>

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Kept share in basis points: round half up of (1 - sparsity) * 10^4.
int32_t keep_basis_points(double sparsity) {
  return (int32_t)std::floor((1.0 - sparsity) * 10000.0 + 0.5);
}

}  // namespace

int make_plan_geometry(const vsa_problem *prob, Plan *p) {
  if (!prob || !p) return VSA_ERR_INVALID_ARG;
  std::memset(p, 0, sizeof(*p));
  if (prob->dtype != VSA_F32 && prob->dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (prob->d != 64 && prob->d != 128) return VSA_ERR_UNSUPPORTED;
  if (prob->B < 1 || prob->H < 1 || prob->N < 1) return VSA_ERR_INVALID_ARG;
  if (prob->T < 1 || prob->Hv < 1 || prob->Wv < 1) return VSA_ERR_INVALID_ARG;
  if (prob->n_prefix < 0 || prob->n_prefix > VSA_MAX_SEGMENTS) return VSA_ERR_INVALID_ARG;
  if (prob->n_shapes < 1 || prob->n_shapes > VSA_MAX_SHAPES) return VSA_ERR_INVALID_ARG;
  if (!prob->tile_shape) return VSA_ERR_INVALID_ARG;
  if ((int64_t)prob->B * prob->H > 65535) return VSA_ERR_SIZE;

  p->B = prob->B; p->H = prob->H; p->N = prob->N; p->d = prob->d;
  p->T = prob->T; p->Hv = prob->Hv; p->Wv = prob->Wv; p->dtype = prob->dtype;
  p->n_prefix = prob->n_prefix;

  int64_t tok = 0, tile = 0;
  for (int s = 0; s < prob->n_prefix; ++s) {
    int32_t L = prob->prefix_len[s];
    if (L < 0) return VSA_ERR_INVALID_ARG;
    p->prefix_len[s] = L;
    p->prefix_off[s] = (int32_t)tok;
    p->prefix_tile0[s] = (int32_t)tile;
    tok += L;
    tile += ceil_div(L, VSA_TILE);
    if (tok > INT32_MAX) return VSA_ERR_SIZE;
  }
  p->prefix_tile0[prob->n_prefix] = (int32_t)tile;
  p->P = (int32_t)tok;
  p->n_prefix_tiles = (int32_t)tile;

  int64_t video = (int64_t)prob->T * prob->Hv * prob->Wv;
  if (tok + video > INT32_MAX) return VSA_ERR_SIZE;
  if (tok + video != prob->N) return VSA_ERR_INVALID_ARG;

  p->n_shapes = prob->n_shapes;
  p->max_tiles = p->max_vt = 0;
  p->ref_t0 = p->n_ref = p->k_ref = 0;
  for (int s = 0; s < prob->n_shapes; ++s) {
    int32_t pt = prob->tile_shape[3 * s], ph = prob->tile_shape[3 * s + 1],
            pw = prob->tile_shape[3 * s + 2];
    if (pt < 1 || ph < 1 || pw < 1) return VSA_ERR_INVALID_ARG;
    if ((int64_t)pt * ph * pw != VSA_TILE) return VSA_ERR_INVALID_ARG;
    p->shape[s][0] = pt; p->shape[s][1] = ph; p->shape[s][2] = pw;
    int64_t gt = ceil_div(prob->T, pt), gh = ceil_div(prob->Hv, ph),
            gw = ceil_div(prob->Wv, pw);
    int64_t nvt = gt * gh * gw;
    if (nvt > VSA_MAX_VIDEO_TILES) return VSA_ERR_SIZE;
    p->grid_t[s] = (int32_t)gt; p->grid_h[s] = (int32_t)gh; p->grid_w[s] = (int32_t)gw;
    p->video_full[s] = prob->T % pt == 0 && prob->Hv % ph == 0 && prob->Wv % pw == 0;
    p->n_vt[s] = (int32_t)nvt;
    if (nvt + p->n_prefix_tiles > VSA_MAX_TILES) return VSA_ERR_SIZE;
    p->n_tiles[s] = (int32_t)(nvt + p->n_prefix_tiles);
    if (p->n_tiles[s] > p->max_tiles) p->max_tiles = p->n_tiles[s];
    if (p->n_vt[s] > p->max_vt) p->max_vt = p->n_vt[s];
  }
  p->tiles_per_batch = 0;
  for (int h = 0; h < prob->H; ++h) p->tiles_per_batch += p->n_tiles[h % p->n_shapes];
  p->tiles_per_cycle = 0;
  for (int s = 0; s < p->n_shapes; ++s) p->tiles_per_cycle += p->n_tiles[s];
  if (p->tiles_per_batch * p->B > INT32_MAX) return VSA_ERR_SIZE;
  return VSA_OK;
}

int make_plan(const vsa_problem *prob, double sparsity, Plan *p) {
  int st = make_plan_geometry(prob, p);
  if (st != VSA_OK) return st;
  if (!(sparsity >= 0.0 && sparsity < 1.0)) return VSA_ERR_INVALID_ARG;  // NaN too
  p->keep_bp = keep_basis_points(sparsity);
  p->dense = (sparsity == 0.0);
  p->k_max = 0;
  for (int s = 0; s < p->n_shapes; ++s) {
    int64_t kk = ceil_div((int64_t)p->keep_bp * p->n_vt[s], 10000);
    if (kk < 1) kk = 1;
    if (kk > p->n_vt[s]) kk = p->n_vt[s];
    p->k[s] = (int32_t)kk;
    if (p->k[s] > p->k_max) p->k_max = p->k[s];
  }
  return VSA_OK;
}

int descriptor_width(int mode, int proj_dim, int d, int *r) {
  if (mode == VSA_SCORE_MEAN_GATE) {
    if (proj_dim != d) return VSA_ERR_INVALID_ARG;
    *r = d;
    return VSA_OK;
  }
  const int stats = trippool_stats(mode);
  if (!stats) return VSA_ERR_INVALID_ARG;
  if (proj_dim < 8 || proj_dim > VSA_MAX_PROJ || (proj_dim & (proj_dim - 1)))
    return VSA_ERR_UNSUPPORTED;
  *r = proj_dim * __builtin_popcount(stats);
  return VSA_OK;
}

int apply_ref_budget(const vsa_ref_budget *rb, Plan *p) {
  if (!rb) return VSA_ERR_INVALID_ARG;
  if (rb->segment < 0 || rb->segment >= p->n_prefix) return VSA_ERR_INVALID_ARG;
  const int t0 = p->prefix_tile0[rb->segment];
  const int n = p->prefix_tile0[rb->segment + 1] - t0;
  if (n < 1) return VSA_ERR_INVALID_ARG;
  if (n > VSA_MAX_VIDEO_TILES) return VSA_ERR_SIZE;     // the select row length limit
  if (rb->k_ref < 1 || rb->k_ref > n) return VSA_ERR_INVALID_ARG;
  p->ref_t0 = t0;
  p->n_ref = n;
  p->k_ref = rb->k_ref;
  return VSA_OK;
}

extern "C" {

VSA_API int vsa_query_sizes(const vsa_problem *prob, double sparsity, vsa_sizes *sz) {
  if (!sz) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  std::memset(sz, 0, sizeof(*sz));
  int64_t bh = (int64_t)p.B * p.H;
  sz->map_elems = (int64_t)p.n_shapes * p.max_tiles * VSA_TILE;
  sz->tiled_elems = bh * p.max_tiles * VSA_TILE * p.d;
  sz->pooled_rows = 2 * bh * p.max_vt;
  sz->score_elems = bh * p.max_vt * p.max_vt;
  sz->idx_elems = bh * p.max_vt * p.k_max;
  sz->out_elems = bh * p.N * p.d;
  sz->n_prefix_tiles = p.n_prefix_tiles;
  sz->max_tiles = p.max_tiles;
  sz->max_video_tiles = p.max_vt;
  sz->k_max = p.k_max;
  sz->keep_bp = p.keep_bp;
  for (int s = 0; s < p.n_shapes; ++s) {
    sz->n_tiles[s] = p.n_tiles[s];
    sz->n_video_tiles[s] = p.n_vt[s];
    sz->k[s] = p.k[s];
  }
  return VSA_OK;
}

VSA_API int vsa_pooled_bytes(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                             int64_t *bytes) {
  if (!bytes) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  int r = 0;
  st = descriptor_width(mode, proj_dim, p.d, &r);
  if (st != VSA_OK) return st;
  *bytes = 2 * (int64_t)p.B * p.H * p.max_vt * r * (int64_t)sizeof(double);
  return VSA_OK;
}

static int kept_stats(const Plan &p, int64_t *kept, double *frac) {
  int64_t k_sum = 0, full = 0;
  for (int h = 0; h < p.H; ++h) {
    int s = h % p.n_shapes;
    int64_t nt = p.n_tiles[s], npt = p.n_prefix_tiles, nv = p.n_vt[s];
    int64_t kk = p.dense ? nv : p.k[s];
    int64_t row = p.dense ? nt : npt - p.n_ref + p.k_ref + kk;
    k_sum += npt * nt + nv * row;
    full += nt * nt;
  }
  *kept = k_sum * p.B;
  *frac = (double)k_sum / (double)full;
  return VSA_OK;
}

VSA_API int vsa_kept_stats(const vsa_problem *prob, double sparsity, int64_t *kept,
                           double *frac) {
  if (!kept || !frac) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  return kept_stats(p, kept, frac);
}

VSA_API int vsa_kept_stats_ref(const vsa_problem *prob, double sparsity,
                               const vsa_ref_budget *budget, int64_t *kept, double *frac) {
  if (!kept || !frac) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (p.dense) return VSA_ERR_INVALID_ARG;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  return kept_stats(p, kept, frac);
}

static int count_flops(const Plan &p, const int32_t *s2t, const int32_t *kv_idx,
                       const int32_t *ref_idx, double *flops) {
  long double total = 0;
  int npt = p.n_prefix_tiles;
  for (int b = 0; b < p.B; ++b) {
    for (int h = 0; h < p.H; ++h) {
      int s = h % p.n_shapes;
      const int32_t *map = s2t + (int64_t)s * p.max_tiles * VSA_TILE;
      auto real = [&](int64_t t) {
        int n = 0;
        for (int j = 0; j < VSA_TILE; ++j) n += map[t * VSA_TILE + j] >= 0;
        return (int64_t)n;
      };
      for (int t = 0; t < p.n_tiles[s]; ++t) {
        int64_t rq = real(t), keys = 0;
        if (t < npt || p.dense) {
          keys = p.N;
        } else {
          keys = p.P;
          const int64_t qrow = ((int64_t)b * p.H + h) * p.max_vt + (t - npt);
          if (p.n_ref > 0) {
            for (int j = 0; j < p.n_ref; ++j) keys -= real(p.ref_t0 + j);
            const int32_t *rrow = ref_idx + qrow * p.k_ref;
            for (int e = 0; e < p.k_ref; ++e) {
              int32_t j = rrow[e];
              if (j < 0 || j >= p.n_ref) return VSA_ERR_INVALID_ARG;
              keys += real(p.ref_t0 + j);
            }
          }
          const int32_t *row = kv_idx + qrow * p.k_max;
          for (int e = 0; e < p.k[s]; ++e) {
            int32_t j = row[e];
            if (j < 0 || j >= p.n_vt[s]) return VSA_ERR_INVALID_ARG;
            keys += real(npt + j);
          }
        }
        total += (long double)rq * keys;
      }
    }
  }
  *flops = (double)(total * 4.0L * p.d);
  return VSA_OK;
}

VSA_API int vsa_count_flops(const vsa_problem *prob, double sparsity,
                            const int32_t *s2t, const int32_t *kv_idx, double *flops) {
  if (!s2t || !flops) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (!p.dense && !kv_idx) return VSA_ERR_INVALID_ARG;
  return count_flops(p, s2t, kv_idx, nullptr, flops);
}

VSA_API int vsa_count_flops_ref(const vsa_problem *prob, double sparsity,
                                const vsa_ref_budget *budget, const int32_t *s2t,
                                const int32_t *kv_idx, const int32_t *ref_idx, double *flops) {
  if (!s2t || !flops || !kv_idx || !ref_idx) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (p.dense) return VSA_ERR_INVALID_ARG;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  return count_flops(p, s2t, kv_idx, ref_idx, flops);
}

VSA_API int vsa_ref_sizes(const vsa_problem *prob, const vsa_ref_budget *budget,
                          int32_t *n_ref_tiles, int64_t *ref_score_elems,
                          int64_t *ref_idx_elems) {
  if (!n_ref_tiles || !ref_score_elems || !ref_idx_elems) return VSA_ERR_INVALID_ARG;
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  const int64_t bh = (int64_t)p.B * p.H;
  *n_ref_tiles = p.n_ref;
  *ref_score_elems = bh * p.max_vt * p.n_ref;
  *ref_idx_elems = bh * p.max_vt * p.k_ref;
  return VSA_OK;
}

VSA_API int vsa_ref_pooled_bytes(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                                 const vsa_ref_budget *budget, int64_t *bytes) {
  if (!bytes) return VSA_ERR_INVALID_ARG;
  int64_t full = 0;
  int st = vsa_pooled_bytes(prob, mode, proj_dim, &full);
  if (st != VSA_OK) return st;
  Plan p;
  st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  const int64_t r = full / (2 * (int64_t)p.B * p.H * p.max_vt * (int64_t)sizeof(double));
  *bytes = (int64_t)p.B * p.H * p.n_ref * r * (int64_t)sizeof(double);
  return VSA_OK;
}

VSA_API const char *vsa_status_string(int status) {
  switch (status) {
    case VSA_OK: return "ok";
    case VSA_ERR_INVALID_ARG: return "invalid argument";
    case VSA_ERR_UNSUPPORTED: return "unsupported head dim or dtype";
    case VSA_ERR_SIZE: return "size exceeds a library limit";
    case VSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

VSA_API int vsa_version(void) { return VSA_VERSION; }

}  // extern "C"
