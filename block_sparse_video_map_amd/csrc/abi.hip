// The C-ABI entry points: validate on the host, then enqueue the kernels.
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "plan.h"

namespace vsa {
hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                            float scale, void *out, float *lse, hipStream_t stream);
hipError_t launch_attn_f32(const Plan &p, const void *qt, const void *kt, const void *vt,
                           const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                           float scale, void *out, float *lse, hipStream_t stream);
}  // namespace vsa

hipError_t launch_attention(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, const int32_t *ref_idx,
                            float scale, void *out, float *lse, hipStream_t stream) {
  if (p.dtype == VSA_BF16)
    return vsa::launch_attn_bf16(p, qt, kt, vt, s2t, kv_idx, ref_idx, scale, out, lse, stream);
  return vsa::launch_attn_f32(p, qt, kt, vt, s2t, kv_idx, ref_idx, scale, out, lse, stream);
}

namespace {

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

}  // namespace

extern "C" {

VSA_API int vsa_map_tiles(const vsa_problem *prob, const void *q, const void *k,
                          const void *v, int32_t *slot_to_token, void *qt, void *kt,
                          void *vt, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  if (!slot_to_token) return VSA_ERR_INVALID_ARG;
  const void *in[3] = {q, k, v};
  void *outp[3] = {qt, kt, vt};
  for (int i = 0; i < 3; ++i) {
    if ((in[i] == nullptr) != (outp[i] == nullptr)) return VSA_ERR_INVALID_ARG;
    if (!aligned16(in[i]) || !aligned16(outp[i])) return VSA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_build_map(p, slot_to_token, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  if (!q && !k && !v) return VSA_OK;
  return hip_status(launch_gather(p, q, k, v, slot_to_token, qt, kt, vt, nullptr, nullptr,
                                  nullptr, nullptr, s));
}

VSA_API int vsa_map_tiles_scores(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                                 const void *q, const void *k, const void *v,
                                 int32_t *slot_to_token, void *qt, void *kt, void *vt,
                                 const float *wq, const float *wk, void *pooled_ws,
                                 float *scores, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  int64_t bytes = 0;
  st = vsa_pooled_bytes(prob, mode, proj_dim, &bytes);
  if (st != VSA_OK) return st;
  if (!slot_to_token || !q || !k || !qt || !kt || !wq || !pooled_ws || !scores)
    return VSA_ERR_INVALID_ARG;
  if (mode != VSA_SCORE_MEAN_GATE && !wk) return VSA_ERR_INVALID_ARG;
  if ((v == nullptr) != (vt == nullptr)) return VSA_ERR_INVALID_ARG;
  const void *in[3] = {q, k, v};
  void *outp[3] = {qt, kt, vt};
  for (int i = 0; i < 3; ++i)
    if (!aligned16(in[i]) || !aligned16(outp[i])) return VSA_ERR_INVALID_ARG;
  if ((uintptr_t)pooled_ws & 7u) return VSA_ERR_INVALID_ARG;
  int r = 0;
  descriptor_width(mode, proj_dim, p.d, &r);         // validated by vsa_pooled_bytes
  hipStream_t s = (hipStream_t)stream;
  double *pooled = (double *)pooled_ws;
  if (launch_build_map(p, slot_to_token, s) != hipSuccess) return VSA_ERR_HIP;
  if (mode == VSA_SCORE_MEAN_GATE) {
    if (launch_gather(p, q, k, v, slot_to_token, qt, kt, vt, nullptr, nullptr, nullptr, nullptr,
                      s, pooled) != hipSuccess)
      return VSA_ERR_HIP;
    if (launch_gate_means(p, wq, wk ? wk : wq, pooled, s) != hipSuccess) return VSA_ERR_HIP;
  } else {
    // TripPool: the plain gather, then the pooling kernel (projecting inside
    // the gather measured slower: the workgroup's memory phase and its f64
    // phase no longer overlap with other workgroups' at the gather's
    // occupancy).
    if (launch_gather(p, q, k, v, slot_to_token, qt, kt, vt, nullptr, nullptr, nullptr, nullptr,
                      s) != hipSuccess)
      return VSA_ERR_HIP;
    PoolJob job;
    job.tile0 = p.n_prefix_tiles;
    job.ntiles = -1;
    job.rows = p.max_vt;
    job.src[0] = qt;
    job.src[1] = kt;
    job.w[0] = wq;
    job.w[1] = wk;
    if (launch_pool(p, mode, proj_dim, job, 2, slot_to_token, pooled, s) != hipSuccess)
      return VSA_ERR_HIP;
  }
  const int64_t bh = (int64_t)p.B * p.H;
  ScoreJob sj;
  sj.q = pooled;
  sj.q_bh = (int64_t)p.max_vt * r;
  sj.k = pooled + bh * p.max_vt * r;
  sj.k_bh = (int64_t)p.max_vt * r;
  sj.ncols = -1;
  sj.out = scores;
  sj.out_row = p.max_vt;
  sj.out_bh = (int64_t)p.max_vt * p.max_vt;
  return hip_status(launch_scores(p, r, sj, s));
}

VSA_API int vsa_map_tiles_fp8(const vsa_problem *prob, const void *q, const void *k,
                              const void *v, int32_t *slot_to_token, void *qt, void *kt,
                              void *vt, void *q8, void *k8, void *v8, void *scales,
                              void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  if (p.dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (!slot_to_token || !q || !k || !v || !qt || !kt || !vt || !q8 || !k8 || !v8 || !scales)
    return VSA_ERR_INVALID_ARG;
  const void *al[10] = {q, k, v, qt, kt, vt, q8, k8, v8, nullptr};
  for (int i = 0; i < 9; ++i)
    if (!aligned16(al[i])) return VSA_ERR_INVALID_ARG;
  if ((uintptr_t)scales & 3u) return VSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_build_map(p, slot_to_token, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  return hip_status(launch_gather(p, q, k, v, slot_to_token, qt, kt, vt, (uint8_t *)q8,
                                  (uint8_t *)k8, (uint8_t *)v8, (uint8_t *)scales, s));
}

VSA_API int vsa_tile_scores(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                            const void *qt, const void *kt, const int32_t *slot_to_token,
                            const float *wq, const float *wk, void *pooled_ws,
                            float *scores, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  int64_t bytes = 0;
  st = vsa_pooled_bytes(prob, mode, proj_dim, &bytes);
  if (st != VSA_OK) return st;
  if (!qt || !kt || !slot_to_token || !wq || !pooled_ws || !scores) return VSA_ERR_INVALID_ARG;
  if (mode != VSA_SCORE_MEAN_GATE && !wk) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || ((uintptr_t)pooled_ws & 7u))
    return VSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  PoolJob job;
  job.tile0 = p.n_prefix_tiles;
  job.ntiles = -1;
  job.rows = p.max_vt;
  job.src[0] = qt;
  job.src[1] = kt;
  job.w[0] = wq;
  job.w[1] = (mode == VSA_SCORE_MEAN_GATE && !wk) ? wq : wk;
  hipError_t e = launch_pool(p, mode, proj_dim, job, 2, slot_to_token, (double *)pooled_ws, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  int r = 0;
  descriptor_width(mode, proj_dim, p.d, &r);         // validated by vsa_pooled_bytes
  const int64_t bh = (int64_t)p.B * p.H;
  ScoreJob sj;
  sj.q = (const double *)pooled_ws;
  sj.q_bh = (int64_t)p.max_vt * r;
  sj.k = (const double *)pooled_ws + bh * p.max_vt * r;
  sj.k_bh = (int64_t)p.max_vt * r;
  sj.ncols = -1;
  sj.out = scores;
  sj.out_row = p.max_vt;
  sj.out_bh = (int64_t)p.max_vt * p.max_vt;
  return hip_status(launch_scores(p, r, sj, s));
}

VSA_API int vsa_select_topk(const vsa_problem *prob, const float *scores, double sparsity,
                            int32_t *kv_idx, void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (!scores || !kv_idx) return VSA_ERR_INVALID_ARG;
  SelectJob j;
  j.scores = scores;
  j.in_row = p.max_vt;
  j.in_bh = (int64_t)p.max_vt * p.max_vt;
  j.ncols = -1;
  j.max_cols = p.max_vt;
  j.k = -1;
  j.out = kv_idx;
  j.out_row = p.k_max;
  j.out_bh = (int64_t)p.max_vt * p.k_max;
  return hip_status(launch_select(p, j, (hipStream_t)stream));
}

VSA_API int vsa_tile_select(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                            const void *qt, const void *kt, const int32_t *slot_to_token,
                            const float *wq, const float *wk, double sparsity, void *pooled_ws,
                            int32_t *kv_idx, void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  int64_t bytes = 0;
  st = vsa_pooled_bytes(prob, mode, proj_dim, &bytes);
  if (st != VSA_OK) return st;
  if (p.dense) return VSA_ERR_INVALID_ARG;            // nothing to select
  if (!qt || !kt || !slot_to_token || !wq || !pooled_ws || !kv_idx) return VSA_ERR_INVALID_ARG;
  if (mode != VSA_SCORE_MEAN_GATE && !wk) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || ((uintptr_t)pooled_ws & 7u))
    return VSA_ERR_INVALID_ARG;
  int r = 0;
  descriptor_width(mode, proj_dim, p.d, &r);         // validated by vsa_pooled_bytes
  if (p.max_vt > VSA_FUSED_MAX_TILES || r % 32 != 0 || r > VSA_FUSED_MAX_R)
    return VSA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  PoolJob job;
  job.tile0 = p.n_prefix_tiles;
  job.ntiles = -1;
  job.rows = p.max_vt;
  job.src[0] = qt;
  job.src[1] = kt;
  job.w[0] = wq;
  job.w[1] = (mode == VSA_SCORE_MEAN_GATE && !wk) ? wq : wk;
  hipError_t e = launch_pool(p, mode, proj_dim, job, 2, slot_to_token, (double *)pooled_ws, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  const int64_t bh = (int64_t)p.B * p.H;
  FusedSelectJob fj;
  fj.q = (const double *)pooled_ws;
  fj.q_bh = (int64_t)p.max_vt * r;
  fj.k = (const double *)pooled_ws + bh * p.max_vt * r;
  fj.k_bh = (int64_t)p.max_vt * r;
  fj.out = kv_idx;
  fj.out_row = p.k_max;
  fj.out_bh = (int64_t)p.max_vt * p.k_max;
  return hip_status(launch_score_select(p, r, fj, s));
}

VSA_API int vsa_sparse_attn_fwd(const vsa_problem *prob, const void *qt, const void *kt,
                                const void *vt, const int32_t *slot_to_token,
                                const int32_t *kv_idx, double sparsity,
                                float softmax_scale, void *out, float *lse,
                                void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (!qt || !kt || !vt || !slot_to_token || !out) return VSA_ERR_INVALID_ARG;
  if (!p.dense && !kv_idx) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || !aligned16(vt) || !aligned16(out))
    return VSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return VSA_ERR_INVALID_ARG;
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.d);
  return hip_status(launch_attention(p, qt, kt, vt, slot_to_token, kv_idx, nullptr, scale, out,
                                     lse, (hipStream_t)stream));
}

VSA_API int vsa_ref_scores(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                           const void *kt, const int32_t *slot_to_token, const float *wq,
                           const float *wk, const vsa_ref_budget *budget,
                           const void *pooled_ws, void *ref_pooled_ws, float *ref_scores,
                           void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  int64_t bytes = 0;
  st = vsa_pooled_bytes(prob, mode, proj_dim, &bytes);
  if (st != VSA_OK) return st;
  if (!kt || !slot_to_token || !wq || !pooled_ws || !ref_pooled_ws || !ref_scores)
    return VSA_ERR_INVALID_ARG;
  if (mode != VSA_SCORE_MEAN_GATE && !wk) return VSA_ERR_INVALID_ARG;
  if (!aligned16(kt) || ((uintptr_t)pooled_ws & 7u) || ((uintptr_t)ref_pooled_ws & 7u))
    return VSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const float *wkey = (mode == VSA_SCORE_MEAN_GATE && !wk) ? wq : wk;
  PoolJob job;
  job.tile0 = p.ref_t0;
  job.ntiles = p.n_ref;
  job.rows = p.n_ref;
  job.src[0] = job.src[1] = kt;
  job.w[0] = job.w[1] = wkey;
  hipError_t e = launch_pool(p, mode, proj_dim, job, 1, slot_to_token,
                             (double *)ref_pooled_ws, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  int r = 0;
  descriptor_width(mode, proj_dim, p.d, &r);         // validated by vsa_pooled_bytes
  ScoreJob sj;
  sj.q = (const double *)pooled_ws;                  // video query descriptors
  sj.q_bh = (int64_t)p.max_vt * r;
  sj.k = (const double *)ref_pooled_ws;
  sj.k_bh = (int64_t)p.n_ref * r;
  sj.ncols = p.n_ref;
  sj.out = ref_scores;
  sj.out_row = p.n_ref;
  sj.out_bh = (int64_t)p.max_vt * p.n_ref;
  return hip_status(launch_scores(p, r, sj, s));
}

VSA_API int vsa_ref_select(const vsa_problem *prob, const vsa_ref_budget *budget,
                           const float *ref_scores, int32_t *ref_idx, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  if (!ref_scores || !ref_idx) return VSA_ERR_INVALID_ARG;
  SelectJob j;
  j.scores = ref_scores;
  j.in_row = p.n_ref;
  j.in_bh = (int64_t)p.max_vt * p.n_ref;
  j.ncols = p.n_ref;
  j.max_cols = p.n_ref;
  j.k = p.k_ref;
  j.out = ref_idx;
  j.out_row = p.k_ref;
  j.out_bh = (int64_t)p.max_vt * p.k_ref;
  return hip_status(launch_select(p, j, (hipStream_t)stream));
}

VSA_API int vsa_sparse_attn_fwd_ref(const vsa_problem *prob, const void *qt, const void *kt,
                                    const void *vt, const int32_t *slot_to_token,
                                    const int32_t *kv_idx, double sparsity,
                                    const vsa_ref_budget *budget, const int32_t *ref_idx,
                                    float softmax_scale, void *out, float *lse,
                                    void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (p.dense) return VSA_ERR_INVALID_ARG;
  st = apply_ref_budget(budget, &p);
  if (st != VSA_OK) return st;
  if (!qt || !kt || !vt || !slot_to_token || !out || !kv_idx || !ref_idx)
    return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || !aligned16(vt) || !aligned16(out))
    return VSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return VSA_ERR_INVALID_ARG;
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.d);
  return hip_status(launch_attention(p, qt, kt, vt, slot_to_token, kv_idx, ref_idx, scale, out,
                                     lse, (hipStream_t)stream));
}

VSA_API int vsa_teacher_map(const vsa_problem *prob, const void *qt, const void *kt,
                            const int32_t *slot_to_token, float softmax_scale, float *lse_ws,
                            float *teacher, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  if (!qt || !kt || !slot_to_token || !lse_ws || !teacher) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt)) return VSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return VSA_ERR_INVALID_ARG;
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.d);
  return hip_status(launch_teacher(p, qt, kt, slot_to_token, scale, lse_ws, teacher,
                                   (hipStream_t)stream));
}

VSA_API int vsa_quantize_fp8(const vsa_problem *prob, const void *qt, const void *kt,
                             const void *vt, void *q8, void *k8, void *v8, void *scales,
                             void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  if (p.dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (!qt || !kt || !vt || !q8 || !k8 || !v8 || !scales) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || !aligned16(vt) || !aligned16(q8) || !aligned16(k8) ||
      !aligned16(v8) || ((uintptr_t)scales & 3u))
    return VSA_ERR_INVALID_ARG;
  return hip_status(launch_quant_fp8(p, qt, kt, vt, (uint8_t *)q8, (uint8_t *)k8,
                                     (uint8_t *)v8, (uint8_t *)scales, (hipStream_t)stream));
}

VSA_API int vsa_sparse_attn_fwd_fp8(const vsa_problem *prob, const void *q8, const void *k8,
                                    const void *v8, const void *scales,
                                    const int32_t *slot_to_token, const int32_t *kv_idx,
                                    double sparsity, const vsa_ref_budget *budget,
                                    const int32_t *ref_idx, float softmax_scale, void *out,
                                    float *lse, void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (p.dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (budget) {
    if (p.dense || !ref_idx) return VSA_ERR_INVALID_ARG;
    st = apply_ref_budget(budget, &p);
    if (st != VSA_OK) return st;
  }
  if (!q8 || !k8 || !v8 || !scales || !slot_to_token || !out) return VSA_ERR_INVALID_ARG;
  if (!p.dense && !kv_idx) return VSA_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(out) ||
      ((uintptr_t)scales & 3u))
    return VSA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return VSA_ERR_INVALID_ARG;
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.d);
  return hip_status(vsa::launch_attn_fp8(p, (const uint8_t *)q8, (const uint8_t *)k8,
                                         (const uint8_t *)v8, (const uint8_t *)scales,
                                         slot_to_token, kv_idx, ref_idx, scale, out, lse,
                                         (hipStream_t)stream));
}

VSA_API int vsa_device_clocks(int32_t *cu_count, int32_t *clock_khz, int32_t *wall_khz) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VSA_ERR_HIP;
  const hipDeviceAttribute_t attr[3] = {hipDeviceAttributeMultiprocessorCount,
                                        hipDeviceAttributeClockRate,
                                        hipDeviceAttributeWallClockRate};
  int32_t *dst[3] = {cu_count, clock_khz, wall_khz};
  for (int i = 0; i < 3; ++i) {
    if (!dst[i]) continue;
    int v = 0;
    if (hipDeviceGetAttribute(&v, attr[i], dev) != hipSuccess) return VSA_ERR_HIP;
    *dst[i] = v;
  }
  return VSA_OK;
}

VSA_API int vsa_mfma_probe(int32_t kind, int32_t iters, int32_t n_workgroups, uint64_t *ticks,
                           void *stream) {
  if (kind < 0 || kind > 4) return VSA_ERR_INVALID_ARG;
  if (iters < 1 || n_workgroups < 1) return VSA_ERR_INVALID_ARG;
  if (iters > (1 << 22) || n_workgroups > (1 << 16)) return VSA_ERR_SIZE;
  if ((uintptr_t)ticks & 7u) return VSA_ERR_INVALID_ARG;
  return hip_status(launch_mfma_probe(kind, iters, n_workgroups, ticks, (hipStream_t)stream));
}

}  // extern "C"
