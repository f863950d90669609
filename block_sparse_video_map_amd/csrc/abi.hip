// The C-ABI entry points: validate on the host, then enqueue the kernels.
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "plan.h"

namespace vsa {
hipError_t launch_attn_bf16(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, float scale,
                            void *out, float *lse, hipStream_t stream);
hipError_t launch_attn_f32(const Plan &p, const void *qt, const void *kt, const void *vt,
                           const int32_t *s2t, const int32_t *kv_idx, float scale,
                           void *out, float *lse, hipStream_t stream);
}  // namespace vsa

hipError_t launch_attention(const Plan &p, const void *qt, const void *kt, const void *vt,
                            const int32_t *s2t, const int32_t *kv_idx, float scale,
                            void *out, float *lse, hipStream_t stream) {
  if (p.dtype == VSA_BF16)
    return vsa::launch_attn_bf16(p, qt, kt, vt, s2t, kv_idx, scale, out, lse, stream);
  return vsa::launch_attn_f32(p, qt, kt, vt, s2t, kv_idx, scale, out, lse, stream);
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
  return hip_status(launch_gather(p, q, k, v, slot_to_token, qt, kt, vt, s));
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
  if (mode == VSA_SCORE_TRIPPOOL && !wk) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt) || ((uintptr_t)pooled_ws & 7u))
    return VSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_pool(p, mode, proj_dim, qt, kt, slot_to_token, wq, wk,
                             (double *)pooled_ws, s);
  if (e != hipSuccess) return VSA_ERR_HIP;
  int r = mode == VSA_SCORE_MEAN_GATE ? p.d : 3 * proj_dim;
  return hip_status(launch_scores(p, r, (const double *)pooled_ws, scores, s));
}

VSA_API int vsa_select_topk(const vsa_problem *prob, const float *scores, double sparsity,
                            int32_t *kv_idx, void *stream) {
  Plan p;
  int st = make_plan(prob, sparsity, &p);
  if (st != VSA_OK) return st;
  if (!scores || !kv_idx) return VSA_ERR_INVALID_ARG;
  return hip_status(launch_select(p, scores, kv_idx, (hipStream_t)stream));
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
  return hip_status(launch_attention(p, qt, kt, vt, slot_to_token, kv_idx, scale, out, lse,
                                     (hipStream_t)stream));
}

}  // extern "C"
