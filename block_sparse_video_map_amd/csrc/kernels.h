// Launchers of the HIP kernels (host side). Each enqueues on `stream` and
// returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

hipError_t launch_build_map(const Plan &p, int32_t *s2t, hipStream_t stream);
hipError_t launch_gather(const Plan &p, const void *q, const void *k, const void *v,
                         const int32_t *s2t, void *qt, void *kt, void *vt,
                         hipStream_t stream);
hipError_t launch_pool(const Plan &p, int mode, int proj_dim, const void *qt,
                       const void *kt, const int32_t *s2t, const float *wq,
                       const float *wk, double *pooled, hipStream_t stream);
hipError_t launch_scores(const Plan &p, int r, const double *pooled, float *scores,
                         hipStream_t stream);
hipError_t launch_select(const Plan &p, const float *scores, int32_t *kv_idx,
                         hipStream_t stream);
hipError_t launch_attention(const Plan &p, const void *qt, const void *kt,
                            const void *vt, const int32_t *s2t, const int32_t *kv_idx,
                            float scale, void *out, float *lse, hipStream_t stream);
