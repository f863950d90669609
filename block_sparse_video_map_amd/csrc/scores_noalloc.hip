// vsa_tile_scores without a caller workspace: the pooled tile descriptors
// live in a fixed device array of the library (`scratch`), for callers that
// cannot allocate device memory. The (batch, head) pairs are taken in chunks
// that fit the array; every chunk is pooled and scored with the same kernels
// as vsa_tile_scores, so the scores are identical.
#include <algorithm>
#include <mutex>

#include "kernels.h"
#include "plan.h"

namespace {

constexpr int64_t kScratchBytes = VSA_NOALLOC_SCRATCH_BYTES;

// One copy per GPU the library runs on, held until the process ends.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current. Host code uses this address, never the
// array's name (a host-side stand-in).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return VSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return VSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

VSA_API int vsa_tile_scores_noalloc(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                                    const void *qt, const void *kt,
                                    const int32_t *slot_to_token, const float *wq,
                                    const float *wk, float *scores, void *stream) {
  Plan p;
  int st = make_plan_geometry(prob, &p);
  if (st != VSA_OK) return st;
  int r = 0;
  st = descriptor_width(mode, proj_dim, p.d, &r);
  if (st != VSA_OK) return st;
  if (!qt || !kt || !slot_to_token || !wq || !scores) return VSA_ERR_INVALID_ARG;
  if (mode != VSA_SCORE_MEAN_GATE && !wk) return VSA_ERR_INVALID_ARG;
  if (!aligned16(qt) || !aligned16(kt)) return VSA_ERR_INVALID_ARG;
  // Q and K descriptors of one (batch, head) must fit the array.
  const int64_t per_bh = 2 * (int64_t)p.max_vt * r * (int64_t)sizeof(double);
  if (per_bh > kScratchBytes) return VSA_ERR_SIZE;
  void *ptr = nullptr;
  st = scratch_address(&ptr);
  if (st != VSA_OK) return st;
  double *pooled = (double *)ptr;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n_bh = (int64_t)p.B * p.H;
  const int64_t chunk = std::min<int64_t>(n_bh, kScratchBytes / per_bh);
  for (int64_t bh0 = 0; bh0 < n_bh; bh0 += chunk) {
    const int32_t n = (int32_t)std::min<int64_t>(chunk, n_bh - bh0);
    PoolJob job;
    job.tile0 = p.n_prefix_tiles;
    job.ntiles = -1;
    job.rows = p.max_vt;
    job.src[0] = qt;
    job.src[1] = kt;
    job.w[0] = wq;
    job.w[1] = (mode == VSA_SCORE_MEAN_GATE && !wk) ? wq : wk;
    job.bh0 = (int32_t)bh0;
    job.nbh = n;
    if (launch_pool(p, mode, proj_dim, job, 2, slot_to_token, pooled, s) != hipSuccess)
      return VSA_ERR_HIP;
    ScoreJob sj;
    sj.q = pooled;
    sj.q_bh = (int64_t)p.max_vt * r;
    sj.k = pooled + (int64_t)n * p.max_vt * r;
    sj.k_bh = (int64_t)p.max_vt * r;
    sj.ncols = -1;
    sj.out = scores;
    sj.out_row = p.max_vt;
    sj.out_bh = (int64_t)p.max_vt * p.max_vt;
    sj.bh0 = (int32_t)bh0;
    sj.nbh = n;
    if (launch_scores(p, r, sj, s) != hipSuccess) return VSA_ERR_HIP;
  }
  return VSA_OK;
}

}  // extern "C"
