"""vsa_tile_scores_noalloc (no workspace; the library's fixed device array)
against vsa_tile_scores (caller workspace) through the C ABI: two calls in a
row, the second on a smaller problem. The same kernels pool and score every
(batch, head), so the two score matrices must be bit-identical.

The first call is large enough that its descriptors take more than one chunk
of the fixed array; the second, smaller call must not see anything the first
one left behind.
"""
import dataclasses

import numpy as np
import pytest

from tests import gpu_support as gs
from workloads import WORKLOADS, Workload

pytestmark = pytest.mark.gpu

# 3a's grid with B = 2, H = 6: 12 (batch, head) pairs of 2 x 1764 x 128
# doubles (3.6 MB) each, more than the 32 MiB array holds at once.
LARGE = Workload("noalloc-large", "bf16", 2, 6, 128, (28, 48, 84), (40, 64, 24),
                 ((4, 4, 4),), "mean_gate", 0.75, 7101)
SMALL = dataclasses.replace(WORKLOADS["4a"], H=6, seed=7102)


def _both(w):
    import torch
    from block_sparse_video_map_amd import vsa
    r = gs.run_library(w, stages=("map",))
    L = r.layer
    mode = vsa.score_mode(w.scorer, w.tripool_mode)
    proj = w.d if w.scorer == "mean_gate" else w.proj_dim
    ref = torch.full_like(L.scores, float("nan"))
    got = torch.full_like(L.scores, float("nan"))
    vsa.vsa_tile_scores(r.prob, mode, proj, L.qt, L.kt, L.slot_to_token, r.wq, r.wk, L.pooled,
                        ref)
    vsa.vsa_tile_scores_noalloc(r.prob, mode, proj, L.qt, L.kt, L.slot_to_token, r.wq, r.wk,
                                got)
    torch.cuda.synchronize()
    sz = L.sizes
    nv = sz.max_video_tiles
    ref = ref.view(w.B * w.H, nv, nv).cpu().numpy()
    got = got.view(w.B * w.H, nv, nv).cpu().numpy()
    return r, ref, got


def _check(w, ref, got, sizes):
    ns = len(w.tile_shapes)
    for bh in range(w.B * w.H):
        n = sizes.n_video_tiles[bh % w.H % ns]
        a, b = ref[bh, :n, :n], got[bh, :n, :n]
        assert np.isfinite(a).all()
        np.testing.assert_array_equal(b, a)


def test_noalloc_scores_equal_workspace_scores_two_calls():
    from block_sparse_video_map_amd import vsa
    per_bh = 2 * 1764 * 128 * 8
    assert LARGE.B * LARGE.H * per_bh > vsa.VSA_NOALLOC_SCRATCH_BYTES    # several chunks
    gs.log("[noalloc] call 1: large mean-gate problem")
    r1, ref1, got1 = _both(LARGE)
    _check(LARGE, ref1, got1, r1.layer.sizes)
    del r1
    gs.log("[noalloc] call 2: smaller TripPool problem")
    r2, ref2, got2 = _both(SMALL)
    assert r2.layer.sizes.max_video_tiles < 1764
    _check(SMALL, ref2, got2, r2.layer.sizes)
    gs.log("[noalloc] both calls equal")
