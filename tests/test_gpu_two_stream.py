"""GPU parity of the two-stream budget (reference-to-video) against the oracle.

One prefix segment (the reference image) is a second sparse stream with its
own top-k per video query tile; text and audio stay dense keys and prefix
rows stay dense. Reference scores must be within one float32 ulp of the
oracle's; both selections bit-exact under the near-tie band rule; outputs
within the bf16 / fp32 tolerances, compared on the GPU's own selections.
"""
import numpy as np
import pytest

from tests import gpu_support as gs
from workloads import WORKLOADS
from workloads.configs import HEAD_AWARE_CYCLE, Workload

pytestmark = pytest.mark.gpu

SMALL = {
    "mean-gate-bf16": (Workload("ts-mg", "bf16", 2, 3, 128, (4, 16, 16), (40, 300, 24),
                                ((4, 4, 4),), "mean_gate", 0.75, 4001), (1, 2)),
    "trippool-bf16": (Workload("ts-tp", "bf16", 1, 3, 128, (5, 16, 20), (100, 700, 30),
                               HEAD_AWARE_CYCLE, "trippool", 0.8, 4002), (1, 4)),
    "mean-gate-f32": (Workload("ts-f32", "f32", 1, 2, 64, (4, 8, 8), (40, 150, 24),
                               ((4, 4, 4),), "mean_gate", 0.5, 4003), (1, 1)),
}


def _check_head(w, r, b, h, ref, query_tiles=None):
    """Compares head (b, h) of the library run with the oracle."""
    lay = r.layer
    sz = lay.sizes
    bh = b * w.H + h
    n_ref = lay.ref_scores.numel() // (w.B * w.H * sz.max_video_tiles)
    k_ref = ref[1]
    orc, _ = gs.oracle_head(w, h, b=b, query_tiles=[], ref=ref)
    tm = orc["tmap"]
    nv = tm.n_video_tiles
    # reference scores and both selections
    rs = lay.ref_scores.view(w.B * w.H, sz.max_video_tiles, n_ref)[bh, :nv].cpu().numpy()
    ulp = np.abs(rs.view(np.int32).astype(np.int64)
                 - orc["ref_scores"].view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    rsel = lay.ref_idx.view(w.B * w.H, sz.max_video_tiles, k_ref)[bh, :nv].cpu().numpy()
    differ, wide, fails = gs.band_rule_check(orc["ref_scores"], rsel, k_ref)
    assert not fails and differ <= wide
    kv = lay.kv_idx[: sz.idx_elems].view(w.B * w.H, sz.max_video_tiles, sz.k_max)
    vsel = kv[bh, :nv].cpu().numpy()
    differ, wide, fails = gs.band_rule_check(orc["scores"], vsel, orc["k"])
    assert not fails and differ <= wide
    # outputs on the GPU's selections
    qt = list(range(tm.n_tiles)) if query_tiles is None else query_tiles
    o2, _ = gs.oracle_head(w, h, b=b, query_tiles=qt, ref=ref,
                           kv_video=vsel[:, :orc["k"]], kv_ref=rsel)
    rows = np.nonzero(~np.isnan(o2["out"][:, 0]))[0]
    got = gs.tensor_f32(lay.out[b, h])[rows]
    mx, mean = gs.bf16_stats(got, o2["out"][rows])
    lse_err = float(np.abs(lay.lse[b, h].cpu().numpy()[rows] - o2["lse"][rows]).max())
    gs.log(f"[two-stream] {w.name} b{b} h{h}: ref k={k_ref}/{n_ref} rows {rows.size} "
           f"max-abs {mx:.2e} mean-abs {mean:.2e} lse {lse_err:.2e}")
    if w.dtype == "f32":
        assert mx <= gs.F32_MAX_ABS and lse_err <= gs.F32_MAX_ABS
    else:
        assert mx <= gs.BF16_MAX_ABS and mean <= gs.BF16_MEAN_ABS
        assert lse_err <= gs.BF16_LSE_ABS


@pytest.mark.parametrize("name", list(SMALL))
def test_two_stream_full_parity(name):
    w, ref = SMALL[name]
    gs.log(f"[two-stream] {name}")
    r = gs.run_library(w, ref=ref)
    for b in range(w.B):
        for h in range(w.H):
            _check_head(w, r, b, h, ref)


def test_two_stream_full_reference_budget_equals_single_stream():
    """Keeping every reference tile allows the same keys as the single-stream
    path; only the order of the key list (hence fp32 summation order)
    differs."""
    w, _ = SMALL["mean-gate-bf16"]
    r1 = gs.run_library(w, ref=(1, 5))              # the whole segment: 5 tiles
    out1 = gs.tensor_f32(r1.layer.out)
    del r1
    r0 = gs.run_library(w)
    out0 = gs.tensor_f32(r0.layer.out)
    mx, mean = gs.bf16_stats(out1, out0.astype(np.float64))
    gs.log(f"[two-stream] full budget vs single stream: max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert mx <= 2.0 ** -7 and mean <= 1e-3


def test_two_stream_headline_shape():
    """3b's shape with the pages' R2VA budget: 32 reference tiles (of 63) and
    32 video tiles (of 1764) per video query tile."""
    base = WORKLOADS["3b"]
    w = Workload("3b-r2va", base.dtype, base.B, base.H, base.d, base.grid, base.prefix,
                 base.tile_shapes, base.scorer, 0.9819, base.seed)
    ref = (1, 32)
    r = gs.run_library(w, ref=ref)
    assert r.layer.sizes.k[0] == 32
    rng = np.random.default_rng(7)
    for h in (0, 23):
        npt = 73
        qt = list(range(npt)) + list(npt + rng.choice(1764, 16, replace=False))
        _check_head(w, r, 0, h, ref, query_tiles=qt)
    gs.assert_same_without_lse(r.layer, " two-stream 3b")
