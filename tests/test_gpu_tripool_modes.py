"""GPU parity of the TripPool statistic modes (tripool_mode maxmin and avg).

The library's double-precision tile descriptors must match the oracle's to
rounding order (1e-12 relative to the descriptor's scale), scores within one
float32 ulp, selections bit-exact under the near-tie band rule, and outputs
(on the GPU's own selections) within the bf16 / fp32 tolerances. Ragged
grids, so edge tiles hold pads; head-aware tile shapes.
"""
import dataclasses

import numpy as np
import pytest

from tests import gpu_support as gs
from workloads.configs import HEAD_AWARE_CYCLE, Workload

pytestmark = pytest.mark.gpu

BASE = {
    "bf16": Workload("tp-modes-bf16", "bf16", 1, 3, 128, (5, 16, 20), (100, 700, 30),
                     HEAD_AWARE_CYCLE, "trippool", 0.8, 4101, proj_dim=32),
    "f32": Workload("tp-modes-f32", "f32", 2, 2, 64, (3, 9, 14), (40, 150, 24),
                    ((4, 4, 4),), "trippool", 0.6, 4102, proj_dim=16),
}
CASES = [(dt, mode) for dt in BASE for mode in ("maxmin", "avg")]


def _check_descriptors(w, r, b, h, orc):
    lay, sz = r.layer, r.layer.sizes
    width = {"maxmin": 2, "avg": 1}[w.tripool_mode] * w.proj_dim
    bh, nbh, nv = b * w.H + h, w.B * w.H, orc["tmap"].n_video_tiles
    pooled = lay.pooled[: 2 * nbh * sz.max_video_tiles * width]
    pooled = pooled.view(2, nbh, sz.max_video_tiles, width).cpu().numpy()
    for got, want, what in ((pooled[0, bh, :nv], orc["qhat"], "Q"),
                            (pooled[1, bh, :nv], orc["khat"], "K")):
        assert want.shape == (nv, width)
        err = float(np.abs(got - want).max())
        scale = float(np.abs(want).max())
        gs.log(f"[tripool] {w.name} {w.tripool_mode} b{b} h{h} {what} descriptors: "
               f"max-abs {err:.2e} (scale {scale:.2e})")
        assert err <= 1e-12 * max(scale, 1.0)


@pytest.mark.parametrize("dt,mode", CASES, ids=[f"{d}-{m}" for d, m in CASES])
def test_tripool_mode_parity(dt, mode):
    w = dataclasses.replace(BASE[dt], tripool_mode=mode)
    gs.log(f"[tripool] {w.name} mode {mode}")
    r = gs.run_library(w)
    lay, sz = r.layer, r.layer.sizes
    nbh = w.B * w.H
    sc = lay.scores.view(nbh, sz.max_video_tiles, sz.max_video_tiles)
    kv = lay.kv_idx[: sz.idx_elems].view(nbh, sz.max_video_tiles, sz.k_max)
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            orc, _ = gs.oracle_head(w, h, b=b, query_tiles=[])
            nv = orc["tmap"].n_video_tiles
            _check_descriptors(w, r, b, h, orc)
            got = sc[bh, :nv, :nv].cpu().numpy()
            ulp = np.abs(got.view(np.int32).astype(np.int64)
                         - orc["scores"].view(np.int32).astype(np.int64))
            assert ulp.max() <= 1
            sel = kv[bh, :nv].cpu().numpy()
            differ, wide, fails = gs.band_rule_check(orc["scores"], sel, orc["k"])
            assert not fails and differ <= wide
            o2, _ = gs.oracle_head(w, h, b=b, query_tiles=None, kv_video=sel[:, :orc["k"]])
            rows = np.nonzero(~np.isnan(o2["out"][:, 0]))[0]
            mx, mean = gs.bf16_stats(gs.tensor_f32(lay.out[b, h])[rows], o2["out"][rows])
            gs.log(f"[tripool] {w.name} {mode} b{b} h{h}: ulp {ulp.max()} "
                   f"max-abs {mx:.2e} mean-abs {mean:.2e}")
            if w.dtype == "f32":
                assert mx <= gs.F32_MAX_ABS
            else:
                assert mx <= gs.BF16_MAX_ABS and mean <= gs.BF16_MEAN_ABS
    # the one-pass gather and pooling writes the same tiles, descriptors and scores
    assert gs.assert_gather_pool_equal(r)


@pytest.mark.parametrize("mode", ["maxmin", "avg"])
def test_tripool_mode_two_stream_reference_scores(mode):
    """The reference stream pools with the same statistics."""
    w = dataclasses.replace(BASE["bf16"], tripool_mode=mode)
    ref = (1, 4)
    r = gs.run_library(w, ref=ref)
    lay, sz = r.layer, r.layer.sizes
    n_ref = lay.ref_scores.numel() // (w.B * w.H * sz.max_video_tiles)
    for h in range(w.H):
        orc, _ = gs.oracle_head(w, h, query_tiles=[], ref=ref)
        nv = orc["tmap"].n_video_tiles
        rs = lay.ref_scores.view(w.B * w.H, sz.max_video_tiles, n_ref)[h, :nv].cpu().numpy()
        ulp = np.abs(rs.view(np.int32).astype(np.int64)
                     - orc["ref_scores"].view(np.int32).astype(np.int64))
        gs.log(f"[tripool] two-stream {mode} h{h}: ref score ulp {ulp.max()}")
        assert ulp.max() <= 1
        rsel = lay.ref_idx.view(w.B * w.H, sz.max_video_tiles, ref[1])[h, :nv].cpu().numpy()
        differ, wide, fails = gs.band_rule_check(orc["ref_scores"], rsel, ref[1])
        assert not fails and differ <= wide
