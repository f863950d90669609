"""GPU parity of the teacher tile map (full attention max-pooled per video
tile pair) against the oracle, and of the teacher's top-k."""
import dataclasses

import numpy as np
import pytest

import oracle
from tests import gpu_support as gs
from workloads import WORKLOADS
from workloads.configs import HEAD_AWARE_CYCLE, Workload

pytestmark = pytest.mark.gpu

SMALL = {
    "f32-d64": Workload("teacher-f32", "f32", 1, 2, 64, (4, 8, 12), (40, 24),
                        ((4, 4, 4),), "mean_gate", 0.5, 5101),
    "bf16-headaware": Workload("teacher-bf16", "bf16", 2, 3, 128, (5, 16, 12), (70, 30),
                               HEAD_AWARE_CYCLE, "mean_gate", 0.75, 5102),
}
# fp32 logits and log-sum-exp against float64: the error of x - lse (log2
# units, |x|, |lse| below ~40 here) is a few fp32 ulps of 40, about 1e-5
# absolute, which is the relative error of 2^(x - lse) after a factor ln 2.
REL = 2e-5


def _teacher(w, run):
    import torch
    from block_sparse_video_map_amd import vsa
    sz = run.layer.sizes
    lse = torch.empty(w.B * w.H * sz.max_video_tiles * 64, dtype=torch.float32, device="cuda")
    t = torch.empty(sz.score_elems, dtype=torch.float32, device="cuda")
    vsa.vsa_teacher_map(run.prob, run.layer.qt, run.layer.kt, run.layer.slot_to_token, 0.0,
                        lse, t)
    torch.cuda.synchronize()
    return t.view(w.B * w.H, sz.max_video_tiles, sz.max_video_tiles)


def _compare(w, run, teacher, b, h, rows=None):
    q, k, _ = gs.head_inputs(w, h, b)
    tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
    rows = list(range(tm.n_video_tiles)) if rows is None else rows
    want = oracle.teacher_tile_map(q, k, tm, 1.0 / np.sqrt(w.d), query_tiles=rows)
    got = teacher[b * w.H + h, rows, :tm.n_video_tiles].cpu().numpy().astype(np.float64)
    err = np.abs(got - want) / np.maximum(want, 1e-30)
    tiny = want < 1e-30
    gs.log(f"[teacher] {w.name} b{b} h{h}: rows {len(rows)} max rel err "
           f"{float(err[~tiny].max()):.2e}")
    assert float(err[~tiny].max()) <= REL
    assert np.all(got[tiny] <= 1e-30)
    return want, got


@pytest.mark.parametrize("name", list(SMALL))
def test_teacher_map_full_parity(name):
    from block_sparse_video_map_amd import vsa
    import torch
    w = SMALL[name]
    run = gs.run_library(w, stages=("map",))
    teacher = _teacher(w, run)
    sz = run.layer.sizes
    kv = torch.empty(sz.idx_elems, dtype=torch.int32, device="cuda")
    vsa.vsa_select_topk(run.prob, teacher.reshape(-1), w.sparsity, kv)
    torch.cuda.synchronize()
    kv = kv.view(w.B * w.H, sz.max_video_tiles, sz.k_max).cpu().numpy()
    for b in range(w.B):
        for h in range(w.H):
            want, _ = _compare(w, run, teacher, b, h)
            k = sz.k[h % len(w.tile_shapes)]
            n = want.shape[0]
            differ, wide, fails = gs.band_rule_check(want.astype(np.float32),
                                                     kv[b * w.H + h, :n], k, rel=1e-3)
            assert not fails


def test_teacher_map_headline_sampled():
    w = WORKLOADS["3a"]
    run = gs.run_library(w, stages=("map",))
    teacher = _teacher(w, run)
    rng = np.random.default_rng(11)
    for h in (0, 17):
        rows = sorted(rng.choice(1764, 3, replace=False).tolist())
        _compare(w, run, teacher, 0, h, rows)


def test_recall_of_both_scorers_is_measured_against_the_teacher():
    """Mean-gate and TripPool selections on the same inputs, scored against
    the teacher's top-k (a measurement; the value is reported, not pinned)."""
    import torch
    from block_sparse_video_map_amd import vsa
    w = SMALL["bf16-headaware"]
    wt = dataclasses.replace(w, scorer="trippool")
    rg = gs.run_library(w, stages=("map", "score", "select"))
    rt = gs.run_library(wt, stages=("map", "score", "select"))
    teacher = _teacher(w, rg)
    sz = rg.layer.sizes
    top = torch.empty(sz.idx_elems, dtype=torch.int32, device="cuda")
    vsa.vsa_select_topk(rg.prob, teacher.reshape(-1), w.sparsity, top)
    torch.cuda.synchronize()
    shp = (w.B * w.H, sz.max_video_tiles, sz.k_max)
    top = top.view(*shp).cpu().numpy()
    for name, r in (("mean gate", rg), ("TripPool", rt)):
        sel = r.layer.kv_idx[: sz.idx_elems].view(*shp).cpu().numpy()
        rec = []
        for bh in range(w.B * w.H):
            s = bh % w.H % len(w.tile_shapes)
            n, k = sz.n_video_tiles[s], sz.k[s]
            hits = [len(set(a[:k]) & set(t[:k])) for a, t in zip(sel[bh, :n], top[bh, :n])]
            rec.append(np.mean(hits) / k)
        gs.log(f"[teacher] recall of {name}: {np.mean(rec):.3f}")
        assert 0.0 <= np.mean(rec) <= 1.0
