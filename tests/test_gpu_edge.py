"""GPU edge cases against the oracle: ragged grids and padded tiles, batch > 1,
no prefix, d = 64, fp32 at d = 128, k = 1 and k = n, the dense path, exact
ties, determinism and batch independence. Every case is small enough for the
oracle to check all heads and all query tiles."""
import numpy as np
import pytest

import oracle
from tests import gpu_support as gs
from workloads import Workload
from workloads.configs import HEAD_AWARE_CYCLE

pytestmark = pytest.mark.gpu

EDGE = {
    # grid 5x12x10 is a multiple of no shape edge: every shape pads, (16,2,2)
    # leaves tiles less than a third full; zero-length middle prefix segment.
    "ragged-headaware-b2": Workload("edge-ragged", "bf16", 2, 3, 128, (5, 12, 10), (7, 0, 70),
                                    HEAD_AWARE_CYCLE, "trippool", 0.7, 2001, proj_dim=16),
    "no-prefix-d64": Workload("edge-d64", "bf16", 1, 2, 64, (4, 16, 12), (),
                              ((4, 4, 4),), "mean_gate", 0.5, 2002),
    "f32-d128-proj8": Workload("edge-f32", "f32", 1, 2, 128, (4, 8, 12), (33,),
                               ((2, 4, 8),), "trippool", 0.6, 2003, proj_dim=8),
    "keep-all": Workload("edge-keep-all", "bf16", 1, 2, 128, (4, 8, 8), (40, 64, 24),
                         ((4, 4, 4),), "mean_gate", 0.0001, 2004),
    "top-1": Workload("edge-top1", "bf16", 1, 2, 128, (8, 16, 16), (100,),
                      ((4, 4, 4), (1, 8, 8)), "mean_gate", 0.999, 2005),
    "proj64-many-shapes": Workload("edge-p64", "bf16", 1, 4, 128, (8, 8, 16), (5, 64, 1),
                                   ((4, 4, 4), (8, 4, 2), (2, 4, 8), (4, 8, 2)),
                                   "trippool", 0.75, 2006, proj_dim=64),
    # the ragged head-aware case at a descriptor width the fused select takes
    "ragged-headaware-b2-p32": Workload("edge-ragged32", "bf16", 2, 3, 128, (5, 12, 10),
                                        (7, 0, 70), HEAD_AWARE_CYCLE, "trippool", 0.7, 2010,
                                        proj_dim=32),
}


def _full_check(w, run, arrays=None, sparsity=None):
    sz = run.layer.sizes
    kv = run.layer.kv_idx[: sz.idx_elems].view(w.B * w.H, sz.max_video_tiles, sz.k_max)
    nv = sz.max_video_tiles
    sc = run.layer.scores.view(w.B * w.H, nv, nv)
    sp = w.sparsity if sparsity is None else sparsity
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            r, _ = gs.oracle_head(w, h, b=b, arrays=arrays, sparsity=sp,
                                  query_tiles=None)
            tm = r["tmap"]
            n, k = tm.n_video_tiles, r["k"]
            if sp != 0.0:
                got_s = sc[bh, :n, :n].cpu().numpy()
                ulp = np.abs(got_s.view(np.int32).astype(np.int64)
                             - r["scores"].view(np.int32).astype(np.int64))
                assert ulp.max() <= 1
                got_k = kv[bh, :n].cpu().numpy()
                differ, wide, fails = gs.band_rule_check(r["scores"], got_k, k)
                assert not fails and differ <= wide
                assert differ == 0, "seeded edge inputs should have no near-ties"
            rows = np.nonzero(~np.isnan(r["out"][:, 0]))[0]
            assert rows.size == w.N
            got = gs.tensor_f32(run.layer.out[b, h])
            mx, mean = gs.bf16_stats(got, r["out"])
            lse_err = float(np.abs(run.layer.lse[b, h].cpu().numpy() - r["lse"]).max())
            gs.log(f"[edge] {w.name} b{b} h{h}: max-abs {mx:.2e} mean-abs {mean:.2e} "
                   f"lse {lse_err:.2e}")
            if w.dtype == "f32":
                assert mx <= gs.F32_MAX_ABS and lse_err <= gs.F32_MAX_ABS
            else:
                assert mx <= gs.BF16_MAX_ABS and mean <= gs.BF16_MEAN_ABS
                assert lse_err <= gs.BF16_LSE_ABS


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_workload_full_parity(name):
    w = EDGE[name]
    gs.log(f"[edge] {name}")
    run = gs.run_library(w)
    # tile maps and gathers, all shapes and heads
    sz = run.layer.sizes
    s2t = run.layer.slot_to_token.cpu().numpy().reshape(len(w.tile_shapes), -1)
    per_head = sz.max_tiles * 64 * w.d
    for si, shape in enumerate(w.tile_shapes):
        tm = oracle.tile_map(*w.grid, w.prefix, shape)
        np.testing.assert_array_equal(s2t[si, : tm.slot_to_token.size], tm.slot_to_token)
        assert (s2t[si, tm.slot_to_token.size:] == -1).all()
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = gs.head_inputs(w, h, b)
            tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
            bh = b * w.H + h
            for x, t, col in ((q, run.layer.qt, False), (k, run.layer.kt, False),
                              (v, run.layer.vt, True)):
                flat = gs.tensor_f32(t[bh * per_head:(bh + 1) * per_head])
                np.testing.assert_array_equal(gs.unpack_tiles(flat, tm.n_tiles, w.d, col),
                                              oracle.gather(x, tm))
    _full_check(w, run)
    gs.assert_fused_equal(run)
    gs.assert_gather_pool_equal(run)


def test_dense_path_equals_dense_attention():
    w = Workload("edge-dense", "bf16", 1, 2, 128, (4, 8, 16), (40, 64, 24), ((4, 4, 4),),
                 "mean_gate", 0.0, 2007)
    run = gs.run_library(w, sparsity=0.0)
    for h in range(w.H):
        q, k, v = gs.head_inputs(w, h)
        o, lse = oracle.dense_attention(q, k, v, gs.default_scale(w.d))
        got = gs.tensor_f32(run.layer.out[0, h])
        mx, mean = gs.bf16_stats(got, o)
        gs.log(f"[edge] dense h{h}: max-abs {mx:.2e} mean-abs {mean:.2e}")
        assert mx <= gs.BF16_MAX_ABS and mean <= gs.BF16_MEAN_ABS
        assert np.abs(run.layer.lse[0, h].cpu().numpy() - lse).max() <= gs.BF16_LSE_ABS


def test_exact_ties_go_to_lower_index():
    """Video key tiles with identical K content score exactly equal for every
    query tile; the lower tile index must be kept."""
    from workloads.inputs import make_qkv
    w = Workload("edge-ties", "bf16", 1, 2, 128, (4, 8, 16), (40,), ((4, 4, 4),),
                 "mean_gate", 0.75, 2008)
    q, k, v = make_qkv(w)
    tm = oracle.tile_map(*w.grid, w.prefix, (4, 4, 4))
    npf = tm.n_prefix_tiles
    # copy K of video tile 1 into video tiles 3 and 6 and tile 0 into 7 (slot by slot)
    for src, dst in ((1, 3), (1, 6), (0, 7)):
        k[:, :, tm.tile_tokens(npf + dst)] = k[:, :, tm.tile_tokens(npf + src)]
    arrays = (q, k, v)
    run = gs.run_library(w, arrays=arrays)
    sz = run.layer.sizes
    kv = run.layer.kv_idx[: sz.idx_elems].view(w.H, sz.max_video_tiles, sz.k_max)
    sc = run.layer.scores.view(w.H, sz.max_video_tiles, sz.max_video_tiles)
    for h in range(w.H):
        r, _ = gs.oracle_head(w, h, arrays=arrays)
        s = sc[h, :8, :8].cpu().numpy()
        assert (s[:, 1] == s[:, 3]).all() and (s[:, 1] == s[:, 6]).all()
        assert (s[:, 0] == s[:, 7]).all()
        got = kv[h, :8, :sz.k[0]].cpu().numpy()
        differ, wide, fails = gs.band_rule_check(r["scores"], got, sz.k[0])
        assert not fails
        for row in got:      # never a later duplicate without the earlier one
            assert not (3 in row or 6 in row) or 1 in row
            assert 7 not in row or 0 in row
    assert gs.assert_fused_equal(run)
    assert gs.assert_gather_pool_equal(run)


def test_deterministic_and_batch_independent():
    w = Workload("edge-det", "bf16", 2, 2, 128, (4, 8, 16), (40, 64), ((4, 4, 4),),
                 "mean_gate", 0.5, 2009)
    from workloads.inputs import make_qkv
    arrays = make_qkv(w)
    a = gs.run_library(w, arrays=arrays)
    b = gs.run_library(w, arrays=arrays)
    for name in ("out", "lse", "kv_idx", "scores", "qt", "vt"):
        x, y = getattr(a.layer, name), getattr(b.layer, name)
        assert x.equal(y), name
    w1 = Workload("edge-det1", "bf16", 1, 2, 128, (4, 8, 16), (40, 64), ((4, 4, 4),),
                  "mean_gate", 0.5, 2009)
    for bi in range(2):
        single = tuple(x[bi:bi + 1] for x in arrays)
        c = gs.run_library(w1, arrays=single)
        assert c.layer.out[0].equal(a.layer.out[bi])
        assert c.layer.lse[0].equal(a.layer.lse[bi])


def test_bf16_rising_max_exact():
    """The bf16 kernel raises its running max lazily: a unit whose
    probability sum passes 2^8 is redone against the raised max. On
    gpu_support.rising_exact_arrays (integer logits in log2 units with
    softmax scale ln 2, lifted by about 2 per key tile) every probability is
    an exact power of two and the max is raised again and again; the outputs
    must match exact attention to the bf16 rounding of the output, dense and
    on the GPU's own selection."""
    import torch
    from block_sparse_video_map_amd import vsa
    from workloads.inputs import make_weights
    w = Workload("edge-rising", "bf16", 2, 2, 128, (5, 16, 20), (40, 300, 24), ((4, 4, 4),),
                 "mean_gate", 0.75, 2011)
    tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[0])
    arrays = gs.rising_exact_arrays(w, tm)
    scale = float(np.log(2.0))
    dq, dk, dv = gs.to_device(w, arrays=arrays)
    wq = torch.from_numpy(make_weights(w)["gate"]).cuda()
    for sp in (0.0, w.sparsity):
        gs.log(f"[edge] bf16 rising max, sparsity {sp}")
        layer = vsa.Layer(gs.problem_of(w), sp, vsa.VSA_SCORE_MEAN_GATE, w.d)
        layer.forward(dq, dk, dv, wq, None, softmax_scale=scale)
        torch.cuda.synchronize()
        sz = layer.sizes
        for b in range(w.B):
            for h in range(w.H):
                if sp == 0.0:
                    allow = np.ones((tm.n_tiles, tm.n_tiles), dtype=bool)
                else:
                    kv = layer.kv_idx[: sz.idx_elems].view(w.B * w.H, sz.max_video_tiles,
                                                           sz.k_max)
                    sel = kv[b * w.H + h, :tm.n_video_tiles].cpu().numpy()
                    allow = oracle.allowed_tiles(
                        tm, sel[:, :oracle.keep_count(sp, tm.n_video_tiles)])
                q, k, v = (np.asarray(x[b, h], dtype=np.float64) for x in arrays)
                want, lse_want = oracle.sparse_attention(q, k, v, tm, allow, scale, None)
                rows = np.nonzero(~np.isnan(want[:, 0]))[0]
                got = gs.tensor_f32(layer.out[b, h])[rows]
                err = np.abs(got - want[rows])
                bound = 2.0 ** -8 * np.abs(want[rows]) + 1e-4
                lse_err = float(np.abs(layer.lse[b, h].cpu().numpy()[rows]
                                       - lse_want[rows]).max())
                gs.log(f"[edge] bf16 rising max b{b} h{h}: rows {rows.size} "
                       f"max-abs {err.max():.2e} worst/bound {(err / bound).max():.2f} "
                       f"lse {lse_err:.2e}")
                assert np.all(err <= bound)
                assert lse_err <= 1e-4 * float(np.abs(lse_want[rows]).max()) + 1e-5


def test_unpaired_long_video_rows():
    """Video query tiles are paired only while a row's list fits one merged
    list (1,024 key tiles); the full clip at 30% sparsity keeps 1,235 video
    tiles per row, so each video query tile runs alone, its list built in
    chunks. Sampled query tiles against the oracle on the GPU's selection."""
    import dataclasses
    from workloads import WORKLOADS
    w = dataclasses.replace(WORKLOADS["3a"], H=2)
    sp = 0.3
    run = gs.run_library(w, sparsity=sp)
    sz = run.layer.sizes
    kv = run.layer.kv_idx[: sz.idx_elems].view(w.B * w.H, sz.max_video_tiles, sz.k_max)
    rng = np.random.default_rng(3)
    for h in range(w.H):
        tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
        k = oracle.keep_count(sp, tm.n_video_tiles)
        assert tm.n_prefix_tiles + k > 1024
        tiles = list(range(tm.n_prefix_tiles)) + sorted(
            int(tm.n_prefix_tiles + i) for i in rng.choice(tm.n_video_tiles, 6, replace=False))
        gpu_sel = kv[h, : tm.n_video_tiles, :k].cpu().numpy()
        ro, _ = gs.oracle_head(w, h, sparsity=sp, query_tiles=tiles, kv_video=gpu_sel)
        rows = np.concatenate([tm.tile_tokens(t) for t in tiles])
        got = gs.tensor_f32(run.layer.out[0, h])[rows]
        mx, mean = gs.bf16_stats(got, ro["out"][rows])
        lse_err = float(np.abs(run.layer.lse[0, h].cpu().numpy()[rows] - ro["lse"][rows]).max())
        gs.log(f"[edge] unpaired rows h{h}: max-abs {mx:.2e} mean-abs {mean:.2e} lse {lse_err:.2e}")
        assert mx <= gs.BF16_MAX_ABS and mean <= gs.BF16_MEAN_ABS
        assert lse_err <= gs.BF16_LSE_ABS
