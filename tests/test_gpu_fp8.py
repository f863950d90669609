"""GPU parity of the fp8 (E4M3) attention variant against the oracle.

The quantizer must be bit-exact: every tile's scale exponent and every E4M3
value equal to oracle.quantize_tiles_e4m3 on the same bf16 tiles. Attention
outputs are compared, on the GPU's own selections, with exact attention over
the oracle's E4M3 inputs, within the fp8 tolerances (the kernel rounds the
probabilities to E4M3; see tests/gpu_support.py). Ragged grids, prefix
segments, head-aware shapes, d = 64 and 128, the two-stream budget, the dense
path and sampled query tiles at the full-clip shape.
"""
import numpy as np
import pytest

import oracle
from tests import gpu_support as gs
from workloads import WORKLOADS
from workloads.configs import HEAD_AWARE_CYCLE, Workload

pytestmark = pytest.mark.gpu

SMALL = {
    "mg-d128": Workload("f8-mg", "bf16", 2, 2, 128, (5, 16, 20), (40, 300, 24),
                        ((4, 4, 4),), "mean_gate", 0.75, 4201),
    "tp-d128": Workload("f8-tp", "bf16", 1, 3, 128, (5, 16, 20), (100, 700, 30),
                        HEAD_AWARE_CYCLE, "trippool", 0.8, 4202),
    "mg-d64": Workload("f8-d64", "bf16", 1, 2, 64, (3, 9, 14), (40, 150, 24),
                       ((4, 4, 4),), "mean_gate", 0.5, 4203),
}


def _run(w, sparsity=None, ref=None):
    import torch
    from block_sparse_video_map_amd import vsa
    sp = w.sparsity if sparsity is None else sparsity
    prob = gs.problem_of(w)
    layer = vsa.Layer(prob, sp, vsa.score_mode(w.scorer, w.tripool_mode),
                      w.d if w.scorer == "mean_gate" else w.proj_dim, ref=ref, fp8=True)
    q, k, v = gs.to_device(w)
    from workloads.inputs import make_weights
    W = make_weights(w)
    if w.scorer == "mean_gate":
        wq, wk = torch.from_numpy(W["gate"]).cuda(), None
    else:
        wq, wk = torch.from_numpy(W["proj_q"]).cuda(), torch.from_numpy(W["proj_k"]).cuda()
    layer.forward(q, k, v, wq, wk)
    torch.cuda.synchronize()
    return layer


def _selection(w, layer, b, h, nv):
    sz = layer.sizes
    kv = layer.kv_idx[: sz.idx_elems].view(w.B * w.H, sz.max_video_tiles, sz.k_max)
    return kv[b * w.H + h, :nv].cpu().numpy()


def _compare(w, layer, b, h, allow, tm, query_tiles=None, label="", arrays=None,
             tol=(gs.FP8_MAX_ABS, gs.FP8_MEAN_ABS, gs.FP8_LSE_ABS)):
    if arrays is None:
        q, k, v = gs.head_inputs(w, h, b)
    else:
        q, k, v = (np.asarray(a[b, h], dtype=np.float64) for a in arrays)
    qq, kq, vq = oracle.fp8_attention_inputs(q, k, v, tm)
    want, lse_want = oracle.sparse_attention(qq, kq, vq, tm, allow, 1.0 / np.sqrt(w.d),
                                             query_tiles)
    rows = np.nonzero(~np.isnan(want[:, 0]))[0]
    got = gs.tensor_f32(layer.out[b, h])[rows]
    mx, mean = gs.bf16_stats(got, want[rows])
    lse_err = float(np.abs(layer.lse[b, h].cpu().numpy()[rows] - lse_want[rows]).max())
    gs.log(f"[fp8] {w.name}{label} b{b} h{h}: rows {rows.size} max-abs {mx:.2e} "
           f"mean-abs {mean:.2e} lse {lse_err:.2e}")
    assert mx <= tol[0] and mean <= tol[1] and lse_err <= tol[2]


@pytest.mark.parametrize("name", list(SMALL))
def test_quantize_fp8_bit_exact(name):
    w = SMALL[name]
    gs.log(f"[fp8] quantize {name}")
    layer = _run(w)
    sz = layer.sizes
    per_head = sz.max_tiles * 64 * w.d
    exps = layer.fp8_scales.cpu().numpy().reshape(w.B * w.H, sz.max_tiles, 4).astype(np.int64)
    exps -= 127
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
            for which, (x, t) in enumerate(zip(gs.head_inputs(w, h, b),
                                               (layer.q8, layer.k8, layer.v8))):
                want, we = oracle.quantize_tiles_e4m3(oracle.gather(x, tm))
                np.testing.assert_array_equal(exps[bh, :tm.n_tiles, which], we)
                codes = t[bh * per_head:(bh + 1) * per_head].cpu().numpy()
                got = gs.unpack_fp8_tiles(codes, exps[bh, :, which], tm.n_tiles, w.d,
                                          col=(which == 2))
                np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_attention_parity(name):
    w = SMALL[name]
    gs.log(f"[fp8] attention {name}")
    layer = _run(w)
    for b in range(w.B):
        for h in range(w.H):
            orc, _ = gs.oracle_head(w, h, b=b, query_tiles=[])
            tm = orc["tmap"]
            sel = _selection(w, layer, b, h, tm.n_video_tiles)
            differ, wide, fails = gs.band_rule_check(orc["scores"], sel, orc["k"])
            assert not fails and differ <= wide
            allow = oracle.allowed_tiles(tm, sel[:, :orc["k"]])
            _compare(w, layer, b, h, allow, tm)


def _extreme_arrays(w, tm):
    """Seeded inputs with tiles that take every branch of the scale rule: all
    zero (e = 0), bf16 subnormals (e clamped to -127), values near the bf16
    maximum (e = 120), and amax exactly 448 * 2^5 (e = 5, no rounding)."""
    from workloads.inputs import bf16_to_f32, bf16_bits
    q, k, v = (np.asarray(a, dtype=np.float32).copy() for a in gs.make_qkv_f32(w))
    npf = tm.n_prefix_tiles
    special = {npf + 0: 0.0, npf + 1: 2.0 ** -130, npf + 2: 3.0e38, npf + 3: 448.0 * 2.0 ** 5}
    rng = np.random.default_rng(9)
    for x in (q, k, v):
        for tile, amp in special.items():
            toks = tm.tile_tokens(tile)
            vals = rng.uniform(-1.0, 1.0, (x.shape[0], x.shape[1], toks.size, w.d)) * amp
            if amp in (448.0 * 2.0 ** 5, 3.0e38):
                vals[..., 0, 0] = amp                      # fixes the tile's amax
            x[:, :, toks, :] = vals
    return [bf16_to_f32(bf16_bits(a)) for a in (q, k, v)]


@pytest.mark.parametrize("fused", [False, True], ids=["quantizer", "fused-gather"])
def test_quantize_fp8_extreme_tiles(fused):
    import torch
    from block_sparse_video_map_amd import vsa
    w = SMALL["mg-d64"]
    tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[0])
    npf = tm.n_prefix_tiles
    arrays = _extreme_arrays(w, tm)
    layer = vsa.Layer(gs.problem_of(w), w.sparsity, vsa.VSA_SCORE_MEAN_GATE, w.d, fp8=True)
    dq, dk, dv = gs.to_device(w, arrays=arrays)
    if fused:
        layer.map_tiles_fp8(dq, dk, dv)
    else:
        layer.map_tiles(dq, dk, dv)
        layer.quantize()
    torch.cuda.synchronize()
    sz = layer.sizes
    per_head = sz.max_tiles * 64 * w.d
    exps = layer.fp8_scales.cpu().numpy().reshape(w.B * w.H, sz.max_tiles, 4).astype(np.int64)
    exps -= 127
    for h in range(w.H):
        for which, (x, t) in enumerate(zip(arrays, (layer.q8, layer.k8, layer.v8))):
            want, we = oracle.quantize_tiles_e4m3(oracle.gather(x[0, h].astype(np.float64), tm))
            got_e = exps[h, :tm.n_tiles, which]
            np.testing.assert_array_equal(got_e, we)
            assert got_e[npf] == 0 and got_e[npf + 1] == -127 and got_e[npf + 2] == 120
            assert got_e[npf + 3] == 5
            codes = t[h * per_head:(h + 1) * per_head].cpu().numpy()
            got = gs.unpack_fp8_tiles(codes, exps[h, :, which], tm.n_tiles, w.d, col=(which == 2))
            np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", ["tp-d128", "mg-d64"])
def test_fused_gather_matches_map_then_quantize(name):
    """vsa_map_tiles_fp8 writes exactly what vsa_map_tiles followed by
    vsa_quantize_fp8 writes: map, bf16 tiles, E4M3 tiles and scale bytes."""
    import torch
    from block_sparse_video_map_amd import vsa
    w = SMALL[name]
    layer = vsa.Layer(gs.problem_of(w), w.sparsity, vsa.score_mode(w.scorer, w.tripool_mode),
                      w.d if w.scorer == "mean_gate" else w.proj_dim, fp8=True)
    dq, dk, dv = gs.to_device(w)
    bufs = (layer.slot_to_token, layer.qt, layer.kt, layer.vt, layer.q8, layer.k8, layer.v8,
            layer.fp8_scales)
    for t in bufs:
        t.zero_()
    layer.map_tiles(dq, dk, dv)
    layer.quantize()
    torch.cuda.synchronize()
    first = [t.clone() for t in bufs]
    for t in bufs:
        t.zero_()
    layer.map_tiles_fp8(dq, dk, dv)
    torch.cuda.synchronize()
    for a, b in zip(first, bufs):
        assert torch.equal(a, b)


def test_fp8_dense_path():
    """sparsity 0: every tile kept, dense attention over the E4M3 inputs."""
    w = SMALL["mg-d64"]
    layer = _run(w, sparsity=0.0)
    for h in range(w.H):
        tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
        allow = np.ones((tm.n_tiles, tm.n_tiles), dtype=bool)
        _compare(w, layer, 0, h, allow, tm, label=" dense")


def test_fp8_two_stream():
    w = SMALL["tp-d128"]
    ref = (1, 4)
    layer = _run(w, ref=ref)
    sz = layer.sizes
    n_ref = layer.ref_scores.numel() // (w.B * w.H * sz.max_video_tiles)
    for h in range(w.H):
        orc, _ = gs.oracle_head(w, h, query_tiles=[], ref=ref)
        tm = orc["tmap"]
        nv = tm.n_video_tiles
        sel = _selection(w, layer, 0, h, nv)[:, :orc["k"]]
        rsel = layer.ref_idx.view(w.B * w.H, sz.max_video_tiles, ref[1])[h, :nv].cpu().numpy()
        assert n_ref == orc["ref_tiles"].size
        allow = oracle.allowed_two_stream(tm, sel, orc["ref_tiles"], rsel)
        _compare(w, layer, 0, h, allow, tm, label=" two-stream")


def test_fp8_full_clip_sampled():
    """The full-clip shape (24 heads, 1,767 tiles, 25% kept): quantizer on
    two heads' sampled tiles, attention on sampled query tiles."""
    import torch
    w = WORKLOADS["3a"]
    gs.log("[fp8] full clip")
    layer = _run(w)
    sz = layer.sizes
    per_head = sz.max_tiles * 64 * w.d
    exps = layer.fp8_scales.cpu().numpy().reshape(w.B * w.H, sz.max_tiles, 4).astype(np.int64)
    exps -= 127
    rng = np.random.default_rng(7)
    for h in (0, 23):
        tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
        q, k, v = gs.head_inputs(w, h)
        tiles = np.sort(rng.choice(tm.n_tiles, 48, replace=False))
        for which, (x, t) in enumerate(zip((q, k, v), (layer.q8, layer.k8, layer.v8))):
            want, we = oracle.quantize_tiles_e4m3(oracle.gather(x, tm)[tiles])
            np.testing.assert_array_equal(exps[h, tiles, which], we)
            codes = t[h * per_head:(h + 1) * per_head].cpu().numpy()
            got = gs.unpack_fp8_tiles(codes, exps[h, :, which], tm.n_tiles, w.d, col=(which == 2))
            np.testing.assert_array_equal(got[tiles], want)
        sel = _selection(w, layer, 0, h, tm.n_video_tiles)
        k_h = oracle.keep_count(w.sparsity, tm.n_video_tiles)
        allow = oracle.allowed_tiles(tm, sel[:, :k_h])
        qt = list(range(tm.n_prefix_tiles)) + sorted(
            int(tm.n_prefix_tiles + i) for i in rng.choice(tm.n_video_tiles, 12, replace=False))
        _compare(w, layer, 0, h, allow, tm, query_tiles=qt, label=" sampled")
    gs.assert_same_without_lse(layer, " fp8 full clip")
    del layer
    torch.cuda.empty_cache()



@pytest.mark.parametrize("sparsity", [0.0, None], ids=["dense", "sparse"])
def test_fp8_rising_max_exact(sparsity):
    """The running max is raised with probabilities pending (see
    gpu_support.rising_exact_arrays); the outputs must match exact attention
    over the same E4M3 inputs to the bf16 rounding of the output, and the LSE
    to float32 accuracy. A wrong rescale of any tile's contribution shows as a
    relative error of at least 2^-1 in that tile's weight."""
    import torch
    from block_sparse_video_map_amd import vsa
    from workloads.inputs import make_weights
    w = SMALL["mg-d128"]
    tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[0])
    arrays = gs.rising_exact_arrays(w, tm)
    sp = w.sparsity if sparsity is None else sparsity
    scale = float(np.log(2.0))
    layer = vsa.Layer(gs.problem_of(w), sp, vsa.VSA_SCORE_MEAN_GATE, w.d, fp8=True)
    dq, dk, dv = gs.to_device(w, arrays=arrays)
    wq = torch.from_numpy(make_weights(w)["gate"]).cuda()
    gs.log(f"[fp8] rising max, sparsity {sp}")
    layer.forward(dq, dk, dv, wq, None, softmax_scale=scale)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            if sp == 0.0:
                allow = np.ones((tm.n_tiles, tm.n_tiles), dtype=bool)
            else:
                sel = _selection(w, layer, b, h, tm.n_video_tiles)
                allow = oracle.allowed_tiles(tm, sel[:, :oracle.keep_count(sp, tm.n_video_tiles)])
            q, k, v = (np.asarray(x[b, h], dtype=np.float64) for x in arrays)
            qq, kq, vq = oracle.fp8_attention_inputs(q, k, v, tm)
            want, lse_want = oracle.sparse_attention(qq, kq, vq, tm, allow, scale, None)
            rows = np.nonzero(~np.isnan(want[:, 0]))[0]
            got = gs.tensor_f32(layer.out[b, h])[rows]
            err = np.abs(got - want[rows])
            bound = 2.0 ** -8 * np.abs(want[rows]) + 1e-4
            lse_err = float(np.abs(layer.lse[b, h].cpu().numpy()[rows] - lse_want[rows]).max())
            gs.log(f"[fp8] rising max b{b} h{h}: rows {rows.size} max-abs {err.max():.2e} "
                   f"worst/bound {(err / bound).max():.2f} lse {lse_err:.2e}")
            assert np.all(err <= bound)
            assert lse_err <= 1e-4 * float(np.abs(lse_want[rows]).max()) + 1e-5



@pytest.mark.parametrize("name", ["ragged-headaware-b2", "no-prefix-d64", "keep-all", "top-1",
                                  "proj64-many-shapes"])
def test_fp8_edge_workloads(name):
    """The fp8 path on the edge workloads of the bf16 tests: ragged grids,
    head-aware and mixed tile shapes, no prefix, k = 1 (a key split with one
    step or none) and keep-all, on the GPU's own selection. Their rows see
    192 to 768 keys, hence the tolerances for short rows."""
    from tests.test_gpu_edge import EDGE
    w = EDGE[name]
    gs.log(f"[fp8] edge {name}")
    layer = _run(w)
    for b in range(w.B):
        for h in range(w.H):
            tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
            sel = _selection(w, layer, b, h, tm.n_video_tiles)
            allow = oracle.allowed_tiles(tm, sel[:, :oracle.keep_count(w.sparsity,
                                                                       tm.n_video_tiles)])
            _compare(w, layer, b, h, allow, tm, label=" edge",
                     tol=(gs.FP8_EDGE_MAX_ABS, gs.FP8_EDGE_MEAN_ABS, gs.FP8_EDGE_LSE_ABS))



def test_fp8_long_rows_in_chunks():
    """Workload 5's shapes (3,853 to 4,105 tiles per head, three heads, one
    per shape): a prefix query tile keeps every key tile, more than one
    chunk of the kernel's step lists (2,048 tiles), so its rows run over two
    chunks. Sampled prefix and video query tiles against the oracle on the
    GPU's own selection."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["5"], H=3)
    gs.log("[fp8] long rows")
    layer = _run(w)
    rng = np.random.default_rng(5)
    for h in range(w.H):
        tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
        assert tm.n_tiles > 2048
        sel = _selection(w, layer, 0, h, tm.n_video_tiles)
        allow = oracle.allowed_tiles(tm, sel[:, :oracle.keep_count(w.sparsity, tm.n_video_tiles)])
        qt = [0, 1, tm.n_prefix_tiles - 1] + sorted(
            int(tm.n_prefix_tiles + i) for i in rng.choice(tm.n_video_tiles, 4, replace=False))
        _compare(w, layer, 0, h, allow, tm, query_tiles=qt, label=" long rows")



def test_fp8_unpaired_long_video_rows():
    """The fp8 kernel's unpaired video rows: the full clip at 30% sparsity
    keeps 1,235 video tiles per row, past the 1,024 of a merged pair list."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["3a"], H=2)
    sp = 0.3
    layer = _run(w, sparsity=sp)
    rng = np.random.default_rng(3)
    for h in range(w.H):
        tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
        k = oracle.keep_count(sp, tm.n_video_tiles)
        assert tm.n_prefix_tiles + k > 1024
        sel = _selection(w, layer, 0, h, tm.n_video_tiles)
        allow = oracle.allowed_tiles(tm, sel[:, :k])
        qt = list(range(tm.n_prefix_tiles)) + sorted(
            int(tm.n_prefix_tiles + i) for i in rng.choice(tm.n_video_tiles, 6, replace=False))
        _compare(w, layer, 0, h, allow, tm, query_tiles=qt, label=" unpaired")
