"""The C-ABI library on the host: it loads, exports every declared symbol,
plans sizes correctly and rejects bad arguments before any launch (CPU only;
no compute call is made)."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from block_sparse_video_map_amd import vsa
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")


def _problem(w, **kw):
    args = dict(B=w.B, H=w.H, d=w.d, grid=w.grid, prefix=w.prefix,
                tile_shapes=w.tile_shapes, dtype=w.dtype)
    args.update(kw)
    return vsa.Problem(**args)


def test_every_declared_symbol_is_exported():
    decl = re.findall(r"VSA_API\s+[^;(]*?\b(vsa_\w+)\s*\(", open(HEADER).read())
    assert set(decl) == set(vsa.EXPORTS)
    L = vsa.lib()
    for name in decl:
        assert hasattr(L, name), name
    assert vsa.vsa_version() == 100


def test_struct_layout_matches_header(tmp_path):
    """ctypes mirrors of the structs agree with the C compiler's layout."""
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "vsa.h"\n'
        'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(vsa_problem),'
        ' offsetof(vsa_problem, tile_shape), offsetof(vsa_problem, dtype),'
        ' sizeof(vsa_sizes), offsetof(vsa_sizes, keep_bp), offsetof(vsa_sizes, k));'
        ' return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(vsa.vsa_problem), vsa.vsa_problem.tile_shape.offset,
            vsa.vsa_problem.dtype.offset, ctypes.sizeof(vsa.vsa_sizes),
            vsa.vsa_sizes.keep_bp.offset, vsa.vsa_sizes.k.offset]
    assert got == want


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_sizes_agree_with_oracle_counts(name):
    w = WORKLOADS[name]
    sz = vsa.vsa_query_sizes(_problem(w), w.sparsity)
    tms = [oracle.tile_map(*w.grid, w.prefix, s) for s in w.tile_shapes]
    assert sz.n_prefix_tiles == tms[0].n_prefix_tiles
    for i, tm in enumerate(tms):
        assert sz.n_tiles[i] == tm.n_tiles
        assert sz.n_video_tiles[i] == tm.n_video_tiles
        assert sz.k[i] == oracle.keep_count(w.sparsity, tm.n_video_tiles)
    assert sz.max_tiles == max(t.n_tiles for t in tms)
    assert sz.tiled_elems == w.B * w.H * sz.max_tiles * 64 * w.d
    assert sz.out_elems == w.B * w.H * w.N * w.d


def test_headline_counts():
    w = WORKLOADS["3a"]
    sz = vsa.vsa_query_sizes(_problem(w), 0.75)
    assert (sz.n_prefix_tiles, sz.n_video_tiles[0], sz.k[0]) == (3, 1764, 441)
    kept, frac = vsa.vsa_kept_stats(_problem(w), 0.75)
    assert kept == 24 * (3 * 1767 + 1764 * (3 + 441))
    assert abs(frac - (3 * 1767 + 1764 * 444) / 1767 ** 2) < 1e-12
    kept0, frac0 = vsa.vsa_kept_stats(_problem(w), 0.0)
    assert frac0 == 1.0


def test_keep_counts_match_oracle_over_a_sweep():
    for sp in np.linspace(0, 0.999, 97):
        for n in (1, 3, 4, 17, 504, 1764, 3780, 4032):
            p = vsa.Problem(1, 1, 64, (1, 1, n), (), ((1, 1, 64),), "bf16") if n <= 8192 else None
            sz = vsa.vsa_query_sizes(p, float(sp))
            tiles = (n + 63) // 64
            assert sz.k[0] == oracle.keep_count(float(sp), tiles)


def test_count_flops_matches_oracle_on_host_arrays():
    w = WORKLOADS["1"]
    p = _problem(w)
    tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[0])
    rng = np.random.default_rng(0)
    sz = vsa.vsa_query_sizes(p, 0.5)
    kv = np.full((w.B * w.H, sz.max_video_tiles, sz.k_max), -1, dtype=np.int32)
    sels = []
    for h in range(w.H):
        sel = np.sort(np.stack([rng.choice(tm.n_video_tiles, sz.k[0], replace=False)
                                for _ in range(tm.n_video_tiles)]), axis=1)
        kv[h, :, :sz.k[0]] = sel
        sels.append(sel)
    s2t = tm.slot_to_token.astype(np.int32)
    got = vsa.vsa_count_flops(p, 0.5, s2t, kv)
    want = sum(oracle.effective_flops(tm, oracle.allowed_tiles(tm, s), w.d) for s in sels)
    assert got == want
    dense = vsa.vsa_count_flops(p, 0.0, s2t, None)
    assert dense == w.H * 4 * w.d * w.N * w.N


@pytest.mark.parametrize("change,status", [
    (dict(d=96), vsa.VSA_ERR_UNSUPPORTED),
    (dict(dtype="f16"), None),
    (dict(tile_shapes=((4, 4, 5),)), vsa.VSA_ERR_INVALID_ARG),
    (dict(tile_shapes=((0, 8, 8),)), vsa.VSA_ERR_INVALID_ARG),
    (dict(N=999), vsa.VSA_ERR_INVALID_ARG),
    (dict(grid=(0, 8, 8)), vsa.VSA_ERR_INVALID_ARG),
    (dict(prefix=(-1,)), vsa.VSA_ERR_INVALID_ARG),
    (dict(grid=(1, 1, 64 * 8193), prefix=(), tile_shapes=((1, 1, 64),)), vsa.VSA_ERR_SIZE),
    # 8192 video tiles plus 8193 prefix tiles: more tiles per head than VSA_MAX_TILES
    (dict(grid=(1, 1, 64 * 8192), prefix=(64 * 8193,), tile_shapes=((1, 1, 64),)),
     vsa.VSA_ERR_SIZE),
])
def test_invalid_problems_rejected(change, status):
    w = WORKLOADS["1"]
    p = _problem(w, **change)
    if status is None:            # unknown dtype string maps to f32 here: still valid
        vsa.vsa_query_sizes(p, 0.75)
        return
    with pytest.raises(vsa.VSAError) as e:
        vsa.vsa_query_sizes(p, 0.75)
    assert e.value.status == status


@pytest.mark.parametrize("sp", [-0.1, 1.0, 1.5, math.nan, math.inf])
def test_sparsity_out_of_range(sp):
    with pytest.raises(vsa.VSAError) as e:
        vsa.vsa_query_sizes(_problem(WORKLOADS["1"]), sp)
    assert e.value.status == vsa.VSA_ERR_INVALID_ARG


def test_null_arguments_rejected_before_launch():
    """Every device entry point returns an error on null/misaligned buffers
    without touching the GPU (these calls never reach a launch). Runs only
    where no GPU is visible, so that a validation bug can never turn the fake
    pointers below into a real launch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check; skipped where a GPU is visible")
    L = vsa.lib()
    p = _problem(WORKLOADS["1"])
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: rejected first
    odd = ctypes.c_void_p(0x10008)
    assert L.vsa_map_tiles(None, fake, fake, fake, fake, fake, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_map_tiles(p.ref, fake, fake, fake, None, fake, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_map_tiles(p.ref, fake, None, fake, fake, fake, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_map_tiles(p.ref, odd, fake, fake, fake, fake, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_tile_scores(p.ref, 0, 64, fake, fake, fake, None, None, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_tile_scores(p.ref, 0, 32, fake, fake, fake, fake, None, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_tile_scores(p.ref, 1, 24, fake, fake, fake, fake, fake, fake, fake, None) \
        == vsa.VSA_ERR_UNSUPPORTED
    assert L.vsa_tile_scores(p.ref, 1, 32, fake, fake, fake, fake, None, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_tile_scores(p.ref, 7, 64, fake, fake, fake, fake, None, fake, fake, None) \
        == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_select_topk(p.ref, None, 0.75, fake, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_select_topk(p.ref, fake, 1.0, fake, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_sparse_attn_fwd(p.ref, fake, fake, fake, fake, None, 0.75, 0.0, fake, None,
                                 None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_sparse_attn_fwd(p.ref, fake, fake, fake, fake, fake, 0.75,
                                 float("nan"), fake, None, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_sparse_attn_fwd(p.ref, fake, fake, odd, fake, fake, 0.75, 0.0, fake, None,
                                 None) == vsa.VSA_ERR_INVALID_ARG
    bad = _problem(WORKLOADS["1"], d=32)
    assert L.vsa_sparse_attn_fwd(bad.ref, fake, fake, fake, fake, fake, 0.75, 0.0, fake, None,
                                 None) == vsa.VSA_ERR_UNSUPPORTED


def test_status_strings():
    for st in (0, -1, -2, -3, -4, 5):
        assert isinstance(vsa.status_string(st), str)
    assert vsa.status_string(-2).startswith("unsupported")


def test_pooled_bytes():
    w = WORKLOADS["4a"]
    p = _problem(w)
    sz = vsa.vsa_query_sizes(p, 0.9)
    assert vsa.vsa_pooled_bytes(p, 1, 32) == sz.pooled_rows * 96 * 8
    assert vsa.vsa_pooled_bytes(p, 0, 128) == sz.pooled_rows * 128 * 8
    # tripool_mode maxmin and avg keep two and one statistics
    assert vsa.vsa_pooled_bytes(p, vsa.VSA_SCORE_TRIPPOOL_MAXMIN, 32) == sz.pooled_rows * 64 * 8
    assert vsa.vsa_pooled_bytes(p, vsa.VSA_SCORE_TRIPPOOL_AVG, 16) == sz.pooled_rows * 16 * 8
    for mode in (1, 2, 3):
        for bad in (4, 12, 128):
            with pytest.raises(vsa.VSAError) as e:
                vsa.vsa_pooled_bytes(p, mode, bad)
            assert e.value.status == vsa.VSA_ERR_UNSUPPORTED
    with pytest.raises(vsa.VSAError) as e:
        vsa.vsa_pooled_bytes(p, 4, 32)
    assert e.value.status == vsa.VSA_ERR_INVALID_ARG
    rb = vsa.ref_budget(1, 8)
    assert (vsa.vsa_ref_pooled_bytes(p, vsa.VSA_SCORE_TRIPPOOL_MAXMIN, 32, rb)
            == 2 * vsa.vsa_ref_pooled_bytes(p, vsa.VSA_SCORE_TRIPPOOL_AVG, 32, rb))


def test_score_mode_names():
    assert vsa.score_mode("mean_gate") == vsa.VSA_SCORE_MEAN_GATE
    assert vsa.score_mode("trippool") == vsa.VSA_SCORE_TRIPPOOL
    assert vsa.score_mode("trippool", "maxmin") == vsa.VSA_SCORE_TRIPPOOL_MAXMIN
    assert vsa.score_mode("trippool", "avg") == vsa.VSA_SCORE_TRIPPOOL_AVG
    for bad in (("trippool", "minmax"), ("gate", "triplet")):
        with pytest.raises(ValueError):
            vsa.score_mode(*bad)


# ------------------------------------------------------------ two-stream budget

def test_ref_budget_struct_layout(tmp_path):
    src = tmp_path / "ref.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "vsa.h"\n'
                   'int main(void){printf("%zu %zu\\n", sizeof(vsa_ref_budget),'
                   ' offsetof(vsa_ref_budget, k_ref)); return 0;}\n')
    exe = tmp_path / "ref"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [ctypes.sizeof(vsa.vsa_ref_budget), vsa.vsa_ref_budget.k_ref.offset]


def test_ref_sizes_follow_the_segment_tiles():
    w = WORKLOADS["3b"]
    p = _problem(w)
    n, se, ie = vsa.vsa_ref_sizes(p, vsa.ref_budget(1, 32))
    assert n == oracle.segment_tiles(w.prefix, 1).size == 63
    sz = vsa.vsa_query_sizes(p, w.sparsity)
    assert se == w.B * w.H * sz.max_video_tiles * 63
    assert ie == w.B * w.H * sz.max_video_tiles * 32
    rb = vsa.vsa_ref_pooled_bytes(p, vsa.VSA_SCORE_MEAN_GATE, w.d, vsa.ref_budget(1, 32))
    assert rb == w.B * w.H * 63 * w.d * 8


@pytest.mark.parametrize("segment,k_ref", [(-1, 1), (3, 1), (1, 0), (1, 64), (2, 3)])
def test_bad_ref_budgets_rejected(segment, k_ref):
    # 3b: segments of 8, 63 and 2 tiles
    p = _problem(WORKLOADS["3b"])
    with pytest.raises(vsa.VSAError) as e:
        vsa.vsa_ref_sizes(p, vsa.ref_budget(segment, k_ref))
    assert e.value.status == vsa.VSA_ERR_INVALID_ARG


def test_long_reference_segment_rejected():
    """A reference segment longer than a select row (VSA_MAX_VIDEO_TILES tiles)
    is refused before any launch."""
    w = WORKLOADS["1"]
    p = _problem(w, prefix=(40, 64 * (vsa.VSA_MAX_VIDEO_TILES + 1), 24))
    with pytest.raises(vsa.VSAError) as e:
        vsa.vsa_ref_sizes(p, vsa.ref_budget(1, 32))
    assert e.value.status == vsa.VSA_ERR_SIZE
    p = _problem(w, prefix=(40, 64 * vsa.VSA_MAX_VIDEO_TILES, 24))
    n, _, _ = vsa.vsa_ref_sizes(p, vsa.ref_budget(1, 32))
    assert n == vsa.VSA_MAX_VIDEO_TILES


def test_zero_length_reference_segment_rejected():
    w = WORKLOADS["1"]
    p = _problem(w, prefix=(40, 0, 24))
    with pytest.raises(vsa.VSAError):
        vsa.vsa_ref_sizes(p, vsa.ref_budget(1, 1))


def test_ref_kept_stats_and_flops_match_oracle():
    prefix = (40, 150, 24)
    w = WORKLOADS["1"]
    p = _problem(w, prefix=prefix)
    budget = vsa.ref_budget(1, 2)
    tm = oracle.tile_map(*w.grid, prefix, w.tile_shapes[0])
    ref = oracle.segment_tiles(prefix, 1)
    rng = np.random.default_rng(1)
    sz = vsa.vsa_query_sizes(p, 0.5)
    kv = np.full((w.B * w.H, sz.max_video_tiles, sz.k_max), -1, dtype=np.int32)
    rf = np.zeros((w.B * w.H, sz.max_video_tiles, 2), dtype=np.int32)
    allows = []
    for h in range(w.H):
        sel = np.sort(np.stack([rng.choice(tm.n_video_tiles, sz.k[0], replace=False)
                                for _ in range(tm.n_video_tiles)]), axis=1)
        rsel = np.sort(np.stack([rng.choice(ref.size, 2, replace=False)
                                 for _ in range(tm.n_video_tiles)]), axis=1)
        kv[h, :, :sz.k[0]] = sel
        rf[h] = rsel
        allows.append(oracle.allowed_two_stream(tm, sel, ref, rsel))
    s2t = tm.slot_to_token.astype(np.int32)
    got = vsa.vsa_count_flops_ref(p, 0.5, budget, s2t, kv, rf)
    want = sum(oracle.effective_flops(tm, a, w.d) for a in allows)
    assert got == want
    kept, frac = vsa.vsa_kept_stats_ref(p, 0.5, budget)
    assert kept == sum(int(a.sum()) for a in allows)
    assert math.isclose(frac, kept / (w.H * tm.n_tiles ** 2), rel_tol=1e-12)


# ------------------------------------------------------------ fp8 variant

def test_fp8_entry_points_reject_before_any_launch():
    """Argument errors come back from the host checks (no device pointer is
    dereferenced: the pointers below are never valid device memory)."""
    L = vsa.lib()
    fake = ctypes.c_void_p(1 << 20)                     # 16-byte aligned, never read
    w = WORKLOADS["1"]                                  # f32 problem
    p32 = _problem(w)
    assert L.vsa_quantize_fp8(p32.ref, fake, fake, fake, fake, fake, fake, fake,
                              None) == vsa.VSA_ERR_UNSUPPORTED
    assert L.vsa_sparse_attn_fwd_fp8(p32.ref, fake, fake, fake, fake, fake, fake,
                                     ctypes.c_double(0.5), None, None, ctypes.c_float(0.0),
                                     fake, None, None) == vsa.VSA_ERR_UNSUPPORTED
    pb = _problem(w, dtype="bf16")
    # missing buffers
    assert L.vsa_quantize_fp8(pb.ref, fake, fake, None, fake, fake, fake, fake,
                              None) == vsa.VSA_ERR_INVALID_ARG
    # scales not 4-byte aligned
    assert L.vsa_quantize_fp8(pb.ref, fake, fake, fake, fake, fake, fake,
                              ctypes.c_void_p((1 << 20) + 2), None) == vsa.VSA_ERR_INVALID_ARG
    # sparse path without kv_idx; budget without ref_idx; budget on the dense path
    assert L.vsa_sparse_attn_fwd_fp8(pb.ref, fake, fake, fake, fake, fake, None,
                                     ctypes.c_double(0.5), None, None, ctypes.c_float(0.0),
                                     fake, None, None) == vsa.VSA_ERR_INVALID_ARG
    rb = vsa.ref_budget(1, 1)
    assert L.vsa_sparse_attn_fwd_fp8(pb.ref, fake, fake, fake, fake, fake, fake,
                                     ctypes.c_double(0.5), ctypes.byref(rb), None,
                                     ctypes.c_float(0.0), fake, None,
                                     None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_sparse_attn_fwd_fp8(pb.ref, fake, fake, fake, fake, fake, fake,
                                     ctypes.c_double(0.0), ctypes.byref(rb), fake,
                                     ctypes.c_float(0.0), fake, None,
                                     None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_sparse_attn_fwd_fp8(pb.ref, fake, fake, fake, fake, fake, fake,
                                     ctypes.c_double(0.5), None, None,
                                     ctypes.c_float(float("nan")), fake, None,
                                     None) == vsa.VSA_ERR_INVALID_ARG


def test_fp8_scale_bytes():
    w = WORKLOADS["3a"]
    p = _problem(w)
    sz = vsa.vsa_query_sizes(p, w.sparsity)
    assert vsa.fp8_scale_bytes(p) == w.B * w.H * sz.max_tiles * 4


def test_fused_map_fp8_rejects_before_any_launch():
    L = vsa.lib()
    fake = ctypes.c_void_p(1 << 20)
    w = WORKLOADS["1"]
    assert L.vsa_map_tiles_fp8(_problem(w).ref, *([fake] * 11), None) == vsa.VSA_ERR_UNSUPPORTED
    pb = _problem(w, dtype="bf16")
    args = [fake] * 11
    for i in range(11):                        # every buffer is required
        a = list(args)
        a[i] = None
        assert L.vsa_map_tiles_fp8(pb.ref, *a, None) == vsa.VSA_ERR_INVALID_ARG
    a = list(args)
    a[10] = ctypes.c_void_p((1 << 20) + 2)      # scales not 4-byte aligned
    assert L.vsa_map_tiles_fp8(pb.ref, *a, None) == vsa.VSA_ERR_INVALID_ARG
    a = list(args)
    a[7] = ctypes.c_void_p((1 << 20) + 8)       # q8 not 16-byte aligned
    assert L.vsa_map_tiles_fp8(pb.ref, *a, None) == vsa.VSA_ERR_INVALID_ARG


# ------------------------------------------------------- measurement aids

def test_mfma_probe_rejects_before_any_launch():
    L = vsa.lib()
    assert L.vsa_mfma_probe(5, 1, 1, None, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_mfma_probe(-1, 1, 1, None, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_mfma_probe(0, 0, 1, None, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_mfma_probe(1, 1, 0, None, None) == vsa.VSA_ERR_INVALID_ARG
    assert L.vsa_mfma_probe(0, (1 << 22) + 1, 1, None, None) == vsa.VSA_ERR_SIZE
    assert L.vsa_mfma_probe(0, 1, (1 << 16) + 1, None, None) == vsa.VSA_ERR_SIZE
    assert L.vsa_mfma_probe(0, 1, 1, ctypes.c_void_p((1 << 20) + 4),
                            None) == vsa.VSA_ERR_INVALID_ARG


def test_mfma_probe_flop_count():
    # one 32x32xK product is 2*32*32*K flops; a workgroup has 4 waves of 4 chains
    # (kinds 2-4: 8 waves, of which kind 4 runs the products in 4)
    assert vsa.MFMA_PROBE_FLOPS == (2 * 32 * 32 * 16,) + (2 * 32 * 32 * 64,) * 4
    assert vsa.MFMA_PROBE_PER_TRIP == (16, 16, 32, 32, 16)


# ------------------------------------------------- random geometries (planner)

from hypothesis import given, settings, strategies as st   # noqa: E402

_SHAPES = [(1 << a, 1 << b, 1 << (6 - a - b)) for a in range(7) for b in range(7 - a)]


@settings(max_examples=150, deadline=None)
@given(T=st.integers(1, 12), Hv=st.integers(1, 20), Wv=st.integers(1, 20),
       prefix=st.lists(st.integers(0, 300), max_size=4),
       shapes=st.lists(st.sampled_from(_SHAPES), min_size=1, max_size=4),
       H=st.integers(1, 6), sparsity=st.floats(0.0, 0.999))
def test_planner_matches_oracle_on_random_geometries(T, Hv, Wv, prefix, shapes, H, sparsity):
    """Tile counts, k per shape and the kept pair count of the host planner
    equal what the oracle's tile map and keep rule give, for any grid, any
    prefix (empty segments included) and any mix of tile shapes."""
    p = vsa.Problem(1, H, 64, (T, Hv, Wv), prefix, shapes, "bf16")
    sz = vsa.vsa_query_sizes(p, sparsity)
    tms = [oracle.tile_map(T, Hv, Wv, prefix, s) for s in shapes]
    assert sz.n_prefix_tiles == tms[0].n_prefix_tiles == sum(-(-L // 64) for L in prefix)
    for i, tm in enumerate(tms):
        assert (sz.n_tiles[i], sz.n_video_tiles[i]) == (tm.n_tiles, tm.n_video_tiles)
        assert sz.k[i] == (tm.n_video_tiles if sparsity == 0.0
                           else oracle.keep_count(sparsity, tm.n_video_tiles))
    kept, _ = vsa.vsa_kept_stats(p, sparsity)
    want = 0
    for h in range(H):
        tm = tms[h % len(shapes)]
        k = sz.k[h % len(shapes)]
        want += tm.n_prefix_tiles * tm.n_tiles + tm.n_video_tiles * (tm.n_prefix_tiles + k)
    assert kept == want


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 6), Hv=st.integers(1, 12), Wv=st.integers(1, 12),
       prefix=st.lists(st.integers(0, 200), max_size=3),
       shapes=st.lists(st.sampled_from(_SHAPES), min_size=1, max_size=3),
       H=st.integers(1, 4), sparsity=st.floats(0.05, 0.95), seed=st.integers(0, 2**31 - 1))
def test_count_flops_matches_oracle_on_random_geometries(T, Hv, Wv, prefix, shapes, H, sparsity,
                                                         seed):
    """Effective FLOPs from the host counter equal the oracle's count of real
    (query, allowed key) pairs for random selections, padded tiles included."""
    p = vsa.Problem(1, H, 64, (T, Hv, Wv), prefix, shapes, "bf16")
    sz = vsa.vsa_query_sizes(p, sparsity)
    tms = [oracle.tile_map(T, Hv, Wv, prefix, s) for s in shapes]
    s2t = np.full((len(shapes), sz.max_tiles * 64), -1, dtype=np.int32)
    for i, tm in enumerate(tms):
        s2t[i, : tm.n_tiles * 64] = tm.slot_to_token
    rng = np.random.default_rng(seed)
    kv = np.full((H, sz.max_video_tiles, sz.k_max), -1, dtype=np.int32)
    want = 0
    for h in range(H):
        i = h % len(shapes)
        tm, k = tms[i], sz.k[i]
        sel = np.sort(np.stack([rng.choice(tm.n_video_tiles, k, replace=False)
                                for _ in range(tm.n_video_tiles)]), axis=1)
        kv[h, : tm.n_video_tiles, :k] = sel
        want += oracle.effective_flops(tm, oracle.allowed_tiles(tm, sel), 64)
    assert vsa.vsa_count_flops(p, sparsity, s2t, kv) == want


def test_fused_select_rejects_before_launch():
    """vsa_tile_select: argument errors and the sizes it does not take come
    back before any launch (fake pointers, never dereferenced)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check; skipped where a GPU is visible")
    L = vsa.lib()
    fake = ctypes.c_void_p(0x10000)
    p = _problem(WORKLOADS["1"])
    call = lambda prob, mode, proj, sp, **kw: L.vsa_tile_select(
        prob.ref, mode, proj, kw.get("qt", fake), fake, fake, fake, kw.get("wk", fake), sp,
        fake, kw.get("kv", fake), None)
    assert call(p, 0, p.d, 0.0) == vsa.VSA_ERR_INVALID_ARG          # dense: nothing to select
    assert call(p, 0, p.d, 0.75, kv=None) == vsa.VSA_ERR_INVALID_ARG
    assert call(p, 0, p.d, 0.75, qt=None) == vsa.VSA_ERR_INVALID_ARG
    assert call(p, 1, 32, 0.75, wk=None) == vsa.VSA_ERR_INVALID_ARG
    # descriptor width 24 (TripPool, proj 8) is not a multiple of 32
    assert call(p, 1, 8, 0.75) == vsa.VSA_ERR_UNSUPPORTED
    # 48 = TripPool with proj 16; maxmin with proj 16 is 32 wide and taken
    assert call(p, vsa.VSA_SCORE_TRIPPOOL, 16, 0.75) == vsa.VSA_ERR_UNSUPPORTED
    big = vsa.Problem(1, 1, 128, (1, 1, 64 * (vsa.VSA_FUSED_MAX_TILES + 1)), (),
                      ((1, 1, 64),), "bf16")
    assert call(big, 0, 128, 0.75) == vsa.VSA_ERR_UNSUPPORTED


def test_fused_select_support_rule():
    """The binding's host-side rule matches the header's limits."""
    w5, w1 = WORKLOADS["5"], WORKLOADS["1"]
    assert vsa.fused_select_supported(_problem(w5), vsa.VSA_SCORE_TRIPPOOL, 32, 0.95)
    assert not vsa.fused_select_supported(_problem(w5), vsa.VSA_SCORE_TRIPPOOL, 32, 0.0)
    assert not vsa.fused_select_supported(_problem(w1), vsa.VSA_SCORE_TRIPPOOL, 8, 0.75)
    assert vsa.fused_select_supported(_problem(w1), vsa.VSA_SCORE_TRIPPOOL_MAXMIN, 16, 0.75)
    assert vsa.fused_select_supported(_problem(w1, d=64), vsa.VSA_SCORE_MEAN_GATE, 64, 0.5)
    n = vsa.VSA_FUSED_MAX_TILES
    ok = vsa.Problem(1, 1, 128, (1, 1, 64 * n), (), ((1, 1, 64),), "bf16")
    too = vsa.Problem(1, 1, 128, (1, 1, 64 * (n + 1)), (), ((1, 1, 64),), "bf16")
    assert vsa.fused_select_supported(ok, vsa.VSA_SCORE_MEAN_GATE, 128, 0.9)
    assert not vsa.fused_select_supported(too, vsa.VSA_SCORE_MEAN_GATE, 128, 0.9)


def test_map_tiles_scores_rejects_before_launch():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check; skipped where a GPU is visible")
    L = vsa.lib()
    fake, odd = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10008)
    p = _problem(WORKLOADS["1"])
    f = lambda mode=0, proj=p.d, **kw: L.vsa_map_tiles_scores(
        p.ref, mode, proj, kw.get("q", fake), kw.get("k", fake), kw.get("v", fake),
        kw.get("s2t", fake), kw.get("qt", fake), kw.get("kt", fake), kw.get("vt", fake),
        kw.get("wq", fake), kw.get("wk", None), kw.get("ws", fake), kw.get("sc", fake), None)
    odd4 = ctypes.c_void_p(0x10004)         # workspace of doubles: 8-byte alignment
    for kw in (dict(q=None), dict(k=None), dict(s2t=None), dict(qt=None), dict(wq=None),
               dict(ws=None), dict(sc=None), dict(vt=None), dict(q=odd), dict(ws=odd4)):
        assert f(**kw) == vsa.VSA_ERR_INVALID_ARG, kw
    assert f(mode=1, proj=32) == vsa.VSA_ERR_INVALID_ARG          # TripPool needs wk
    assert f(mode=1, proj=24, wk=fake) == vsa.VSA_ERR_UNSUPPORTED  # not a power of two
    assert f(mode=0, proj=32) == vsa.VSA_ERR_INVALID_ARG          # mean gate: proj_dim = d
    bad = _problem(WORKLOADS["1"], d=96)
    assert L.vsa_map_tiles_scores(bad.ref, 0, 96, fake, fake, fake, fake, fake, fake, fake, fake,
                                  None, fake, fake, None) == vsa.VSA_ERR_UNSUPPORTED
