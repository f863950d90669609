"""Pins for the oracle's tile map and gather (CPU only).

The oracle builds the map slot -> token (the inverse direction). These tests
rebuild it token -> slot with explicit Python loops, so a swapped axis, a
wrong stride or a misplaced prefix offset fails here.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")

GEOMS = [
    # (T, Hv, Wv), prefix, shape
    ((4, 8, 8), (40, 64, 24), (4, 4, 4)),
    ((5, 6, 10), (1, 0, 130), (4, 4, 4)),
    ((8, 12, 20), (512, 64, 128), (1, 8, 8)),
    ((8, 6, 4), (), (16, 2, 2)),
    ((3, 9, 7), (65,), (2, 4, 8)),
    ((2, 5, 33), (7, 7), (8, 4, 2)),
]


def brute_force_map(T, Hv, Wv, prefix, shape):
    """token -> (tile, slot) by explicit loops, returned as slot -> token."""
    pt, ph, pw = shape
    n_pre = sum((L + 63) // 64 for L in prefix)
    nt, nh, nw = (T + pt - 1) // pt, (Hv + ph - 1) // ph, (Wv + pw - 1) // pw
    n_tiles = n_pre + nt * nh * nw
    s2t = [-1] * (n_tiles * 64)
    tile0, tok = 0, 0
    for L in prefix:
        for j in range(L):
            s2t[(tile0 + j // 64) * 64 + j % 64] = tok + j
        tile0 += (L + 63) // 64
        tok += L
    for t in range(T):
        for y in range(Hv):
            for x in range(Wv):
                tile = n_pre + ((t // pt) * nh + y // ph) * nw + x // pw
                slot = ((t % pt) * ph + y % ph) * pw + x % pw
                s2t[tile * 64 + slot] = tok + (t * Hv + y) * Wv + x
    return np.array(s2t), n_pre, nt * nh * nw


@pytest.mark.parametrize("grid,prefix,shape", GEOMS)
def test_map_matches_token_to_slot_enumeration(grid, prefix, shape):
    tm = oracle.tile_map(*grid, prefix, shape)
    want, n_pre, n_vid = brute_force_map(*grid, prefix, shape)
    assert tm.n_prefix_tiles == n_pre and tm.n_video_tiles == n_vid
    np.testing.assert_array_equal(tm.slot_to_token, want)


@pytest.mark.parametrize("grid,prefix,shape", GEOMS)
def test_map_is_bijection_and_pad_count(grid, prefix, shape):
    T, Hv, Wv = grid
    tm = oracle.tile_map(*grid, prefix, shape)
    N = sum(prefix) + T * Hv * Wv
    real = tm.slot_to_token[tm.slot_to_token >= 0]
    np.testing.assert_array_equal(np.sort(real), np.arange(N))
    pads = sum(64 * ((L + 63) // 64) - L for L in prefix) \
        + 64 * tm.n_video_tiles - T * Hv * Wv
    assert int((tm.slot_to_token < 0).sum()) == pads


@pytest.mark.parametrize("grid,prefix,shape", GEOMS)
def test_prefix_tiles_are_segment_pure(grid, prefix, shape):
    tm = oracle.tile_map(*grid, prefix, shape)
    bounds = np.cumsum((0,) + tuple(prefix))
    seg_of_tile = []
    for t in range(tm.n_prefix_tiles):
        toks = tm.tile_tokens(t)
        segs = set(np.searchsorted(bounds, toks, side="right") - 1)
        assert len(segs) == 1, "a prefix tile mixes segments"
        seg_of_tile.append(segs.pop())
    # no video token lands in a prefix tile and vice versa
    P = sum(prefix)
    for t in range(tm.n_prefix_tiles, tm.n_tiles):
        assert (tm.tile_tokens(t) >= P).all()


def test_video_tile_is_a_3d_box():
    tm = oracle.tile_map(8, 8, 8, (), (4, 4, 4))
    toks = tm.tile_tokens(0)
    t, y, x = toks // 64, (toks // 8) % 8, toks % 8
    assert set(t) == {0, 1, 2, 3} and set(y) == {0, 1, 2, 3} and set(x) == {0, 1, 2, 3}
    toks = tm.tile_tokens(1)      # next along w
    assert set(toks % 8) == {4, 5, 6, 7} and set((toks // 8) % 8) == {0, 1, 2, 3}


def test_pages_tile_facts():
    facts = json.load(open(GOLDEN))
    assert np.prod(facts["tile_tokens"]["vsa_shape"]) == facts["tile_tokens"]["value"] == oracle.TILE
    shapes = [tuple(int(v) for v in s.split(","))
              for s in facts["custom_tiling_default"]["value"].split(";")]
    for sh in shapes:
        assert np.prod(sh) == 64
        tm = oracle.tile_map(8, 12, 20, (40,), sh)
        want, _, _ = brute_force_map(8, 12, 20, (40,), sh)
        np.testing.assert_array_equal(tm.slot_to_token, want)


def test_gather_rows_and_zero_pads():
    rng = np.random.default_rng(0)
    tm = oracle.tile_map(4, 6, 6, (10, 70), (4, 4, 4))
    N = 80 + 144
    x = rng.standard_normal((N, 8))
    g = oracle.gather(x, tm)
    assert g.shape == (tm.n_tiles, 64, 8)
    for tile in range(tm.n_tiles):
        for slot in range(64):
            tok = tm.slot_to_token[tile * 64 + slot]
            if tok < 0:
                assert (g[tile, slot] == 0).all()
            else:
                assert (g[tile, slot] == x[tok]).all()


def test_zero_length_segment_has_no_tile():
    a = oracle.tile_map(4, 4, 4, (40, 0, 24), (4, 4, 4))
    b = oracle.tile_map(4, 4, 4, (40, 24), (4, 4, 4))
    assert a.n_prefix_tiles == 2
    np.testing.assert_array_equal(a.slot_to_token, b.slot_to_token)
