"""Pins for the oracle's tile pooling and scoring (CPU only)."""
import numpy as np
import pytest

import oracle


def _tiles(grid, prefix, shape, d, seed=0):
    rng = np.random.default_rng(seed)
    tm = oracle.tile_map(*grid, prefix, shape)
    N = sum(prefix) + int(np.prod(grid))
    x = rng.standard_normal((N, d))
    return tm, x, oracle.gather(x, tm)


def test_mean_gate_constant_tile_closed_form():
    d = 6
    tm = oracle.tile_map(8, 4, 4, (5,), (16, 2, 2))   # video tiles half padded
    N = 5 + 128
    x = np.zeros((N, d))
    c = np.array([1.5, -2.0, 0.25, 3.0, -0.5, 1.0])
    x[5:] = c                                         # every video token = c
    gate = np.arange(d * d, dtype=np.float64).reshape(d, d) / 7.0 - 2.0
    got = oracle.pool_mean_gate(oracle.gather(x, tm), tm, gate)
    want = [sum(c[i] * gate[i][j] for i in range(d)) for j in range(d)]
    assert got.shape == (tm.n_video_tiles, d)
    for row in got:                                   # pads must not dilute the mean
        np.testing.assert_allclose(row, want, rtol=1e-14, atol=1e-14)


def test_mean_gate_is_mean_of_projected_tokens():
    tm, x, xt = _tiles((5, 6, 10), (3,), (4, 4, 4), 16)
    gate = np.random.default_rng(1).standard_normal((16, 16))
    got = oracle.pool_mean_gate(xt, tm, gate)
    for i in range(tm.n_video_tiles):
        toks = tm.tile_tokens(tm.n_prefix_tiles + i)
        proj = [x[t] @ gate for t in toks]            # project first, then average
        np.testing.assert_allclose(got[i], np.mean(proj, axis=0), rtol=1e-12, atol=1e-12)


def test_trippool_order_and_values_by_hand():
    # one video tile, three real tokens; projection = first two channels
    tm = oracle.tile_map(1, 1, 3, (), (4, 4, 4))
    x = np.array([[1.0, -4.0, 9.0], [2.0, 5.0, 9.0], [6.0, 0.5, 9.0]])
    proj = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    got = oracle.pool_trippool(oracle.gather(x, tm), tm, proj)
    # [avg(c0), avg(c1), max(c0), max(c1), min(c0), min(c1)]
    np.testing.assert_allclose(got[0], [3.0, 0.5, 6.0, 5.0, 1.0, -4.0], rtol=0, atol=1e-15)


def test_tripool_modes_by_hand():
    # tripool_mode maxmin keeps [Max | Min], avg keeps [Avg]; same tile as above
    tm = oracle.tile_map(1, 1, 3, (), (4, 4, 4))
    x = np.array([[1.0, -4.0, 9.0], [2.0, 5.0, 9.0], [6.0, 0.5, 9.0]])
    proj = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    xt = oracle.gather(x, tm)
    mm = oracle.pool_trippool(xt, tm, proj, stats="maxmin")
    av = oracle.pool_trippool(xt, tm, proj, stats="avg")
    np.testing.assert_allclose(mm[0], [6.0, 5.0, 1.0, -4.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(av[0], [3.0, 0.5], rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.pool_trippool(xt, tm, proj, stats="minmax")


def test_tripool_avg_is_the_projected_mean_gate():
    # Avg of projected tokens = (mean of tokens) x projection: the mean-gate
    # descriptor with the projection as the gate (linearity of the mean);
    # ragged grid, so edge tiles hold pads
    tm, x, xt = _tiles((5, 6, 7), (40, 64, 24), (4, 4, 4), 16)
    assert not tm.valid()[tm.n_prefix_tiles:].all()
    proj = np.random.default_rng(6).standard_normal((16, 16))
    np.testing.assert_allclose(oracle.pool_trippool(xt, tm, proj, stats="avg"),
                               oracle.pool_mean_gate(xt, tm, proj), rtol=1e-12, atol=1e-12)


def test_tripool_maxmin_constant_tiles_score_is_twice_mean_gate_score():
    d, r = 8, 5
    tm = oracle.tile_map(8, 8, 8, (), (4, 4, 4))
    rng = np.random.default_rng(7)
    consts = rng.standard_normal((tm.n_video_tiles, d))
    x = np.zeros((512, d))
    for i in range(tm.n_video_tiles):
        x[tm.tile_tokens(i)] = consts[i]
    xt = oracle.gather(x, tm)
    pq, pk = rng.standard_normal((d, r)), rng.standard_normal((d, r))
    mm = oracle.tile_scores(oracle.pool_trippool(xt, tm, pq, stats="maxmin"),
                            oracle.pool_trippool(xt, tm, pk, stats="maxmin"))
    mean = oracle.tile_scores(oracle.pool_mean_gate(xt, tm, pq),
                              oracle.pool_mean_gate(xt, tm, pk))
    np.testing.assert_allclose(mm, 2.0 * mean, rtol=2e-7)


def test_trippool_max_ge_avg_ge_min_and_pads_excluded():
    tm, x, xt = _tiles((8, 6, 4), (2,), (16, 2, 2), 8)
    x = x + 10.0                                      # all projected values far from 0
    xt = oracle.gather(x, tm)
    proj = np.random.default_rng(2).standard_normal((8, 4))
    got = oracle.pool_trippool(xt, tm, proj)
    r = 4
    avg, mx, mn = got[:, :r], got[:, r:2 * r], got[:, 2 * r:]
    assert (mx >= avg - 1e-12).all() and (avg >= mn - 1e-12).all()
    for i in range(tm.n_video_tiles):
        y = x[tm.tile_tokens(tm.n_prefix_tiles + i)] @ proj
        np.testing.assert_allclose(mx[i], y.max(0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(mn[i], y.min(0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(avg[i], y.mean(0), rtol=1e-12, atol=1e-12)


def test_trippool_single_token_tile():
    tm = oracle.tile_map(1, 1, 1, (), (4, 4, 4))
    x = np.array([[0.5, -1.0, 2.0, 0.0]])
    proj = np.random.default_rng(3).standard_normal((4, 3))
    got = oracle.pool_trippool(oracle.gather(x, tm), tm, proj)[0]
    y = [sum(x[0, c] * proj[c, j] for c in range(4)) for j in range(3)]
    np.testing.assert_allclose(got, y * 3, rtol=1e-14, atol=1e-14)


def test_trippool_constant_tiles_score_is_three_times_mean_gate_score():
    d, r = 8, 5
    tm = oracle.tile_map(8, 8, 8, (), (4, 4, 4))
    rng = np.random.default_rng(4)
    consts = rng.standard_normal((tm.n_video_tiles, d))
    x = np.zeros((512, d))
    for i in range(tm.n_video_tiles):
        x[tm.tile_tokens(i)] = consts[i]
    xt = oracle.gather(x, tm)
    pq, pk = rng.standard_normal((d, r)), rng.standard_normal((d, r))
    trip = oracle.tile_scores(oracle.pool_trippool(xt, tm, pq),
                              oracle.pool_trippool(xt, tm, pk))
    mean = oracle.tile_scores(oracle.pool_mean_gate(xt, tm, pq),
                              oracle.pool_mean_gate(xt, tm, pk))
    np.testing.assert_allclose(trip, 3.0 * mean, rtol=2e-7)


def test_scores_direct_formula_and_orientation():
    qhat = np.array([[1.0, 0.0], [0.5, 2.0], [0.0, -1.0]])
    khat = np.array([[0.0, 1.0], [1.0, 0.0]])
    s = oracle.tile_scores(qhat, khat)
    assert s.dtype == np.float32 and s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            assert s[i, j] == np.float32(sum(qhat[i, c] * khat[j, c] for c in range(2)))
    assert s[0, 0] == 0.0 and s[0, 1] == 1.0        # query rows, key columns


def test_scores_symmetric_when_q_equals_k():
    tm, x, xt = _tiles((4, 8, 8), (40, 64, 24), (4, 4, 4), 16)
    gate = np.random.default_rng(5).standard_normal((16, 16))
    h = oracle.pool_mean_gate(xt, tm, gate)
    s = oracle.tile_scores(h, h)
    np.testing.assert_array_equal(s, s.T)


def test_scores_rounded_once_to_f32():
    qhat = np.array([[1.0 + 2.0 ** -30]])
    khat = np.array([[1.0]])
    assert oracle.tile_scores(qhat, khat)[0, 0] == np.float32(1.0)
