"""Pins for the oracle's masked tile attention (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _problem(grid=(4, 8, 8), prefix=(40, 64, 24), shape=(4, 4, 4), d=16,
             sparsity=0.75, seed=0):
    rng = np.random.default_rng(seed)
    N = sum(prefix) + int(np.prod(grid))
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    gate = rng.standard_normal((d, d)) / math.sqrt(d)
    r = oracle.head_forward(q, k, v, grid, prefix, shape, sparsity, "mean_gate", gate)
    return q, k, v, r


def token_mask(tm, allow):
    """bool [N, N]: token i may attend to token j (expanded from tiles)."""
    tile_of = np.empty(tm.slot_to_token.max() + 1, dtype=np.int64)
    real = tm.slot_to_token >= 0
    tile_of[tm.slot_to_token[real]] = np.nonzero(real)[0] // 64
    return allow[tile_of[:, None], tile_of[None, :]]


def sdpa(q, k, v, mask, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(mask), scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("grid,prefix,shape,sparsity", [
    ((4, 8, 8), (40, 64, 24), (4, 4, 4), 0.75),
    ((5, 6, 10), (1, 130), (4, 4, 4), 0.6),
    ((8, 6, 4), (7,), (16, 2, 2), 0.5),
    ((3, 9, 7), (), (2, 4, 8), 0.9),
])
def test_sparse_matches_torch_masked_sdpa(grid, prefix, shape, sparsity):
    q, k, v, r = _problem(grid, prefix, shape, 16, sparsity)
    scale = 1 / math.sqrt(16)
    mask = token_mask(r["tmap"], r["allow"])
    np.testing.assert_allclose(r["out"], sdpa(q, k, v, mask, scale), rtol=0, atol=1e-12)
    lse = logsumexp(np.where(mask, (q @ k.T) * scale, -np.inf), axis=1)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


def test_full_keep_equals_dense():
    facts = json.load(open(GOLDEN))["full_keep_equals_dense"]
    q, k, v, r = _problem(sparsity=0.0)
    o, lse = oracle.dense_attention(q, k, v, 1 / 4)
    assert np.abs(r["out"] - o).max() <= facts["max_abs_error"]
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-13)
    N = q.shape[0]
    np.testing.assert_allclose(o, sdpa(q, k, v, np.ones((N, N), bool), 0.25), atol=1e-12)


@pytest.mark.parametrize("sparsity", [0.25, 0.75, 0.95])
def test_prefix_rows_are_dense_at_any_sparsity(sparsity):
    q, k, v, r = _problem(grid=(4, 8, 16), sparsity=sparsity)
    o, _ = oracle.dense_attention(q, k, v, 0.25)
    P = 128
    np.testing.assert_allclose(r["out"][:P], o[:P], rtol=0, atol=1e-13)
    assert r["allow"][:, :r["tmap"].n_prefix_tiles].all()


def test_constant_values_give_constant_output():
    q, k, v, _ = _problem()
    v[:] = np.arange(16) * 0.5 - 3.0
    r = _problem()[3]
    tm, allow = r["tmap"], r["allow"]
    out, _ = oracle.sparse_attention(q, k, v, tm, allow, 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(v[0], out.shape), rtol=0, atol=1e-13)


def test_zero_keys_average_values_over_allowed_set():
    q, k, v, r = _problem()
    tm, allow = r["tmap"], r["allow"]
    out, lse = oracle.sparse_attention(q, np.zeros_like(k), v, tm, allow, 0.25)
    for tq in range(tm.n_tiles):
        keys = [t for tk in range(tm.n_tiles) if allow[tq, tk] for t in tm.tile_tokens(tk)]
        want = np.mean(v[keys], axis=0)
        for row in tm.tile_tokens(tq):
            np.testing.assert_allclose(out[row], want, rtol=0, atol=1e-13)
            assert abs(lse[row] - math.log(len(keys))) < 1e-13


def test_video_query_sees_prefix_plus_selected_only():
    q, k, v, r = _problem()
    tm, allow, sel = r["tmap"], r["allow"], r["kv_video"]
    npf = tm.n_prefix_tiles
    for i in range(tm.n_video_tiles):
        want = set(range(npf)) | {npf + int(j) for j in sel[i]}
        assert set(np.nonzero(allow[npf + i])[0]) == want
    assert sel.shape == (tm.n_video_tiles, 1)


def test_effective_flops_counts_token_pairs():
    q, k, v, r = _problem(grid=(5, 6, 10), prefix=(1, 130), sparsity=0.6)
    mask = token_mask(r["tmap"], r["allow"])
    assert oracle.effective_flops(r["tmap"], r["allow"], 16) == 4 * 16 * int(mask.sum())


def test_sparse_attention_subset_leaves_other_rows_nan():
    q, k, v, r = _problem()
    tm, allow = r["tmap"], r["allow"]
    out, lse = oracle.sparse_attention(q, k, v, tm, allow, 0.25, query_tiles=[4])
    rows = tm.tile_tokens(4)
    assert not np.isnan(out[rows]).any()
    assert np.isnan(np.delete(out, rows, axis=0)).all()
    np.testing.assert_array_equal(out[rows], r["out"][rows])
