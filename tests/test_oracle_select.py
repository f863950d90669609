"""Pins for the oracle's top-k selection and keep count (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def rank_select(row, k):
    """Rank definition written out: keep j iff rank(j) < k (O(n^2))."""
    n = len(row)
    kept = []
    for j in range(n):
        rank = sum(1 for jj in range(n) if row[jj] > row[j]) \
            + sum(1 for jj in range(j) if row[jj] == row[j])
        if rank < k:
            kept.append(j)
    return kept


@pytest.mark.parametrize("n,k,levels", [(4, 1, 0), (17, 5, 3), (33, 33, 0),
                                        (40, 1, 4), (64, 16, 6), (50, 49, 2)])
def test_select_matches_rank_definition(n, k, levels):
    rng = np.random.default_rng(n * 100 + k)
    s = rng.standard_normal((12, n)).astype(np.float32)
    if levels:                               # many exact ties
        s = np.round(s * levels).astype(np.float32) / levels
    got = oracle.select_topk(s, k)
    assert got.shape == (12, k)
    for i in range(12):
        assert list(got[i]) == rank_select(list(s[i]), k)


def test_ties_go_to_lower_index_and_signed_zero_ties():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    assert list(oracle.select_topk(s, 2)[0]) == [1, 2]
    s = np.array([[0.0, -0.0, -1.0, -0.0]], dtype=np.float32)
    assert list(oracle.select_topk(s, 2)[0]) == [0, 1]
    s = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    assert list(oracle.select_topk(s, 1)[0]) == [0]


def test_k_equals_n_and_k_one():
    s = np.random.default_rng(7).standard_normal((5, 9)).astype(np.float32)
    np.testing.assert_array_equal(oracle.select_topk(s, 9), np.tile(np.arange(9), (5, 1)))
    np.testing.assert_array_equal(oracle.select_topk(s, 1)[:, 0], s.argmax(axis=1))


def test_output_rows_ascending():
    s = np.random.default_rng(8).standard_normal((30, 100)).astype(np.float32)
    got = oracle.select_topk(s, 25)
    assert (np.diff(got, axis=1) > 0).all()


@pytest.mark.parametrize("sparsity,n,k", [
    (0.75, 4, 1), (0.75, 504, 126), (0.75, 1764, 441), (0.90, 504, 51),
    (0.90, 528, 53), (0.90, 1008, 101), (0.95, 3780, 189), (0.95, 3960, 198),
    (0.95, 4032, 202), (0.0, 77, 77), (0.9999, 4, 1), (0.5, 3, 2),
])
def test_keep_count_integer_rounding(sparsity, n, k):
    assert oracle.keep_count(sparsity, n) == k


def test_keep_count_exact_where_float_ceil_is_not():
    # (1 - 0.95) * 3780 is 189.00000000000017 in IEEE double: a float ceil
    # would keep 190 tiles. 5% of 3780 is exactly 189.
    assert np.ceil((1 - 0.95) * 3780) == 190
    assert oracle.keep_count(0.95, 3780) == 189


def test_pages_keep_percent_example():
    f = json.load(open(GOLDEN))["keep_percent_example"]
    assert abs((1 - f["sparsity"]) * 100 - f["keep_percent"]) < 1e-9
    assert oracle.keep_count(f["sparsity"], 2000) == 100
    r = json.load(open(GOLDEN))["ref2va_sparsity"]
    assert oracle.keep_count(r["value"], 1764) == int(r["kept_fraction_of_video_tiles"] * 1764)
