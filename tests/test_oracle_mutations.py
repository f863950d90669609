"""Planted mistakes in the oracle must trip its pins (CPU only).

Each case swaps one oracle step for a plausibly wrong variant (a transposed
axis, a dropped mask, a wrong tie rule, a missing scale ...) and checks that
at least one pin test fails on it. The oracle itself is untouched outside
the monkeypatched scope.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.vsa_oracle as vo
from tests import test_oracle_attention as ta
from tests import test_oracle_fp8 as tf8
from tests import test_oracle_map as tm_
from tests import test_oracle_pool_score as tp
from tests import test_oracle_select as ts
from tests import test_oracle_teacher as tte
from tests import test_oracle_two_stream as tts


def _map_swapped_xy(T, Hv, Wv, prefix, shape):
    return _orig_tile_map(T, Wv, Hv, prefix, shape)   # wrong axis order


def _map_prefix_shared(T, Hv, Wv, prefix, shape):
    # all prefix segments packed together (modalities share tiles)
    return _orig_tile_map(T, Hv, Wv, (sum(prefix),) if prefix else (), shape)


def _pool_mean_with_pads(xt, tmap, gate, tiles=None):
    x, v = vo._tiles_part(xt, tmap, tiles)
    return x.mean(axis=1) @ np.asarray(gate, dtype=np.float64)


def _trippool_wrong_order(xt, tmap, proj, tiles=None, stats="triplet"):
    r = np.asarray(proj).shape[1]
    p = _orig_trippool(xt, tmap, proj, tiles, stats)
    return np.concatenate([p[:, r:2 * r], p[:, :r], p[:, 2 * r:]], axis=1)


def _trippool_maxmin_swapped(xt, tmap, proj, tiles=None, stats="triplet"):
    p = _orig_trippool(xt, tmap, proj, tiles, stats)
    if stats != "maxmin":
        return p
    r = np.asarray(proj).shape[1]
    return np.concatenate([p[:, r:], p[:, :r]], axis=1)   # [Min | Max]


def _trippool_avg_with_pads(xt, tmap, proj, tiles=None, stats="triplet"):
    if stats != "avg":
        return _orig_trippool(xt, tmap, proj, tiles, stats)
    x, _ = vo._tiles_part(xt, tmap, tiles)
    return (x @ np.asarray(proj, dtype=np.float64)).mean(axis=1)   # pads counted


def _scores_transposed(qhat, khat):
    return _orig_scores(qhat, khat).T.copy()


def _select_high_index_ties(scores, k):
    s = np.asarray(scores, dtype=np.float32)
    out = np.empty((s.shape[0], k), dtype=np.int64)
    for i in range(s.shape[0]):
        order = np.lexsort((-np.arange(s.shape[1]), -s[i]))
        out[i] = np.sort(order[:k])
    return out


def _keep_count_float_ceil(sparsity, n):
    return max(1, int(math.ceil((1.0 - sparsity) * n)))


def _softmax_no_scale(q, k, v, scale):
    return _orig_softmax(q, k, v, 1.0)


def _allowed_no_prefix_rows(tmap, kv_video):
    a = _orig_allowed(tmap, kv_video)
    a[:tmap.n_prefix_tiles, tmap.n_prefix_tiles:] = False
    return a


def _two_stream_reference_dense(tmap, kv_video, ref_tiles, kv_ref):
    # the budget is ignored: every reference tile stays a dense key
    a = _orig_two_stream(tmap, kv_video, ref_tiles, kv_ref)
    a[tmap.n_prefix_tiles:, np.asarray(ref_tiles, dtype=np.int64)] = True
    return a


def _segment_tiles_shifted(prefix, segment):
    return _orig_segment_tiles(prefix, segment) + 1


def _teacher_max_logit(q, k, tmap, scale, query_tiles=None):
    # pools the raw logits instead of the attention probabilities
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    npf = tmap.n_prefix_tiles
    rows = range(tmap.n_video_tiles) if query_tiles is None else query_tiles
    out = np.zeros((len(rows), tmap.n_video_tiles))
    for r, i in enumerate(rows):
        qs = tmap.tile_tokens(npf + i)
        for j in range(tmap.n_video_tiles):
            out[r, j] = ((q[qs] @ k[tmap.tile_tokens(npf + j)].T) * scale).max()
    return out


def _recall_over_n(selection, teacher_rows, k):
    return _orig_recall(selection, teacher_rows, k) * k / np.asarray(teacher_rows).shape[1]


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -6.0)
    step = np.exp2(e - 3.0)
    return np.copysign(np.floor(ax / step + 0.5) * step, x)


def _scale_exponent_plus_one(amax):
    return _orig_scale_exp(amax) + (1 if amax else 0)


def _quantize_per_tensor(xt):
    xt = np.asarray(xt, dtype=np.float64)
    e = _orig_scale_exp(np.abs(xt).max())
    return vo.e4m3_round(xt * 2.0 ** -e) * 2.0 ** e, np.full(len(xt), e, dtype=np.int64)


_orig_scale_exp = vo.tile_scale_exponent
_orig_recall = vo.tile_recall
_orig_two_stream = vo.allowed_two_stream
_orig_segment_tiles = vo.segment_tiles
_orig_tile_map = vo.tile_map
_orig_trippool = vo.pool_trippool
_orig_scores = vo.tile_scores
_orig_softmax = vo.softmax_attention
_orig_allowed = vo.allowed_tiles

GEOM = tm_.GEOMS[1]


def _run_map_pin():
    tm_.test_map_matches_token_to_slot_enumeration(*GEOM)


def _run_prefix_pin():
    tm_.test_prefix_tiles_are_segment_pure(*tm_.GEOMS[0])


CASES = [
    ("tile_map", _map_swapped_xy, _run_map_pin),
    ("tile_map", _map_prefix_shared, _run_prefix_pin),
    ("pool_mean_gate", _pool_mean_with_pads, tp.test_mean_gate_constant_tile_closed_form),
    ("pool_trippool", _trippool_wrong_order, tp.test_trippool_order_and_values_by_hand),
    ("pool_trippool", _trippool_maxmin_swapped, tp.test_tripool_modes_by_hand),
    ("pool_trippool", _trippool_avg_with_pads, tp.test_tripool_avg_is_the_projected_mean_gate),
    ("tile_scores", _scores_transposed, tp.test_scores_direct_formula_and_orientation),
    ("select_topk", _select_high_index_ties, ts.test_ties_go_to_lower_index_and_signed_zero_ties),
    ("keep_count", _keep_count_float_ceil, ts.test_keep_count_exact_where_float_ceil_is_not),
    ("softmax_attention", _softmax_no_scale, ta.test_full_keep_equals_dense),
    ("allowed_tiles", _allowed_no_prefix_rows,
     lambda: ta.test_prefix_rows_are_dense_at_any_sparsity(0.75)),
    ("allowed_two_stream", _two_stream_reference_dense, tts.test_allowed_sets_by_brute_force),
    ("segment_tiles", _segment_tiles_shifted, tts.test_segment_tiles_follow_the_tile_map),
    ("teacher_tile_map", _teacher_max_logit, tte.test_teacher_map_by_brute_force),
    ("tile_recall", _recall_over_n, tte.test_tile_recall_hand_cases),
    ("e4m3_round", _e4m3_ties_away, tf8.test_e4m3_code_table_fixed_points_and_even_ties),
    ("tile_scale_exponent", _scale_exponent_plus_one, tf8.test_tile_scale_exponent_brute_force),
    ("quantize_tiles_e4m3", _quantize_per_tensor,
     tf8.test_quantize_tiles_error_bound_and_per_tile_scale),
]


@pytest.mark.parametrize("name,bad,pin", CASES, ids=[c[0] + "-" + c[1].__name__ for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, bad, pin):
    monkeypatch.setattr(vo, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    with pytest.raises(AssertionError):
        pin()


@pytest.mark.parametrize("name,bad,pin", CASES[:1], ids=["sanity"])
def test_pins_pass_on_the_real_oracle(name, bad, pin):
    pin()
