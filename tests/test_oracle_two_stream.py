"""Pins of the oracle's two-stream budget (reference-to-video).

The reference-image segment becomes a sparse stream with its own top-k per
video query tile; other prefix segments stay dense keys and every prefix
query row stays dense ("BSAI-ComfyUI-VedaSparse" README, section "v3.4.2
Vendored Official Veda (Pull-and-Go)", R2VA predictor row).
"""

import numpy as np
import pytest

import oracle
from workloads.configs import Workload
from workloads.inputs import head_qkv, make_weights

W = Workload("two-stream-tiny", "f32", 1, 1, 32, (4, 8, 8), (40, 150, 24),
             ((4, 4, 4),), "mean_gate", 0.5, 3001)
REF = 1                                   # the 150-token segment: 3 tiles


def _run(w, budget, **kw):
    q, k, v = head_qkv(w, 0, 0)
    wt = make_weights(w)
    wq = wt["gate"][0] if w.scorer == "mean_gate" else wt["proj_q"][0]
    wk = None if w.scorer == "mean_gate" else wt["proj_k"][0]
    return oracle.head_forward(q, k, v, w.grid, w.prefix, w.tile_shapes[0], w.sparsity,
                               w.scorer, wq, wk, ref_budget=budget, **kw), (q, k, v)


def test_segment_tiles_follow_the_tile_map():
    tm = oracle.tile_map(*W.grid, W.prefix, W.tile_shapes[0])
    got = oracle.segment_tiles(W.prefix, REF)
    np.testing.assert_array_equal(got, [1, 2, 3])
    toks = np.concatenate([tm.tile_tokens(t) for t in got])
    np.testing.assert_array_equal(toks, np.arange(40, 190))
    assert oracle.segment_tiles((64, 0, 5), 1).size == 0


def test_full_reference_budget_equals_the_single_stream_path():
    r1, _ = _run(W, (REF, 3))
    r0, _ = _run(W, None)
    np.testing.assert_array_equal(r1["allow"], r0["allow"])
    np.testing.assert_allclose(r1["out"], r0["out"], rtol=0, atol=0)


def test_allowed_sets_by_brute_force():
    k_ref = 2
    r, _ = _run(W, (REF, k_ref))
    tm, npf = r["tmap"], r["tmap"].n_prefix_tiles
    ref = [1, 2, 3]

    def ranked(row, k):
        n = row.size
        rank = [sum(row[j2] > row[j] for j2 in range(n)) +
                sum(row[j2] == row[j] for j2 in range(j)) for j in range(n)]
        return {j for j in range(n) if rank[j] < k}

    for tq in range(tm.n_tiles):
        allowed = set(np.nonzero(r["allow"][tq])[0].tolist())
        if tq < npf:
            assert allowed == set(range(tm.n_tiles))          # conditioning rows dense
            continue
        i = tq - npf
        want = {0, 4}                                          # text and audio stay dense
        want |= {ref[j] for j in ranked(r["ref_scores"][i], k_ref)}
        want |= {npf + j for j in ranked(r["scores"][i], r["k"])}
        assert allowed == want


def test_reference_scores_use_the_reference_tiles_descriptors():
    r, (q, k, v) = _run(W, (REF, 1))
    tm = r["tmap"]
    gate = make_weights(W)["gate"][0].astype(np.float64)
    for col, tile in enumerate([1, 2, 3]):
        toks = tm.tile_tokens(tile)
        khat = k[toks].astype(np.float64).mean(axis=0) @ gate
        np.testing.assert_allclose(r["khat_ref"][col], khat, rtol=1e-13, atol=1e-13)
        want = (r["qhat"] @ khat).astype(np.float32)
        np.testing.assert_array_equal(r["ref_scores"][:, col], want)


def test_prefix_rows_do_not_depend_on_the_reference_budget():
    outs = []
    for k_ref in (1, 2, 3):
        r, _ = _run(W, (REF, k_ref))
        tm = r["tmap"]
        rows = np.concatenate([tm.tile_tokens(t) for t in range(tm.n_prefix_tiles)])
        outs.append(r["out"][rows])
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("k_ref", [1, 2])
def test_video_rows_match_attention_over_the_explicit_key_set(k_ref):
    r, (q, k, v) = _run(W, (REF, k_ref))
    tm = r["tmap"]
    scale = 1.0 / np.sqrt(W.d)
    for tq in range(tm.n_prefix_tiles, tm.n_tiles):
        rows = tm.tile_tokens(tq)
        keys = np.concatenate([tm.tile_tokens(t) for t in np.nonzero(r["allow"][tq])[0]])
        lg = (q[rows].astype(np.float64) @ k[keys].astype(np.float64).T) * scale
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        o = (p / p.sum(axis=1, keepdims=True)) @ v[keys].astype(np.float64)
        np.testing.assert_allclose(r["out"][rows], o, rtol=1e-12, atol=1e-12)


def test_trippool_reference_stream():
    w = Workload("two-stream-trip", "f32", 1, 1, 32, (4, 8, 8), (40, 150, 24),
                 ((1, 8, 8),), "trippool", 0.5, 3002, proj_dim=8)
    r, _ = _run(w, (REF, 2))
    assert r["khat_ref"].shape == (3, 24)
    assert r["kv_ref"].shape == (r["tmap"].n_video_tiles, 2)
    for row in r["kv_ref"]:
        assert list(row) == sorted(set(row)) and all(0 <= j < 3 for j in row)


def test_ties_in_the_reference_stream_go_to_the_lower_index():
    tm = oracle.tile_map(4, 8, 8, (40, 150, 24), (4, 4, 4))
    ref = oracle.segment_tiles((40, 150, 24), 1)
    scores = np.zeros((tm.n_video_tiles, ref.size), dtype=np.float32)
    kv_ref = oracle.select_topk(scores, 2)
    assert all(list(row) == [0, 1] for row in kv_ref)
    allow = oracle.allowed_two_stream(tm, [[0]] * tm.n_video_tiles, ref, kv_ref)
    for tq in range(tm.n_prefix_tiles, tm.n_tiles):
        assert allow[tq, 1] and allow[tq, 2] and not allow[tq, 3]
