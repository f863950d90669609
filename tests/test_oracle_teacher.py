"""Pins of the oracle's teacher tile map (full attention, max-pooled per tile
pair) and of tile recall ("Veda Sparse Attention в ComfyUI", section "Что
делает Veda"; "BSAI-ComfyUI-VedaSparse" README, Overview table)."""

import numpy as np

import oracle
from workloads.configs import Workload
from workloads.inputs import head_qkv

W = Workload("teacher-tiny", "f32", 1, 1, 32, (4, 8, 12), (40, 24),
             ((4, 4, 4),), "mean_gate", 0.5, 5001)


def _inputs():
    q, k, v = head_qkv(W, 0, 0)
    tm = oracle.tile_map(*W.grid, W.prefix, W.tile_shapes[0])
    return q, k, tm


def test_teacher_map_by_brute_force():
    q, k, tm = _inputs()
    scale = 1.0 / np.sqrt(W.d)
    got = oracle.teacher_tile_map(q, k, tm, scale)
    real = [t for t in range(tm.n_tiles) for _ in [0]]
    toks = {t: list(tm.tile_tokens(t)) for t in range(tm.n_tiles)}
    all_keys = [x for t in range(tm.n_tiles) for x in toks[t]]
    npf = tm.n_prefix_tiles
    for i in range(tm.n_video_tiles):
        for j in range(tm.n_video_tiles):
            best = 0.0
            for qi in toks[npf + i]:
                row = [float(np.dot(q[qi].astype(np.float64), k[kk].astype(np.float64))) * scale
                       for kk in all_keys]
                m = max(row)
                den = sum(np.exp(x - m) for x in row)
                for kk in toks[npf + j]:
                    p = np.exp(float(np.dot(q[qi].astype(np.float64),
                                            k[kk].astype(np.float64))) * scale - m) / den
                    best = max(best, p)
            assert abs(got[i, j] - best) <= 1e-12 * max(1.0, best)
    assert real  # every tile was visited


def test_teacher_values_are_probabilities_and_peak_on_a_dominant_key():
    q, k, tm = _inputs()
    q, k = q.copy(), k.copy()
    npf = tm.n_prefix_tiles
    rows = tm.tile_tokens(npf + 0)
    q[rows] = q[rows[0]]                                  # every query of tile 0 alike
    target = tm.tile_tokens(npf + 2)[5]
    k[target] = 1e3 * q[rows[0]]                          # one key dominates them all
    got = oracle.teacher_tile_map(q, k, tm, 1.0 / np.sqrt(W.d), query_tiles=[0])
    assert np.all(got >= 0) and np.all(got <= 1.0 + 1e-15)
    assert abs(got[0, 2] - 1.0) < 1e-9
    assert np.all(np.delete(got[0], 2) < 1e-6)


def test_tile_recall_hand_cases():
    teacher = np.array([[0.9, 0.1, 0.5, 0.3],
                        [0.2, 0.2, 0.8, 0.1]])           # top-2: {0, 2} and {2, 0}
    assert oracle.tile_recall(np.array([[0, 2], [0, 2]]), teacher, 2) == 1.0
    assert oracle.tile_recall(np.array([[1, 3], [1, 3]]), teacher, 2) == 0.0
    # row 0 keeps 0 (hit) and 1 (miss); row 1 keeps 1 (miss: tie goes to 0) and 2 (hit)
    assert oracle.tile_recall(np.array([[0, 1], [1, 2]]), teacher, 2) == 0.5


def test_recall_of_the_teachers_own_selection_is_one():
    q, k, tm = _inputs()
    t = oracle.teacher_tile_map(q, k, tm, 1.0 / np.sqrt(W.d))
    top = oracle.select_topk(t.astype(np.float32), 3)
    assert oracle.tile_recall(top, t, 3) == 1.0
