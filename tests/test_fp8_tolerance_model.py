"""Where the fp8 tolerances come from (CPU only).

The fp8 kernel computes attention over the E4M3 inputs exactly except for one
rounding: every probability 2^(x - m) (m kept 8 below the row max, in log2
units) is rounded to E4M3 before it weights V, and the row sum is taken over
the rounded values. This model applies that rounding to exact logits of the
small fp8 GPU test workloads (whose rows see the fewest keys, so the largest
errors), on random selections of the same size, and checks that the output
and LSE errors stay within 0.6 of the tolerances the GPU tests use; the rest
of the margin covers the f8 MFMA's own summation (about 2^-13 relative per 64
products) and the bf16 store of the output.
"""
import numpy as np

import oracle
from tests import gpu_support as gs
from tests.test_gpu_fp8 import SMALL
from workloads.inputs import head_qkv


def _model_rows(qq, kq, vq, tm, allow, scale, rows):
    out, lse = [], []
    for tq in rows:
        qs = tm.tile_tokens(tq)
        keys = np.concatenate([tm.tile_tokens(t) for t in np.nonzero(allow[tq])[0]])
        x = (qq[qs] @ kq[keys].T) * scale / np.log(2.0)
        m = np.ceil(x.max(axis=1, keepdims=True)) - 8.0
        p = oracle.e4m3_round(np.exp2(x - m))
        out.append((p @ vq[keys]) / p.sum(axis=1, keepdims=True))
        lse.append((m[:, 0] + np.log2(p.sum(axis=1))) * np.log(2.0))
    return np.concatenate(out), np.concatenate(lse)


def _model_worst(workloads):
    worst = [0.0, 0.0, 0.0]
    for w in workloads:
        scale = 1.0 / np.sqrt(w.d)
        for h in range(w.H):
            rng = np.random.default_rng(h)
            q, k, v = head_qkv(w, 0, h)
            tm = oracle.tile_map(*w.grid, w.prefix, w.tile_shapes[h % len(w.tile_shapes)])
            qq, kq, vq = oracle.fp8_attention_inputs(q, k, v, tm)
            kk = oracle.keep_count(w.sparsity, tm.n_video_tiles)
            sel = np.sort(np.stack([rng.choice(tm.n_video_tiles, kk, replace=False)
                                    for _ in range(tm.n_video_tiles)]), axis=1)
            allow = oracle.allowed_tiles(tm, sel)
            rows = list(range(tm.n_tiles))
            want, lse_want = oracle.sparse_attention(qq, kq, vq, tm, allow, scale, rows)
            got, lse_got = _model_rows(qq, kq, vq, tm, allow, scale, rows)
            tok = np.concatenate([tm.tile_tokens(t) for t in rows])
            err = np.abs(got - want[tok])
            lerr = np.abs(lse_got - lse_want[tok])
            worst = [max(worst[0], err.max()), max(worst[1], err.mean()),
                     max(worst[2], lerr.max())]
    return worst


def test_probability_rounding_error_is_within_the_fp8_tolerance():
    worst = _model_worst(SMALL.values())
    assert worst[0] <= 0.6 * gs.FP8_MAX_ABS
    assert worst[1] <= 0.6 * gs.FP8_MEAN_ABS
    assert worst[2] <= 0.6 * gs.FP8_LSE_ABS
    # the rounding does matter: well above the bf16 path's error bounds
    assert worst[2] > 4 * gs.BF16_LSE_ABS and worst[0] > 0.5 * gs.BF16_MAX_ABS


def test_short_rows_are_within_the_edge_tolerance():
    """The edge workloads' rows see 192 to 768 keys; the same model on them
    stays within 0.6 of the short-row tolerances, and needs them: it exceeds
    the long-row LSE bound."""
    from tests.test_gpu_edge import EDGE
    names = ("ragged-headaware-b2", "no-prefix-d64", "keep-all", "top-1", "proj64-many-shapes")
    worst = _model_worst(EDGE[n] for n in names)
    assert worst[0] <= 0.6 * gs.FP8_EDGE_MAX_ABS
    assert worst[1] <= 0.6 * gs.FP8_EDGE_MEAN_ABS
    assert worst[2] <= 0.6 * gs.FP8_EDGE_LSE_ABS
    assert worst[2] > gs.FP8_LSE_ABS
