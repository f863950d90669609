"""Pins of the oracle's fp8 (OCP E4M3) quantization (CPU only).

e4m3_round is checked against torch's float8_e4m3fn cast (a library
routine) and against the format's own value table, read out of torch by
decoding all 256 codes: every finite code value is a fixed point, every
midpoint between neighbours goes to the neighbour with the even code. The
tile exponent is checked by brute force over e; per-tile quantization
against the e4m3 error bound and against tiles of very different scale.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _code_values():
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    return v.numpy()


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    parts = [rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]
    x = np.concatenate(parts + [rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_round(x), want)


def test_e4m3_code_table_fixed_points_and_even_ties():
    vals = _code_values()
    codes = np.arange(256)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254 and vals[finite].max() == 448.0 == oracle.E4M3_MAX
    np.testing.assert_array_equal(oracle.e4m3_round(vals[finite]), vals[finite])
    # positive codes 0..126 are increasing; midpoints tie to the even code
    pos = vals[:127]
    assert np.all(np.diff(pos) > 0)
    mids = (pos[:-1] + pos[1:]) / 2
    even_nb = np.where(codes[:126] % 2 == 0, pos[:-1], pos[1:])
    np.testing.assert_array_equal(oracle.e4m3_round(mids), even_nb)
    np.testing.assert_array_equal(oracle.e4m3_round(-mids), -even_nb)
    # a hair either side of a midpoint goes to the nearer neighbour
    eps = (pos[1:] - pos[:-1]) * 1e-3
    np.testing.assert_array_equal(oracle.e4m3_round(mids - eps), pos[:-1])
    np.testing.assert_array_equal(oracle.e4m3_round(mids + eps), pos[1:])


def test_e4m3_round_rejects_out_of_range():
    for bad in (448.5, -1000.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            oracle.e4m3_round([bad])


def test_tile_scale_exponent_brute_force():
    rng = np.random.default_rng(12)
    amaxes = np.concatenate([np.exp(rng.uniform(-30, 30, 4000)),
                             [448.0, 448.0 * (1 + 2 ** -40), 224.0, 224.0 * (1 - 2 ** -40),
                              1.0, 2.0 ** -149, 3.0e38]])
    for a in amaxes:
        e = oracle.tile_scale_exponent(a)
        assert math.ldexp(a, -e) <= 448.0          # in range
        if e > -127:
            assert math.ldexp(a, -(e - 1)) > 448.0     # and e is the least such
        else:                                      # clamped: the scale byte's floor
            assert a <= math.ldexp(448.0, -127)
    assert oracle.tile_scale_exponent(0.0) == 0
    assert oracle.tile_scale_exponent(2.0 ** -149) == -127
    assert oracle.tile_scale_exponent(math.ldexp(448.0, -127)) == -127
    assert oracle.tile_scale_exponent(math.ldexp(449.0, -127)) == -126


def test_quantize_tiles_error_bound_and_per_tile_scale():
    rng = np.random.default_rng(13)
    xt = rng.standard_normal((3, 64, 16))
    xt[1] *= 1e-4                                    # a tile 10^4 times smaller
    xt[2] = 0.0                                      # an all-zero tile
    xq, exps = oracle.quantize_tiles_e4m3(xt)
    assert exps[2] == 0 and not xq[2].any()
    for t in range(2):
        e = int(exps[t])
        assert 224.0 < np.abs(xt[t]).max() * 2.0 ** -e <= 448.0
        # normals: relative error <= 2^-4; subnormals: absolute <= 2^(e-10)
        err = np.abs(xq[t] - xt[t])
        bound = np.maximum(np.abs(xt[t]) * 2.0 ** -4, 2.0 ** (e - 10))
        assert np.all(err <= bound)
        # the small tile keeps its own precision (a per-tensor scale would not)
        assert np.median(err / np.abs(xt[t])) < 3e-2
    # values already on the scaled grid are unchanged
    np.testing.assert_array_equal(oracle.quantize_tiles_e4m3(xq)[0], xq)


def test_ungather_inverts_gather_on_real_tokens():
    tm = oracle.tile_map(3, 5, 7, (40, 70), (4, 4, 4))
    n = 40 + 70 + 3 * 5 * 7
    x = np.random.default_rng(14).standard_normal((n, 8))
    np.testing.assert_array_equal(oracle.ungather(oracle.gather(x, tm), tm, n), x)


def test_fp8_inputs_keep_all_attention_is_dense_attention_on_quantized_values():
    tm = oracle.tile_map(2, 8, 8, (40,), (4, 4, 4))
    n = 40 + 128
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((n, 16)) for _ in range(3))
    qq, kq, vq = oracle.fp8_attention_inputs(q, k, v, tm)
    for a, b in ((q, qq), (k, kq), (v, vq)):
        assert np.abs(a - b).max() <= np.abs(a).max() * 2.0 ** -4
        assert not np.array_equal(a, b)
    allow = oracle.allowed_tiles(tm, oracle.select_topk(
        np.zeros((tm.n_video_tiles, tm.n_video_tiles), np.float32), tm.n_video_tiles))
    out, lse = oracle.sparse_attention(qq, kq, vq, tm, allow, 0.25)
    o2, l2 = oracle.dense_attention(qq, kq, vq, 0.25)
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)
