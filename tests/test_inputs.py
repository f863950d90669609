"""The seeded input generator: determinism and the stated recipe (CPU only)."""
import dataclasses

import numpy as np

from workloads import WORKLOADS, Workload
from workloads.inputs import (bf16_bits, bf16_round, bf16_to_f32, head_qkv,
                              make_qkv, make_weights)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                  -2.5, 3.0e38], dtype=np.float32)
    got = bf16_round(x)
    np.testing.assert_array_equal(got[:3], [1.0, 1.0, 1.0 + 2 ** -6])
    assert got[3] == 1.0 and got[4] == -2.5
    np.testing.assert_array_equal(bf16_to_f32(bf16_bits(got)), got)


def test_heads_regenerate_independently():
    w = WORKLOADS["1"]
    q, k, v = make_qkv(w)
    q1, k1, v1 = head_qkv(w, 0, 1)
    np.testing.assert_array_equal(q[0, 1], q1)
    np.testing.assert_array_equal(v[0, 1], v1)
    q2, _, _ = make_qkv(w, heads=[1])
    np.testing.assert_array_equal(q2[0, 0], q1)
    assert not np.array_equal(q[0, 0], q[0, 1])


def test_bf16_workload_values_are_bf16_exact():
    w = Workload("t", "bf16", 1, 2, 16, (4, 4, 8), (3, 5), ((4, 4, 4),),
                 "mean_gate", 0.5, 7)
    q, k, v = make_qkv(w)
    np.testing.assert_array_equal(bf16_round(q), q)
    bits = make_qkv(w, as_bf16_bits=True)[2]
    np.testing.assert_array_equal(bf16_to_f32(bits), v)


def test_q_and_k_share_the_video_wave():
    # Q - K on video tokens is pure noise difference: its mean over tokens is ~0
    # while Q itself carries the 0.5-amplitude wave per channel.
    w = Workload("t", "f32", 1, 1, 8, (4, 16, 16), (0,), ((4, 4, 4),),
                 "mean_gate", 0.5, 11)
    q, k, v = head_qkv(w, 0, 0)
    assert np.abs((q - k).mean(axis=0)).max() < 0.1
    assert q.shape == (1024, 8)


def test_weights_shapes_and_scale():
    w = WORKLOADS["2"]
    g = make_weights(w)["gate"]
    assert g.shape == (24, 128, 128) and g.dtype == np.float32
    assert abs(g.std() - 1 / np.sqrt(128)) < 2e-3
    p = make_weights(WORKLOADS["4a"])
    assert p["proj_q"].shape == (24, 128, 32)
    assert not np.array_equal(p["proj_q"], p["proj_k"])


def test_parallel_generation_matches_sequential(monkeypatch):
    """Heads drawn in parallel threads give the same values as one thread."""
    w = dataclasses.replace(WORKLOADS["1"], H=5)
    monkeypatch.setenv("VSA_INPUT_THREADS", "4")
    par = make_qkv(w)
    monkeypatch.setenv("VSA_INPUT_THREADS", "1")
    seq = make_qkv(w)
    for a, b in zip(par, seq):
        np.testing.assert_array_equal(a, b)
