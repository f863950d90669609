"""Seeded synthetic inputs shared by the oracle side and the library side.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no tiling, pooling, scoring, selection or attention).

Recipe (every draw is seeded, per (seed, tensor, batch, head) so that any
subset of heads can be regenerated on its own):

* Video token at latent position (t, y, x), channel c, head h:
      X = z + 0.5 * sin(2*pi*(f_t*t/T + f_y*y/Hv + f_x*x/Wv) + phi)
  with z ~ N(0, 1) i.i.d. (float32), integer frequencies f_* drawn uniformly
  from {0, 1, 2} and phi ~ U[0, 2*pi), drawn per (head, channel). Q and K
  share (f, phi) so that nearby tiles correlate the way video attention does;
  V draws its own. Prefix tokens (text, reference image, reference audio) have
  no 3D position and are z only. Video tokens follow the prefix, row-major in
  (t, y, x).
* Per-head gate G_h (d x d) ~ N(0, 1/d) for the mean-pool gate scorer, and
  per-head projections Pq_h, Pk_h (d x proj_dim) ~ N(0, 1/d) for TripPool,
  all float32.
* bf16 workloads round Q, K and V to bfloat16 (round to nearest even) once,
  here; both sides read exactly those values.
* Score rows for the select step alone (row lengths no workload reaches):
  even rows N(0, 1) float32; odd rows drawn from the 81 levels j/8,
  j = -40..40, so that exact ties are common, with -0.0 in place of +0.0 in
  every other tied zero.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

_TAG = {"q": 1, "k": 2, "v": 3, "qk_wave": 4, "v_wave": 5,
        "gate": 6, "proj_q": 7, "proj_k": 8, "score_rows": 9}


def _rng(seed: int, tag: str, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, _TAG[tag], b, h])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even)."""
    return bf16_to_f32(bf16_bits(x))


def _wave_params(w: Workload, tag: str, b: int, h: int):
    g = _rng(w.seed, tag, b, h)
    freq = g.integers(0, 3, size=(3, w.d))            # (f_t, f_y, f_x) per channel
    phase = g.uniform(0.0, 2.0 * np.pi, size=w.d)
    return freq, phase


def _video_wave(w: Workload, freq: np.ndarray, phase: np.ndarray) -> np.ndarray:
    T, Hv, Wv = w.grid
    t = np.arange(T, dtype=np.float64)[:, None, None, None]
    y = np.arange(Hv, dtype=np.float64)[None, :, None, None]
    x = np.arange(Wv, dtype=np.float64)[None, None, :, None]
    arg = (freq[0] * t / T + freq[1] * y / Hv + freq[2] * x / Wv)
    wave = 0.5 * np.sin(2.0 * np.pi * arg + phase)
    return wave.reshape(T * Hv * Wv, w.d)


def head_qkv(w: Workload, b: int, h: int):
    """Q, K, V of one (batch, head) as float32 [N, d] (bf16-exact for bf16)."""
    P = sum(w.prefix)
    out = []
    qk_wave = _video_wave(w, *_wave_params(w, "qk_wave", b, h))
    v_wave = _video_wave(w, *_wave_params(w, "v_wave", b, h))
    for tag, wave in (("q", qk_wave), ("k", qk_wave), ("v", v_wave)):
        z = _rng(w.seed, tag, b, h).standard_normal((w.N, w.d), dtype=np.float32)
        x = z.astype(np.float64)
        x[P:] += wave
        x = x.astype(np.float32)
        if w.dtype == "bf16":
            x = bf16_round(x)
        out.append(x)
    return tuple(out)


def make_qkv(w: Workload, heads=None, batches=None, as_bf16_bits: bool = False):
    """Q, K, V as [B', H', N, d] arrays for the selected batches and heads.

    float32 by default (bf16-exact values for bf16 workloads); with
    ``as_bf16_bits`` the bf16 bit patterns as uint16 (half the memory).
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    batches = list(range(w.B)) if batches is None else list(batches)
    dt = np.uint16 if as_bf16_bits else np.float32
    shape = (len(batches), len(heads), w.N, w.d)
    q, k, v = (np.empty(shape, dtype=dt) for _ in range(3))

    def fill(job):
        bi, b, hi, h = job
        for dst, src in zip((q, k, v), head_qkv(w, b, h)):
            dst[bi, hi] = bf16_bits(src) if as_bf16_bits else src

    jobs = [(bi, b, hi, h) for bi, b in enumerate(batches) for hi, h in enumerate(heads)]
    # Every (batch, head) has its own random streams, so the heads are drawn
    # in parallel threads (NumPy releases the GIL in its array kernels); the
    # values do not depend on the thread count.
    workers = min(len(jobs), int(os.environ.get("VSA_INPUT_THREADS", "0"))
                  or min(16, os.cpu_count() or 1))
    if workers <= 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, jobs))
    return q, k, v


def make_weights(w: Workload) -> dict:
    """Per-head scorer weights, float32.

    mean_gate: {"gate": [H, d, d]};  trippool: {"proj_q", "proj_k": [H, d, P]}.
    """
    std = 1.0 / np.sqrt(w.d)
    if w.scorer == "mean_gate":
        gate = np.stack([_rng(w.seed, "gate", 0, h).standard_normal(
            (w.d, w.d)) * std for h in range(w.H)]).astype(np.float32)
        return {"gate": gate}
    pq = np.stack([_rng(w.seed, "proj_q", 0, h).standard_normal(
        (w.d, w.proj_dim)) * std for h in range(w.H)]).astype(np.float32)
    pk = np.stack([_rng(w.seed, "proj_k", 0, h).standard_normal(
        (w.d, w.proj_dim)) * std for h in range(w.H)]).astype(np.float32)
    return {"proj_q": pq, "proj_k": pk}


def score_rows(seed: int, n_rows: int, n: int) -> np.ndarray:
    """float32 [n_rows, n] synthetic tile scores (see the recipe above)."""
    g = _rng(seed, "score_rows", 0, 0)
    out = g.standard_normal((n_rows, n), dtype=np.float32)
    levels = g.integers(-40, 41, size=(n_rows // 2, n)).astype(np.float32) / np.float32(8.0)
    zero = levels == 0
    levels[zero & (np.arange(n)[None, :] % 2 == 1)] = np.float32(-0.0)
    out[1::2] = levels
    return out
