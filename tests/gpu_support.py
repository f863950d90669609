"""Helpers for the GPU parity tests: run the library, run the oracle on the
same seeded inputs, unpack the tiled layouts, and compare.

The tiled-layout formulas below are restated from include/vsa.h (the ABI
contract); they are test-side readers of the library's output, not shared
code. Nothing here computes any step of the method: the expected values come
from the oracle alone.
"""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np

import oracle
from workloads import Workload
from workloads.inputs import bf16_to_f32, make_qkv, make_weights


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------ tiled layouts

def row_layout_index(d: int) -> np.ndarray:
    """perm[s*d + c] = offset of (slot s, channel c) in a Q/K tile."""
    s = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    off = ((s // 32) * (d // 16) + c // 16) * 512 + (((c % 16) // 8) * 32 + s % 32) * 8 + c % 8
    return off.reshape(-1)


def col_layout_index(d: int) -> np.ndarray:
    """perm[s*d + c] = offset of (slot s, channel c) in a V tile."""
    s = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    off = ((c // 32) * 4 + s // 16) * 512 + (((s % 8) // 4) * 32 + c % 32) * 8 \
        + ((s % 16) // 8) * 4 + s % 4
    return off.reshape(-1)


def fp8_row_layout_index(d: int) -> np.ndarray:
    """perm[s*d + c] = byte offset of (slot s, channel c) in an fp8 Q/K tile."""
    s = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    w = c % 64
    off = ((s // 32) * (d // 64) + c // 64) * 2048 + ((w % 32) // 16) * 1024 \
        + (s % 32 + 32 * (w // 32)) * 16 + w % 16
    return off.reshape(-1)


def fp8_col_layout_index(d: int) -> np.ndarray:
    """perm[s*d + c] = byte offset of (key s, channel c) in an fp8 V tile."""
    s = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    w = s % 32
    g, r = (w // 4) % 2, (w // 8) * 4 + w % 4
    off = (c // 32) * 2048 + (s // 32) * 1024 + (c % 32 + 32 * g) * 16 + r
    return off.reshape(-1)


def unpack_fp8_tiles(codes: np.ndarray, exps: np.ndarray, n_tiles: int, d: int,
                     col: bool) -> np.ndarray:
    """uint8 E4M3 codes in the fp8 layout -> [n_tiles, 64, d] float64 values
    times 2^exps[tile]."""
    import torch
    perm = fp8_col_layout_index(d) if col else fp8_row_layout_index(d)
    t = np.ascontiguousarray(codes[: n_tiles * 64 * d].reshape(n_tiles, 64 * d)[:, perm])
    vals = torch.from_numpy(t).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals.reshape(n_tiles, 64, d) * np.exp2(exps[:n_tiles].astype(np.float64))[:, None, None]


def unpack_tiles(flat: np.ndarray, n_tiles: int, d: int, col: bool) -> np.ndarray:
    """[n_tiles*64*d] tiled layout -> [n_tiles, 64, d] plain rows."""
    perm = col_layout_index(d) if col else row_layout_index(d)
    t = flat[: n_tiles * 64 * d].reshape(n_tiles, 64 * d)
    return t[:, perm].reshape(n_tiles, 64, d)


# ------------------------------------------------------------ library runs

@dataclass
class GpuRun:
    w: Workload
    prob: object
    layer: object
    q: object
    k: object
    v: object
    wq: object
    wk: object


def to_device(w: Workload, heads=None, arrays=None):
    """Q, K, V on the device; ``arrays`` (float32 [B, H, N, d], bf16-exact for
    bf16 workloads) overrides the seeded generator."""
    import torch
    from workloads.inputs import bf16_bits
    if arrays is None:
        q, k, v = make_qkv(w, heads=heads, as_bf16_bits=(w.dtype == "bf16"))
    elif w.dtype == "bf16":
        q, k, v = (bf16_bits(np.ascontiguousarray(a, dtype=np.float32)) for a in arrays)
    else:
        q, k, v = (np.ascontiguousarray(a, dtype=np.float32) for a in arrays)
    if w.dtype == "bf16":
        t = [torch.from_numpy(x).view(torch.bfloat16).cuda() for x in (q, k, v)]
    else:
        t = [torch.from_numpy(x).cuda() for x in (q, k, v)]
    return t


def make_qkv_f32(w: Workload):
    """The workload's seeded Q, K, V as float32 [B, H, N, d] (bf16-exact for
    bf16 workloads)."""
    q, k, v = make_qkv(w, as_bf16_bits=(w.dtype == "bf16"))
    if w.dtype == "bf16":
        return tuple(bf16_to_f32(x) for x in (q, k, v))
    return q, k, v


def rising_exact_arrays(w: Workload, tm):
    """Inputs on which the attention kernels are exact up to the bf16 store of
    their output, while their running max rises along every key list.
    Q and K are small integers: every query has 2 in channels 0..63, every key
    of tile t has 1 in channels 0..t-1, and channels 64..66 of both are random
    in {-1, 0, 1}. So q.k = 2t + r with r in [-3, 3]. With softmax scale ln 2,
    the kernels' logits in log2 units are these integers, every probability is
    a power of two that E4M3 and bf16 hold exactly, and every key tile lifts
    the max by about 2, so the max is raised again and again along each key
    list. V is the seeded bf16 V."""
    assert tm.n_tiles <= 64 and w.d >= 67
    rng = np.random.default_rng(11)
    q, k, v = (np.asarray(a, dtype=np.float32).copy() for a in make_qkv_f32(w))
    q[...] = 0.0
    k[...] = 0.0
    q[..., :64] = 2.0
    q[..., 64:67] = rng.integers(-1, 2, size=q[..., 64:67].shape)
    for t in range(tm.n_tiles):
        k[:, :, tm.tile_tokens(t), :t] = 1.0
    k[..., 64:67] = rng.integers(-1, 2, size=k[..., 64:67].shape)
    return q, k, v


def problem_of(w: Workload, H=None):
    from block_sparse_video_map_amd import vsa
    return vsa.Problem(w.B, w.H if H is None else H, w.d, w.grid, w.prefix, w.tile_shapes,
                       w.dtype)


def run_library(w: Workload, sparsity=None, stages=("map", "score", "select", "attn"),
                arrays=None, ref=None):
    """Runs the library's layer on the workload's seeded inputs (all heads);
    ``ref`` = (segment, k_ref) turns on the two-stream budget."""
    import torch
    from block_sparse_video_map_amd import vsa
    sp = w.sparsity if sparsity is None else sparsity
    prob = problem_of(w)
    mode = vsa.score_mode(w.scorer, w.tripool_mode)
    proj = w.d if w.scorer == "mean_gate" else w.proj_dim
    layer = vsa.Layer(prob, sp, mode, proj, ref=ref)
    q, k, v = to_device(w, arrays=arrays)
    W = make_weights(w)
    if w.scorer == "mean_gate":
        wq = torch.from_numpy(W["gate"]).cuda()
        wk = None
    else:
        wq = torch.from_numpy(W["proj_q"]).cuda()
        wk = torch.from_numpy(W["proj_k"]).cuda()
    layer.map_tiles(q, k, v)
    if "score" in stages and sp != 0.0:
        layer.tile_scores(wq, wk)
    if "select" in stages and sp != 0.0:
        layer.select()
    if "attn" in stages:
        layer.attend()
    torch.cuda.synchronize()
    return GpuRun(w, prob, layer, q, k, v, wq, wk)


def assert_same_without_lse(layer, label=""):
    """Attention called without an LSE buffer, the form the benchmark times,
    writes the same output bit for bit as the call that returned one (the
    layer's current output, checked against the oracle by the caller)."""
    import torch
    out, lse = layer.out, layer.lse
    try:
        layer.out = torch.full_like(out, float("nan"))
        layer.lse = None
        layer.attend()
        torch.cuda.synchronize()
        same = torch.equal(layer.out.view(torch.uint8), out.view(torch.uint8))
    finally:
        layer.out, layer.lse = out, lse
    log(f"[no-lse]{label}: output {'identical' if same else 'DIFFERS'} without the LSE buffer")
    assert same


def fused_kv(run: GpuRun, sparsity=None):
    """kv_idx from vsa_tile_select (pooling, scores and top-k in one call) on
    the run's tiled copies, or None when the call does not take the problem."""
    import torch
    from block_sparse_video_map_amd import vsa
    w, L = run.w, run.layer
    sp = w.sparsity if sparsity is None else sparsity
    if not vsa.fused_select_supported(run.prob, L.mode, L.proj_dim, sp):
        return None
    kv = torch.full_like(L.kv_idx, -7)
    pooled = torch.empty_like(L.pooled)
    vsa.vsa_tile_select(run.prob, L.mode, L.proj_dim, L.qt, L.kt, L.slot_to_token, run.wq,
                        run.wk, sp, pooled, kv)
    torch.cuda.synchronize()
    return kv


def assert_fused_equal(run: GpuRun, sparsity=None):
    """The fused call's lists equal the two-call path's (vsa_tile_scores then
    vsa_select_topk), row for row over every head's video query tiles."""
    kvf = fused_kv(run, sparsity)
    if kvf is None:
        log(f"[fused] {run.w.name}: problem not taken by vsa_tile_select")
        return False
    sz = run.layer.sizes
    shape = (run.w.B * run.w.H, sz.max_video_tiles, sz.k_max)
    a = run.layer.kv_idx[: sz.idx_elems].view(shape).cpu().numpy()
    b = kvf[: sz.idx_elems].view(shape).cpu().numpy()
    for bh in range(shape[0]):
        n = sz.n_video_tiles[(bh % run.w.H) % len(run.w.tile_shapes)]
        np.testing.assert_array_equal(b[bh, :n], a[bh, :n])
    log(f"[fused] {run.w.name}: vsa_tile_select lists equal the two-call path's")
    return True


def assert_gather_pool_equal(run: GpuRun):
    """vsa_map_tiles_scores (the pooling done in the gather pass, then the
    scores) writes bit for bit what vsa_map_tiles + vsa_tile_scores wrote into
    the run's layer: tile map, tiled Q/K/V, descriptors and scores."""
    import torch
    from block_sparse_video_map_amd import vsa
    w, L = run.w, run.layer
    s2t = torch.full_like(L.slot_to_token, -7)
    qt, kt, vt = (torch.zeros_like(L.qt) for _ in range(3))
    pooled = torch.full_like(L.pooled, float("nan"))
    scores = torch.full_like(L.scores, float("nan"))
    vsa.vsa_map_tiles_scores(run.prob, L.mode, L.proj_dim, run.q, run.k, run.v, s2t, qt, kt, vt,
                             run.wq, run.wk, pooled, scores)
    torch.cuda.synchronize()
    sz = L.sizes
    assert torch.equal(s2t, L.slot_to_token)
    per_head = sz.max_tiles * 64 * w.d
    nv, BH = sz.max_video_tiles, w.B * w.H
    r = vsa.vsa_pooled_bytes(run.prob, L.mode, L.proj_dim) // (8 * 2 * BH * nv)
    sc_a, sc_b = L.scores.view(BH, nv, nv), scores.view(BH, nv, nv)
    pd_a = L.pooled[: 2 * BH * nv * r].view(2, BH, nv, r)
    pd_b = pooled[: 2 * BH * nv * r].view(2, BH, nv, r)
    for bh in range(BH):
        si = (bh % w.H) % len(w.tile_shapes)
        nt, n = sz.n_tiles[si], sz.n_video_tiles[si]
        for a, b in ((L.qt, qt), (L.kt, kt), (L.vt, vt)):
            seg = slice(bh * per_head, bh * per_head + nt * 64 * w.d)
            assert torch.equal(a[seg], b[seg]), bh
        assert torch.equal(pd_a[:, bh, :n], pd_b[:, bh, :n]), bh
        assert torch.equal(sc_a[bh, :n, :n], sc_b[bh, :n, :n]), bh
    log(f"[gather-pool] {w.name}: one-pass gather and pooling equal the two calls")
    return True


def tensor_f32(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


# ------------------------------------------------------------ oracle runs

def head_inputs(w: Workload, h: int, b: int = 0):
    from workloads.inputs import head_qkv
    return head_qkv(w, b, h)


def oracle_head(w: Workload, h: int, sparsity=None, query_tiles=(), b: int = 0,
                arrays=None, ref=None, kv_video=None, kv_ref=None):
    """The oracle's whole path for one head (attention only on query_tiles);
    ``ref`` = (segment, k_ref) as for run_library; kv_video / kv_ref replace
    the oracle's selections (to compare outputs on the GPU's selection)."""
    if arrays is None:
        q, k, v = head_inputs(w, h, b)
    else:
        q, k, v = (np.asarray(a[b, h], dtype=np.float32) for a in arrays)
    W = make_weights(w)
    shape = w.tile_shapes[h % len(w.tile_shapes)]
    if w.scorer == "mean_gate":
        wq, wk = W["gate"][h], None
    else:
        wq, wk = W["proj_q"][h], W["proj_k"][h]
    sp = w.sparsity if sparsity is None else sparsity
    qt = None if query_tiles is None else list(query_tiles)
    return oracle.head_forward(q, k, v, w.grid, w.prefix, shape, sp, w.scorer, wq, wk,
                               query_tiles=qt, ref_budget=ref, kv_video=kv_video,
                               kv_ref=kv_ref, tripool_mode=w.tripool_mode), (q, k, v)


# ------------------------------------------------------------ comparisons

def band_rule_check(scores_orc: np.ndarray, sel_gpu: np.ndarray, k: int, rel=1e-6):
    """Selection comparison with near-ties excluded.

    Returns (n_rows_differing, n_rows_with_band_gt1, failures).
    For each row: tau = k-th ranked oracle score; A = near-ties of tau. The
    GPU list must be k strictly ascending entries, contain every j outside A
    scoring above tau and no j outside A scoring below tau.
    """
    n_q, n = scores_orc.shape
    sel_orc = oracle.select_topk(scores_orc, k)
    differ, wide, fails = 0, 0, []
    for i in range(n_q):
        g = sel_gpu[i, :k]
        if not (np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < n):
            fails.append((i, "not strictly ascending / out of range"))
            continue
        if np.array_equal(g, sel_orc[i]):
            continue
        differ += 1
        s = scores_orc[i].astype(np.float64)
        order = np.lexsort((np.arange(n), -scores_orc[i]))
        tau = s[order[k - 1]]
        band = np.abs(s - tau) <= rel * np.maximum(np.abs(s), abs(tau))
        if band.sum() > 1:
            wide += 1
        gs = set(g.tolist())
        must = set(np.nonzero((s > tau) & ~band)[0].tolist())
        never = set(np.nonzero((s < tau) & ~band)[0].tolist())
        if not must <= gs or gs & never:
            fails.append((i, "outside the near-tie band"))
    return differ, wide, fails


def bf16_stats(got: np.ndarray, want: np.ndarray):
    diff = np.abs(got.astype(np.float64) - want)
    return float(diff.max()), float(diff.mean())


BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 5e-3
F32_MAX_ABS = 1e-5
# bf16 path: the row sum behind the LSE is taken over the bf16-rounded
# probabilities that weight V (each within 2^-9 relative of the exact one), so
# the log of the sum is within 2^-9 of the exact LSE, plus fp32 rounding of the
# logits and the sum.
BF16_LSE_ABS = 2.0 ** -9 + 1e-4
# fp8 path, against exact attention over the same E4M3 inputs: the kernel
# rounds every probability to E4M3 (relative error <= 2^-4) and sums the
# rounded values; the f8 MFMA sums its 64 products at about 2^-13 relative.
# A CPU model of the probability rounding (tests/test_fp8_tolerance_model.py)
# stays within 0.6 of these on the small fp8 test workloads, whose rows see
# the fewest keys (700 to 2,000; errors shrink as rows see more keys).
FP8_MAX_ABS, FP8_MEAN_ABS, FP8_LSE_ABS = 5e-2, 4e-3, 2e-2
# Rows that see few keys (the edge workloads: 192 to 768 keys per row) average
# the probability rounding over fewer terms; the same CPU model stays within
# 0.6 of these wider bounds on them (tests/test_fp8_tolerance_model.py).
FP8_EDGE_MAX_ABS, FP8_EDGE_MEAN_ABS, FP8_EDGE_LSE_ABS = 6e-2, 5e-3, 4e-2


def default_scale(d):
    return 1.0 / math.sqrt(d)
