"""Thin ctypes binding of libvsa.so (include/vsa.h), same names as the C ABI.

Only argument marshalling lives here: shapes and dtypes are checked, torch
tensors provide device memory, and the current torch stream is passed as the
hipStream_t. Every step of the computation runs in the library's kernels.
There is no fallback: if libvsa.so is missing the import of the library
raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# VSA_LIBRARY names another build of the same library (e.g. a tuning build).
LIB_PATH = os.environ.get("VSA_LIBRARY") or os.path.join(_PKG, "libvsa.so")

VSA_OK, VSA_ERR_INVALID_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_SIZE, VSA_ERR_HIP = 0, -1, -2, -3, -4
VSA_F32, VSA_BF16 = 0, 1
VSA_SCORE_MEAN_GATE, VSA_SCORE_TRIPPOOL = 0, 1
VSA_SCORE_TRIPPOOL_MAXMIN, VSA_SCORE_TRIPPOOL_AVG = 2, 3
VSA_TILE, VSA_MAX_SEGMENTS, VSA_MAX_SHAPES = 64, 8, 16
VSA_MAX_VIDEO_TILES, VSA_MAX_PROJ, VSA_MAX_TILES = 8192, 64, 16383
VSA_NOALLOC_SCRATCH_BYTES = 32 << 20     # fixed device array of vsa_tile_scores_noalloc
VSA_FUSED_MAX_TILES = 4096               # vsa_tile_select: video tiles per head
VSA_FUSED_MAX_R = 192                    # vsa_tile_select: descriptor width (doubles)

# Names declared in include/vsa.h.
EXPORTS = ("vsa_query_sizes", "vsa_pooled_bytes", "vsa_map_tiles", "vsa_tile_scores",
           "vsa_tile_scores_noalloc",
           "vsa_select_topk", "vsa_tile_select", "vsa_map_tiles_scores", "vsa_sparse_attn_fwd", "vsa_kept_stats",
           "vsa_count_flops", "vsa_ref_sizes", "vsa_ref_pooled_bytes", "vsa_ref_scores",
           "vsa_ref_select", "vsa_sparse_attn_fwd_ref", "vsa_kept_stats_ref",
           "vsa_count_flops_ref", "vsa_teacher_map", "vsa_quantize_fp8", "vsa_map_tiles_fp8",
           "vsa_sparse_attn_fwd_fp8", "vsa_device_clocks", "vsa_mfma_probe",
           "vsa_status_string", "vsa_version")


class vsa_problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("T", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("Wv", ctypes.c_int32), ("n_prefix", ctypes.c_int32),
                ("prefix_len", ctypes.c_int32 * VSA_MAX_SEGMENTS),
                ("n_shapes", ctypes.c_int32),
                ("tile_shape", ctypes.POINTER(ctypes.c_int32)),
                ("dtype", ctypes.c_int32)]


class vsa_sizes(ctypes.Structure):
    _fields_ = [("map_elems", ctypes.c_int64), ("tiled_elems", ctypes.c_int64),
                ("pooled_rows", ctypes.c_int64), ("score_elems", ctypes.c_int64),
                ("idx_elems", ctypes.c_int64), ("out_elems", ctypes.c_int64),
                ("n_prefix_tiles", ctypes.c_int32), ("max_tiles", ctypes.c_int32),
                ("max_video_tiles", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("keep_bp", ctypes.c_int32),
                ("n_tiles", ctypes.c_int32 * VSA_MAX_SHAPES),
                ("n_video_tiles", ctypes.c_int32 * VSA_MAX_SHAPES),
                ("k", ctypes.c_int32 * VSA_MAX_SHAPES)]


class vsa_ref_budget(ctypes.Structure):
    _fields_ = [("segment", ctypes.c_int32), ("k_ref", ctypes.c_int32)]


class VSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libvsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_video_map_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.POINTER(vsa_problem), ctypes.POINTER(vsa_sizes)
        R = ctypes.POINTER(vsa_ref_budget)
        vp, i32, i64, f64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_float)
        sig = {
            "vsa_query_sizes": [P, f64, S],
            "vsa_pooled_bytes": [P, i32, i32, ctypes.POINTER(i64)],
            "vsa_map_tiles": [P, vp, vp, vp, vp, vp, vp, vp, vp],
            "vsa_tile_scores": [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp],
            "vsa_tile_scores_noalloc": [P, i32, i32, vp, vp, vp, vp, vp, vp, vp],
            "vsa_select_topk": [P, vp, f64, vp, vp],
            "vsa_tile_select": [P, i32, i32, vp, vp, vp, vp, vp, f64, vp, vp, vp],
            "vsa_map_tiles_scores": [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "vsa_sparse_attn_fwd": [P, vp, vp, vp, vp, vp, f64, f32, vp, vp, vp],
            "vsa_kept_stats": [P, f64, ctypes.POINTER(i64), ctypes.POINTER(f64)],
            "vsa_count_flops": [P, f64, vp, vp, ctypes.POINTER(f64)],
            "vsa_ref_sizes": [P, R, ctypes.POINTER(i32), ctypes.POINTER(i64),
                              ctypes.POINTER(i64)],
            "vsa_ref_pooled_bytes": [P, i32, i32, R, ctypes.POINTER(i64)],
            "vsa_ref_scores": [P, i32, i32, vp, vp, vp, vp, R, vp, vp, vp, vp],
            "vsa_ref_select": [P, R, vp, vp, vp],
            "vsa_sparse_attn_fwd_ref": [P, vp, vp, vp, vp, vp, f64, R, vp, f32, vp, vp, vp],
            "vsa_kept_stats_ref": [P, f64, R, ctypes.POINTER(i64), ctypes.POINTER(f64)],
            "vsa_count_flops_ref": [P, f64, R, vp, vp, vp, ctypes.POINTER(f64)],
            "vsa_teacher_map": [P, vp, vp, vp, f32, vp, vp, vp],
            "vsa_quantize_fp8": [P, vp, vp, vp, vp, vp, vp, vp, vp],
            "vsa_map_tiles_fp8": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "vsa_sparse_attn_fwd_fp8": [P, vp, vp, vp, vp, vp, vp, f64, R, vp, f32, vp, vp, vp],
            "vsa_device_clocks": [ctypes.POINTER(i32)] * 3,
            "vsa_mfma_probe": [i32, i32, i32, vp, vp],
            "vsa_status_string": [ctypes.c_int],
            "vsa_version": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "vsa_status_string" else ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().vsa_status_string(int(status)).decode()


def vsa_version() -> int:
    return lib().vsa_version()


def _check(fn: str, status: int):
    if status != VSA_OK:
        raise VSAError(fn, status)


@dataclass
class Problem:
    """Geometry of one attention layer (mirrors vsa_problem)."""
    B: int
    H: int
    d: int
    grid: Tuple[int, int, int]
    prefix: Sequence[int]
    tile_shapes: Sequence[Tuple[int, int, int]]
    dtype: str = "bf16"         # "bf16" or "f32"
    N: Optional[int] = None     # defaults to sum(prefix) + T*Hv*Wv

    def __post_init__(self):
        self.prefix = tuple(int(x) for x in self.prefix)
        self.tile_shapes = tuple(tuple(int(v) for v in s) for s in self.tile_shapes)
        if self.N is None:
            T, Hv, Wv = self.grid
            self.N = sum(self.prefix) + T * Hv * Wv
        if len(self.prefix) > VSA_MAX_SEGMENTS or len(self.tile_shapes) > VSA_MAX_SHAPES:
            raise ValueError("too many prefix segments or tile shapes")
        flat = [v for s in self.tile_shapes for v in s]
        self._shape_arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
        st = vsa_problem()
        st.B, st.H, st.N, st.d = self.B, self.H, self.N, self.d
        st.T, st.Hv, st.Wv = self.grid
        st.n_prefix = len(self.prefix)
        for i, L in enumerate(self.prefix):
            st.prefix_len[i] = L
        st.n_shapes = len(self.tile_shapes)
        st.tile_shape = ctypes.cast(self._shape_arr, ctypes.POINTER(ctypes.c_int32))
        st.dtype = VSA_BF16 if self.dtype == "bf16" else VSA_F32
        self._struct = st

    @property
    def ref(self):
        return ctypes.byref(self._struct)


def score_mode(scorer: str, tripool_mode: str = "triplet") -> int:
    """vsa_score_mode for a scorer name ("mean_gate" or "trippool") and, for
    TripPool, the statistics kept ("triplet", "maxmin" or "avg")."""
    if scorer == "mean_gate":
        return VSA_SCORE_MEAN_GATE
    if scorer != "trippool":
        raise ValueError(f"unknown scorer {scorer!r}")
    modes = {"triplet": VSA_SCORE_TRIPPOOL, "maxmin": VSA_SCORE_TRIPPOOL_MAXMIN,
             "avg": VSA_SCORE_TRIPPOOL_AVG}
    if tripool_mode not in modes:
        raise ValueError(f"unknown tripool mode {tripool_mode!r}")
    return modes[tripool_mode]


def vsa_query_sizes(prob: Problem, sparsity: float) -> vsa_sizes:
    sz = vsa_sizes()
    _check("vsa_query_sizes", lib().vsa_query_sizes(prob.ref, float(sparsity), ctypes.byref(sz)))
    return sz


def vsa_pooled_bytes(prob: Problem, mode: int, proj_dim: int) -> int:
    b = ctypes.c_int64()
    _check("vsa_pooled_bytes", lib().vsa_pooled_bytes(prob.ref, int(mode), int(proj_dim),
                                                      ctypes.byref(b)))
    return b.value


def vsa_kept_stats(prob: Problem, sparsity: float):
    kept, frac = ctypes.c_int64(), ctypes.c_double()
    _check("vsa_kept_stats", lib().vsa_kept_stats(prob.ref, float(sparsity),
                                                  ctypes.byref(kept), ctypes.byref(frac)))
    return kept.value, frac.value


def vsa_count_flops(prob: Problem, sparsity: float, slot_to_token_host, kv_idx_host=None):
    """Effective FLOPs; the arrays are host int32 numpy arrays."""
    import numpy as np
    s2t = np.ascontiguousarray(slot_to_token_host, dtype=np.int32)
    kvp = None
    if kv_idx_host is not None:
        kv = np.ascontiguousarray(kv_idx_host, dtype=np.int32)
        kvp = kv.ctypes.data
    out = ctypes.c_double()
    _check("vsa_count_flops", lib().vsa_count_flops(prob.ref, float(sparsity), s2t.ctypes.data,
                                                    kvp, ctypes.byref(out)))
    return out.value


# ---------------------------------------------------------------- device calls

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _elem_dtype(prob: Problem):
    import torch
    return torch.bfloat16 if prob.dtype == "bf16" else torch.float32


def _need(t, numel, dtype, name):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if t.dtype != dtype or t.numel() < numel:
        raise ValueError(f"{name}: need {numel} elements of {dtype}, got "
                         f"{t.numel()} of {t.dtype}")


def vsa_map_tiles(prob: Problem, q, k, v, slot_to_token, qt, kt, vt, stream=None):
    sz = vsa_query_sizes(prob, 0.0)
    import torch
    et = _elem_dtype(prob)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(x, prob.B * prob.H * prob.N * prob.d, et, name)
    for name, x in (("qt", qt), ("kt", kt), ("vt", vt)):
        _need(x, sz.tiled_elems, et, name)
    _need(slot_to_token, sz.map_elems, torch.int32, "slot_to_token")
    _check("vsa_map_tiles", lib().vsa_map_tiles(
        prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(slot_to_token), _ptr(qt), _ptr(kt),
        _ptr(vt), _stream(stream)))


def vsa_tile_scores(prob: Problem, mode: int, proj_dim: int, qt, kt, slot_to_token, wq, wk,
                    pooled_ws, scores, stream=None):
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    _need(scores, sz.score_elems, torch.float32, "scores")
    _need(wq, 1, torch.float32, "wq")
    _need(wk, 1, torch.float32, "wk")
    if pooled_ws.numel() * pooled_ws.element_size() < vsa_pooled_bytes(prob, mode, proj_dim):
        raise ValueError("pooled_ws too small")
    _check("vsa_tile_scores", lib().vsa_tile_scores(
        prob.ref, int(mode), int(proj_dim), _ptr(qt), _ptr(kt), _ptr(slot_to_token), _ptr(wq),
        _ptr(wk), _ptr(pooled_ws), _ptr(scores), _stream(stream)))


def vsa_map_tiles_scores(prob: Problem, mode: int, proj_dim: int, q, k, v, slot_to_token, qt, kt,
                         vt, wq, wk, pooled_ws, scores, stream=None):
    """vsa_map_tiles + vsa_tile_scores in one call (mean gate: the pooling done
    in the gather pass)."""
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    et = _elem_dtype(prob)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _need(t, sz.out_elems, et, name)
    for name, t in (("qt", qt), ("kt", kt), ("vt", vt)):
        if t is not None:
            _need(t, sz.tiled_elems, et, name)
    _need(slot_to_token, sz.map_elems, torch.int32, "slot_to_token")
    _need(scores, sz.score_elems, torch.float32, "scores")
    _need(wq, 1, torch.float32, "wq")
    _need(wk, 1, torch.float32, "wk")
    if pooled_ws.numel() * pooled_ws.element_size() < vsa_pooled_bytes(prob, mode, proj_dim):
        raise ValueError("pooled_ws too small")
    _check("vsa_map_tiles_scores", lib().vsa_map_tiles_scores(
        prob.ref, int(mode), int(proj_dim), _ptr(q), _ptr(k), _ptr(v), _ptr(slot_to_token),
        _ptr(qt), _ptr(kt), _ptr(vt), _ptr(wq), _ptr(wk), _ptr(pooled_ws), _ptr(scores),
        _stream(stream)))


def vsa_tile_scores_noalloc(prob: Problem, mode: int, proj_dim: int, qt, kt, slot_to_token, wq,
                            wk, scores, stream=None):
    """vsa_tile_scores without a workspace (the library's fixed device array)."""
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    _need(scores, sz.score_elems, torch.float32, "scores")
    _need(wq, 1, torch.float32, "wq")
    _need(wk, 1, torch.float32, "wk")
    _check("vsa_tile_scores_noalloc", lib().vsa_tile_scores_noalloc(
        prob.ref, int(mode), int(proj_dim), _ptr(qt), _ptr(kt), _ptr(slot_to_token), _ptr(wq),
        _ptr(wk), _ptr(scores), _stream(stream)))


def vsa_select_topk(prob: Problem, scores, sparsity: float, kv_idx, stream=None):
    import torch
    sz = vsa_query_sizes(prob, sparsity)
    _need(scores, sz.score_elems, torch.float32, "scores")
    _need(kv_idx, sz.idx_elems, torch.int32, "kv_idx")
    _check("vsa_select_topk", lib().vsa_select_topk(
        prob.ref, _ptr(scores), float(sparsity), _ptr(kv_idx), _stream(stream)))


def fused_select_supported(prob: Problem, mode: int, proj_dim: int, sparsity: float) -> bool:
    """Whether vsa_tile_select takes this problem (host-side check, no HIP call)."""
    if sparsity == 0.0:
        return False
    sz = vsa_query_sizes(prob, sparsity)
    r = vsa_pooled_bytes(prob, mode, proj_dim) // (8 * sz.pooled_rows)
    return (sz.max_video_tiles <= VSA_FUSED_MAX_TILES and r % 32 == 0
            and r <= VSA_FUSED_MAX_R)


def vsa_tile_select(prob: Problem, mode: int, proj_dim: int, qt, kt, slot_to_token, wq, wk,
                    sparsity: float, pooled_ws, kv_idx, stream=None):
    """Pooling, scores and top-k in one call; the score matrix is never written."""
    import torch
    sz = vsa_query_sizes(prob, sparsity)
    _need(kv_idx, sz.idx_elems, torch.int32, "kv_idx")
    _need(wq, 1, torch.float32, "wq")
    _need(wk, 1, torch.float32, "wk")
    if pooled_ws.numel() * pooled_ws.element_size() < vsa_pooled_bytes(prob, mode, proj_dim):
        raise ValueError("pooled_ws too small")
    _check("vsa_tile_select", lib().vsa_tile_select(
        prob.ref, int(mode), int(proj_dim), _ptr(qt), _ptr(kt), _ptr(slot_to_token), _ptr(wq),
        _ptr(wk), float(sparsity), _ptr(pooled_ws), _ptr(kv_idx), _stream(stream)))


def vsa_sparse_attn_fwd(prob: Problem, qt, kt, vt, slot_to_token, kv_idx, sparsity: float,
                        softmax_scale: float, out, lse=None, stream=None):
    import torch
    sz = vsa_query_sizes(prob, sparsity)
    et = _elem_dtype(prob)
    for name, x in (("qt", qt), ("kt", kt), ("vt", vt)):
        _need(x, sz.tiled_elems, et, name)
    _need(out, sz.out_elems, et, "out")
    _need(lse, prob.B * prob.H * prob.N, torch.float32, "lse")
    if kv_idx is not None:
        _need(kv_idx, sz.idx_elems, torch.int32, "kv_idx")
    _check("vsa_sparse_attn_fwd", lib().vsa_sparse_attn_fwd(
        prob.ref, _ptr(qt), _ptr(kt), _ptr(vt), _ptr(slot_to_token), _ptr(kv_idx),
        float(sparsity), float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))


# ---------------------------------------------------- two-stream budget calls

def ref_budget(segment: int, k_ref: int) -> vsa_ref_budget:
    return vsa_ref_budget(int(segment), int(k_ref))


def vsa_ref_sizes(prob: Problem, budget: vsa_ref_budget):
    n, se, ie = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check("vsa_ref_sizes", lib().vsa_ref_sizes(prob.ref, ctypes.byref(budget), ctypes.byref(n),
                                                ctypes.byref(se), ctypes.byref(ie)))
    return n.value, se.value, ie.value


def vsa_ref_pooled_bytes(prob: Problem, mode: int, proj_dim: int, budget: vsa_ref_budget) -> int:
    b = ctypes.c_int64()
    _check("vsa_ref_pooled_bytes", lib().vsa_ref_pooled_bytes(
        prob.ref, int(mode), int(proj_dim), ctypes.byref(budget), ctypes.byref(b)))
    return b.value


def vsa_ref_scores(prob: Problem, mode: int, proj_dim: int, kt, slot_to_token, wq, wk,
                   budget: vsa_ref_budget, pooled_ws, ref_pooled_ws, ref_scores, stream=None):
    import torch
    _, se, _ = vsa_ref_sizes(prob, budget)
    _need(ref_scores, se, torch.float32, "ref_scores")
    _need(wq, 1, torch.float32, "wq")
    _need(wk, 1, torch.float32, "wk")
    if pooled_ws.numel() * pooled_ws.element_size() < vsa_pooled_bytes(prob, mode, proj_dim):
        raise ValueError("pooled_ws too small")
    if (ref_pooled_ws.numel() * ref_pooled_ws.element_size()
            < vsa_ref_pooled_bytes(prob, mode, proj_dim, budget)):
        raise ValueError("ref_pooled_ws too small")
    _check("vsa_ref_scores", lib().vsa_ref_scores(
        prob.ref, int(mode), int(proj_dim), _ptr(kt), _ptr(slot_to_token), _ptr(wq), _ptr(wk),
        ctypes.byref(budget), _ptr(pooled_ws), _ptr(ref_pooled_ws), _ptr(ref_scores),
        _stream(stream)))


def vsa_ref_select(prob: Problem, budget: vsa_ref_budget, ref_scores, ref_idx, stream=None):
    import torch
    _, se, ie = vsa_ref_sizes(prob, budget)
    _need(ref_scores, se, torch.float32, "ref_scores")
    _need(ref_idx, ie, torch.int32, "ref_idx")
    _check("vsa_ref_select", lib().vsa_ref_select(
        prob.ref, ctypes.byref(budget), _ptr(ref_scores), _ptr(ref_idx), _stream(stream)))


def vsa_sparse_attn_fwd_ref(prob: Problem, qt, kt, vt, slot_to_token, kv_idx, sparsity: float,
                            budget: vsa_ref_budget, ref_idx, softmax_scale: float, out,
                            lse=None, stream=None):
    import torch
    sz = vsa_query_sizes(prob, sparsity)
    _, _, ie = vsa_ref_sizes(prob, budget)
    et = _elem_dtype(prob)
    for name, x in (("qt", qt), ("kt", kt), ("vt", vt)):
        _need(x, sz.tiled_elems, et, name)
    _need(out, sz.out_elems, et, "out")
    _need(lse, prob.B * prob.H * prob.N, torch.float32, "lse")
    _need(kv_idx, sz.idx_elems, torch.int32, "kv_idx")
    _need(ref_idx, ie, torch.int32, "ref_idx")
    _check("vsa_sparse_attn_fwd_ref", lib().vsa_sparse_attn_fwd_ref(
        prob.ref, _ptr(qt), _ptr(kt), _ptr(vt), _ptr(slot_to_token), _ptr(kv_idx),
        float(sparsity), ctypes.byref(budget), _ptr(ref_idx), float(softmax_scale), _ptr(out),
        _ptr(lse), _stream(stream)))


def vsa_kept_stats_ref(prob: Problem, sparsity: float, budget: vsa_ref_budget):
    kept, frac = ctypes.c_int64(), ctypes.c_double()
    _check("vsa_kept_stats_ref", lib().vsa_kept_stats_ref(
        prob.ref, float(sparsity), ctypes.byref(budget), ctypes.byref(kept), ctypes.byref(frac)))
    return kept.value, frac.value


def vsa_count_flops_ref(prob: Problem, sparsity: float, budget: vsa_ref_budget,
                        slot_to_token_host, kv_idx_host, ref_idx_host):
    import numpy as np
    s2t = np.ascontiguousarray(slot_to_token_host, dtype=np.int32)
    kv = np.ascontiguousarray(kv_idx_host, dtype=np.int32)
    rf = np.ascontiguousarray(ref_idx_host, dtype=np.int32)
    out = ctypes.c_double()
    _check("vsa_count_flops_ref", lib().vsa_count_flops_ref(
        prob.ref, float(sparsity), ctypes.byref(budget), s2t.ctypes.data, kv.ctypes.data,
        rf.ctypes.data, ctypes.byref(out)))
    return out.value


def vsa_teacher_map(prob: Problem, qt, kt, slot_to_token, softmax_scale: float, lse_ws,
                    teacher, stream=None):
    """Teacher tile map into ``teacher`` (scores layout); lse_ws holds
    B*H*max_video_tiles*64 floats."""
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    et = _elem_dtype(prob)
    for name, x in (("qt", qt), ("kt", kt)):
        _need(x, sz.tiled_elems, et, name)
    _need(lse_ws, prob.B * prob.H * sz.max_video_tiles * VSA_TILE, torch.float32, "lse_ws")
    _need(teacher, sz.score_elems, torch.float32, "teacher")
    _check("vsa_teacher_map", lib().vsa_teacher_map(
        prob.ref, _ptr(qt), _ptr(kt), _ptr(slot_to_token), float(softmax_scale), _ptr(lse_ws),
        _ptr(teacher), _stream(stream)))


# ------------------------------------------------------------- fp8 variant

def fp8_scale_bytes(prob: Problem) -> int:
    """Bytes of the per-tile scale array: 4 per (batch, head, tile)."""
    sz = vsa_query_sizes(prob, 0.0)
    return prob.B * prob.H * sz.max_tiles * 4


def vsa_quantize_fp8(prob: Problem, qt, kt, vt, q8, k8, v8, scales, stream=None):
    """E4M3 copies of the bf16 tiles (uint8 tensors of tiled_elems) and their
    per-tile scale bytes (uint8, fp8_scale_bytes)."""
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    et = _elem_dtype(prob)
    for name, x in (("qt", qt), ("kt", kt), ("vt", vt)):
        _need(x, sz.tiled_elems, et, name)
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        _need(x, sz.tiled_elems, torch.uint8, name)
    _need(scales, fp8_scale_bytes(prob), torch.uint8, "scales")
    _check("vsa_quantize_fp8", lib().vsa_quantize_fp8(
        prob.ref, _ptr(qt), _ptr(kt), _ptr(vt), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(scales),
        _stream(stream)))


def vsa_map_tiles_fp8(prob: Problem, q, k, v, slot_to_token, qt, kt, vt, q8, k8, v8, scales,
                      stream=None):
    """vsa_map_tiles plus the E4M3 copies and scale bytes, in one pass."""
    import torch
    sz = vsa_query_sizes(prob, 0.0)
    et = _elem_dtype(prob)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(x, sz.out_elems, et, name)
    for name, x in (("qt", qt), ("kt", kt), ("vt", vt)):
        _need(x, sz.tiled_elems, et, name)
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        _need(x, sz.tiled_elems, torch.uint8, name)
    _need(slot_to_token, sz.map_elems, torch.int32, "slot_to_token")
    _need(scales, fp8_scale_bytes(prob), torch.uint8, "scales")
    _check("vsa_map_tiles_fp8", lib().vsa_map_tiles_fp8(
        prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(slot_to_token), _ptr(qt), _ptr(kt), _ptr(vt),
        _ptr(q8), _ptr(k8), _ptr(v8), _ptr(scales), _stream(stream)))


def vsa_sparse_attn_fwd_fp8(prob: Problem, q8, k8, v8, scales, slot_to_token, kv_idx,
                            sparsity: float, softmax_scale: float, out, lse=None,
                            budget: Optional[vsa_ref_budget] = None, ref_idx=None,
                            stream=None):
    import torch
    sz = vsa_query_sizes(prob, sparsity)
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        _need(x, sz.tiled_elems, torch.uint8, name)
    _need(scales, fp8_scale_bytes(prob), torch.uint8, "scales")
    _need(out, sz.out_elems, torch.bfloat16, "out")
    _need(lse, prob.B * prob.H * prob.N, torch.float32, "lse")
    if kv_idx is not None:
        _need(kv_idx, sz.idx_elems, torch.int32, "kv_idx")
    if budget is not None:
        _, _, ie = vsa_ref_sizes(prob, budget)
        _need(ref_idx, ie, torch.int32, "ref_idx")
    _check("vsa_sparse_attn_fwd_fp8", lib().vsa_sparse_attn_fwd_fp8(
        prob.ref, _ptr(q8), _ptr(k8), _ptr(v8), _ptr(scales), _ptr(slot_to_token), _ptr(kv_idx),
        float(sparsity), None if budget is None else ctypes.byref(budget), _ptr(ref_idx),
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))


# ------------------------------------------------------- measurement aids

# flop per MFMA of each probe kind: bf16, then fp8 (kinds 1-4), and MFMAs per
# workgroup and trip
MFMA_PROBE_FLOPS = (32 * 32 * 16 * 2,) + (32 * 32 * 64 * 2,) * 4
MFMA_PROBE_PER_TRIP = (16, 16, 32, 32, 16)


def vsa_device_clocks():
    """(compute units, engine clock in kHz, real-time counter rate in kHz) of
    the current device, as the runtime reports them."""
    cu, clk, wall = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check("vsa_device_clocks", lib().vsa_device_clocks(ctypes.byref(cu), ctypes.byref(clk),
                                                        ctypes.byref(wall)))
    return cu.value, clk.value, wall.value


def vsa_mfma_probe(kind: int, iters: int, n_workgroups: int, ticks=None, stream=None) -> int:
    """Enqueues the matrix-core load (kind 0 bf16, 1 fp8; in 8-wave
    workgroups: 2 fp8, 3 fp8 with exponentials in the same waves, 4 fp8
    beside waves of exponentials); ticks is an int64 device tensor of
    4 * n_workgroups counters or None. Returns the flops the launch
    performs."""
    import torch
    _need(ticks, 4 * n_workgroups, torch.int64, "ticks")
    _check("vsa_mfma_probe", lib().vsa_mfma_probe(int(kind), int(iters), int(n_workgroups),
                                                  _ptr(ticks), _stream(stream)))
    return n_workgroups * MFMA_PROBE_PER_TRIP[kind] * iters * MFMA_PROBE_FLOPS[kind]


# ---------------------------------------------------------- whole-layer helper

class Layer:
    """Device buffers for one layer and the four calls in order.

    Allocates with torch on the current device: slot_to_token, tiled Q/K/V,
    the pooling workspace, scores, kv_idx, out and lse. ``fp8=True`` adds the
    E4M3 tile copies and runs attention on them (bf16 problems only).
    """

    def __init__(self, prob: Problem, sparsity: float, mode: int, proj_dim: int,
                 device="cuda", with_lse: bool = True, ref: Optional[Tuple[int, int]] = None,
                 fp8: bool = False, fused: bool = False):
        import torch
        self.prob, self.sparsity, self.mode, self.proj_dim = prob, sparsity, mode, proj_dim
        # fused=True: forward() scores and selects in one call (vsa_tile_select),
        # which needs no score matrix but is slower than the two calls.
        if fused and not fused_select_supported(prob, mode, proj_dim, sparsity):
            raise ValueError("vsa_tile_select does not take this problem")
        self.fused = bool(fused)
        # Mean gate: forward() gathers and pools in one pass (vsa_map_tiles_scores),
        # which writes exactly what vsa_map_tiles + vsa_tile_scores write.
        self.gather_pool = (mode == VSA_SCORE_MEAN_GATE and not fp8 and sparsity != 0.0
                            and not self.fused)
        self.sizes = sz = vsa_query_sizes(prob, sparsity)
        et = _elem_dtype(prob)
        dev = torch.device(device)
        self.slot_to_token = torch.empty(sz.map_elems, dtype=torch.int32, device=dev)
        self.qt, self.kt, self.vt = (torch.empty(sz.tiled_elems, dtype=et, device=dev)
                                     for _ in range(3))
        nbytes = vsa_pooled_bytes(prob, mode, proj_dim)
        self.pooled = torch.empty((nbytes + 7) // 8, dtype=torch.float64, device=dev)
        self.scores = torch.empty(sz.score_elems, dtype=torch.float32, device=dev)
        self.kv_idx = torch.empty(max(1, sz.idx_elems), dtype=torch.int32, device=dev)
        self.out = torch.empty((prob.B, prob.H, prob.N, prob.d), dtype=et, device=dev)
        self.lse = (torch.empty((prob.B, prob.H, prob.N), dtype=torch.float32, device=dev)
                    if with_lse else None)
        # Two-stream budget (segment, k_ref): buffers of the reference stream.
        self.budget = None if ref is None else ref_budget(*ref)
        if self.budget is not None:
            if sparsity == 0.0:
                raise ValueError("the two-stream budget needs sparsity > 0")
            _, se, ie = vsa_ref_sizes(prob, self.budget)
            rb = vsa_ref_pooled_bytes(prob, mode, proj_dim, self.budget)
            self.ref_pooled = torch.empty((rb + 7) // 8, dtype=torch.float64, device=dev)
            self.ref_scores = torch.empty(se, dtype=torch.float32, device=dev)
            self.ref_idx = torch.empty(ie, dtype=torch.int32, device=dev)
        self.fp8 = fp8
        if fp8:
            if prob.dtype != "bf16":
                raise ValueError("the fp8 variant takes bf16 problems")
            self.q8, self.k8, self.v8 = (torch.empty(sz.tiled_elems, dtype=torch.uint8,
                                                     device=dev) for _ in range(3))
            self.fp8_scales = torch.empty(fp8_scale_bytes(prob), dtype=torch.uint8, device=dev)

    def map_tiles(self, q, k, v, stream=None):
        vsa_map_tiles(self.prob, q, k, v, self.slot_to_token, self.qt, self.kt, self.vt, stream)

    def map_tiles_fp8(self, q, k, v, stream=None):
        vsa_map_tiles_fp8(self.prob, q, k, v, self.slot_to_token, self.qt, self.kt, self.vt,
                          self.q8, self.k8, self.v8, self.fp8_scales, stream)

    def quantize(self, stream=None):
        vsa_quantize_fp8(self.prob, self.qt, self.kt, self.vt, self.q8, self.k8, self.v8,
                         self.fp8_scales, stream)

    def map_tiles_scores(self, q, k, v, wq, wk, stream=None):
        """map_tiles + tile_scores with the pooling done in the gather pass."""
        vsa_map_tiles_scores(self.prob, self.mode, self.proj_dim, q, k, v, self.slot_to_token,
                             self.qt, self.kt, self.vt, wq, wk, self.pooled, self.scores, stream)
        if self.budget is not None:
            vsa_ref_scores(self.prob, self.mode, self.proj_dim, self.kt, self.slot_to_token, wq,
                           wk, self.budget, self.pooled, self.ref_pooled, self.ref_scores,
                           stream)

    def tile_scores(self, wq, wk, stream=None):
        vsa_tile_scores(self.prob, self.mode, self.proj_dim, self.qt, self.kt,
                        self.slot_to_token, wq, wk, self.pooled, self.scores, stream)
        if self.budget is not None:
            vsa_ref_scores(self.prob, self.mode, self.proj_dim, self.kt, self.slot_to_token, wq,
                           wk, self.budget, self.pooled, self.ref_pooled, self.ref_scores,
                           stream)

    def select(self, stream=None):
        vsa_select_topk(self.prob, self.scores, self.sparsity, self.kv_idx, stream)
        if self.budget is not None:
            vsa_ref_select(self.prob, self.budget, self.ref_scores, self.ref_idx, stream)

    def score_select(self, wq, wk, stream=None):
        """Scores and top-k in one call (vsa_tile_select); the score matrix
        is left unwritten. The two-stream budget's reference scores and
        selection run as separate calls."""
        vsa_tile_select(self.prob, self.mode, self.proj_dim, self.qt, self.kt,
                        self.slot_to_token, wq, wk, self.sparsity, self.pooled, self.kv_idx,
                        stream)
        if self.budget is not None:
            vsa_ref_scores(self.prob, self.mode, self.proj_dim, self.kt, self.slot_to_token, wq,
                           wk, self.budget, self.pooled, self.ref_pooled, self.ref_scores,
                           stream)
            vsa_ref_select(self.prob, self.budget, self.ref_scores, self.ref_idx, stream)

    def attend(self, softmax_scale: float = 0.0, stream=None, kv_idx=None, ref_idx=None):
        kv = self.kv_idx if kv_idx is None else kv_idx
        if self.fp8:
            rf = None
            if self.budget is not None:
                rf = self.ref_idx if ref_idx is None else ref_idx
            vsa_sparse_attn_fwd_fp8(self.prob, self.q8, self.k8, self.v8, self.fp8_scales,
                                    self.slot_to_token, None if self.sparsity == 0.0 else kv,
                                    self.sparsity, softmax_scale, self.out, self.lse,
                                    self.budget, rf, stream)
            return
        if self.budget is not None:
            rf = self.ref_idx if ref_idx is None else ref_idx
            vsa_sparse_attn_fwd_ref(self.prob, self.qt, self.kt, self.vt, self.slot_to_token, kv,
                                    self.sparsity, self.budget, rf, softmax_scale, self.out,
                                    self.lse, stream)
            return
        vsa_sparse_attn_fwd(self.prob, self.qt, self.kt, self.vt, self.slot_to_token,
                            None if self.sparsity == 0.0 else kv, self.sparsity,
                            softmax_scale, self.out, self.lse, stream)

    def forward(self, q, k, v, wq, wk, softmax_scale: float = 0.0, stream=None):
        """One whole layer: map+gather, scores, top-k, attention (fp8: the
        gather also writes the E4M3 tiles). Gather and pooling are one call
        when self.gather_pool; scores and top-k are one call
        (vsa_tile_select) when self.fused."""
        if self.fp8:
            self.map_tiles_fp8(q, k, v, stream)
        elif self.gather_pool:
            self.map_tiles_scores(q, k, v, wq, wk, stream)
        else:
            self.map_tiles(q, k, v, stream)
        if self.sparsity != 0.0:
            if self.fused:
                self.score_select(wq, wk, stream)
            else:
                if not self.gather_pool:
                    self.tile_scores(wq, wk, stream)
                self.select(stream)
        self.attend(softmax_scale, stream)
        return self.out


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
