"""CPU oracle for tile-sparse video attention.

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library; it is
not part of the product path. Only the test suite, the package's smoke check
and the benchmark's CPU-baseline leg may import or call it. It shares no code
with the HIP path and imports nothing from it.

Everything is plain NumPy in float64 (scores are additionally rounded to
float32, because that is the precision the ranking is taken in). Each
function follows one step of the method as the pages describe it, in their
order, with the pages' notation where they have one:

  1. tile map          segment-pure prefix tiles, then 3D video tiles
  2. gather            tokens into tile-major order, pads are zero
  3. pool              mean-pool through a gate (VSA) or Avg/Max/Min TripPool
  4. score             dot products of pooled tile descriptors
  5. select            top-k video key tiles per video query tile
  6. mask              prefix keys and prefix query rows always dense
  7. attention         softmax attention over the allowed real keys

and, outside that order: the two-stream budget (8), the teacher tile map
and tile recall (9), and the fp8 e4m3 attention inputs (10).

Where the pages leave a step open, the reading taken is stated in the
function's docstring (the full list of readings is in the design notes).

Pins (what checks this oracle against something other than itself) live in
tests/test_oracle_*.py: brute-force enumeration of the map, closed forms of
pooling and attention, an O(n^2) rank definition for selection and
torch's scaled_dot_product_attention with an explicit mask in float64.
Parity unpinned against the pages themselves: they print no worked example,
only the property that keeping 100% of tiles reproduces dense attention
("BSAI-ComfyUI-VedaSparse" README, section "正确性验证 / Correctness").
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TILE = 64  # tokens per tile ("From 650 s to 72 s", section "The method": 4x4x4 = 64)


# --------------------------------------------------------------------------
# 1. Tile map
# --------------------------------------------------------------------------

@dataclass
class TileMap:
    slot_to_token: np.ndarray   # int64 [n_tiles * 64]; -1 marks a pad slot
    n_prefix_tiles: int
    n_video_tiles: int
    video_grid: tuple           # (nt, nh, nw) tiles per axis

    @property
    def n_tiles(self) -> int:
        return self.n_prefix_tiles + self.n_video_tiles

    def tile_tokens(self, tile: int) -> np.ndarray:
        """Real token indices of one tile, in slot order."""
        s = self.slot_to_token[tile * TILE:(tile + 1) * TILE]
        return s[s >= 0]

    def valid(self) -> np.ndarray:
        """bool [n_tiles, 64]: slot holds a real token."""
        return (self.slot_to_token >= 0).reshape(self.n_tiles, TILE)


def tile_map(T: int, Hv: int, Wv: int, prefix, shape) -> TileMap:
    """Token -> tile layout for one head shape.

    Prefix segments (text, reference image, reference audio, in the caller's
    sequence order) each get their own tiles so no tile mixes modalities
    ("Ref2VA VSA" node news, section "Патч внимания с двумя уровнями",
    item 1; ComfyUI-Ref2VA-VSA README, "Multimodal Dense-Exempt Prefix").
    Segment s with offset o_s and length L_s fills ceil(L_s / 64) tiles;
    slot j holds token o_s + j while j < L_s and is a pad after that.

    Video tokens follow the prefix, row-major in (t, y, x). They are grouped
    in 3D tiles of (pt, ph, pw) = ``shape`` with pt*ph*pw = 64: 4x4x4 for VSA
    ("From 650 s to 72 s", section "The method"), any per-head shape for
    Veda ("BSAI-ComfyUI-VedaSparse" README, Overview table, Head-Aware
    Tiling). Reading: each axis is padded up to a multiple of the tile edge;
    video tile (ti, hi, wi) is tile n_prefix_tiles + (ti*nh + hi)*nw + wi, and
    slot (a*ph + b)*pw + c holds position (ti*pt + a, hi*ph + b, wi*pw + c),
    or a pad when that falls outside the grid.
    """
    pt, ph, pw = (int(s) for s in shape)
    assert pt * ph * pw == TILE, "tile shape must hold 64 tokens"
    slots = []
    offset = 0
    n_prefix_tiles = 0
    for L in prefix:
        L = int(L)
        n = -(-L // TILE)
        j = np.arange(n * TILE)
        slots.append(np.where(j < L, offset + j, -1))
        offset += L
        n_prefix_tiles += n
    P = offset
    nt, nh, nw = -(-T // pt), -(-Hv // ph), -(-Wv // pw)
    ti, hi, wi, a, b, c = np.meshgrid(np.arange(nt), np.arange(nh), np.arange(nw),
                                      np.arange(pt), np.arange(ph), np.arange(pw),
                                      indexing="ij")
    t, y, x = ti * pt + a, hi * ph + b, wi * pw + c
    inside = (t < T) & (y < Hv) & (x < Wv)
    video = np.where(inside, P + (t * Hv + y) * Wv + x, -1).reshape(-1)
    slots.append(video)
    s2t = np.concatenate(slots).astype(np.int64)
    return TileMap(s2t, n_prefix_tiles, nt * nh * nw, (nt, nh, nw))


# --------------------------------------------------------------------------
# 2. Gather
# --------------------------------------------------------------------------

def gather(x: np.ndarray, tmap: TileMap) -> np.ndarray:
    """[N, d] token rows -> [n_tiles, 64, d] tile-major rows; pads are zero.

    The whole-tile row gather of the memory-bounded engine
    ("BSAI-ComfyUI-VedaSparse" README, section "六、实现说明 / Implementation").
    """
    s2t = tmap.slot_to_token
    out = np.zeros((s2t.size, x.shape[1]), dtype=x.dtype)
    real = s2t >= 0
    out[real] = x[s2t[real]]
    return out.reshape(tmap.n_tiles, TILE, x.shape[1])


# --------------------------------------------------------------------------
# 3. Pool
# --------------------------------------------------------------------------

def _tiles_part(xt: np.ndarray, tmap: TileMap, tiles=None):
    """Rows and real-slot masks of the given tiles (default: the video tiles)."""
    if tiles is None:
        tiles = np.arange(tmap.n_prefix_tiles, tmap.n_tiles)
    tiles = np.asarray(tiles, dtype=np.int64)
    return np.asarray(xt[tiles], dtype=np.float64), tmap.valid()[tiles]


def pool_mean_gate(xt: np.ndarray, tmap: TileMap, gate: np.ndarray, tiles=None) -> np.ndarray:
    """VSA tile descriptor: mean of a video tile's real rows, times the gate.

    The gating projection to_gate_compress decides which tiles a query tile
    attends to ("From 650 s to 72 s", section "The method"). Reading: the
    same per-head d x d gate multiplies the pooled Q tile and the pooled K
    tile; pad slots are left out of the mean. ``tiles`` picks other tiles
    (the reference stream of the two-stream budget). Returns float64
    [n_tiles, r].
    """
    x, v = _tiles_part(xt, tmap, tiles)
    counts = v.sum(axis=1).astype(np.float64)
    mean = (x * v[:, :, None]).sum(axis=1) / counts[:, None]
    return mean @ np.asarray(gate, dtype=np.float64)


TRIPOOL_MODES = ("triplet", "maxmin", "avg")


def pool_trippool(xt: np.ndarray, tmap: TileMap, proj: np.ndarray, tiles=None,
                  stats: str = "triplet") -> np.ndarray:
    """Veda TripPool tile descriptor: [Avg, Max, Min] of projected tokens.

    Each real token of a video tile is projected by the head's d x r matrix,
    then the channel-wise mean, maximum and minimum over the tile's real
    tokens are concatenated ("BSAI-ComfyUI-VedaSparse" README, Overview table,
    TripPool row: Avg, Max and Min statistics per tile; Implementation
    section, the TripPool descriptor). Reading: project first, pool after;
    pads are left out. ``tiles`` as for pool_mean_gate.

    ``stats`` is the README's tripool_mode parameter (parameter table:
    triplet, the default and the paper's best, or maxmin, or avg). Reading:
    maxmin keeps the [Max, Min] blocks and avg the [Avg] block, in the
    triplet's order. Returns float64 [n_tiles, 3r], [n_tiles, 2r] or
    [n_tiles, r].
    """
    if stats not in TRIPOOL_MODES:
        raise ValueError(f"unknown tripool mode {stats!r}")
    x, v = _tiles_part(xt, tmap, tiles)
    y = x @ np.asarray(proj, dtype=np.float64)            # [n_video, 64, r]
    counts = v.sum(axis=1).astype(np.float64)
    m = v[:, :, None]
    avg = np.where(m, y, 0.0).sum(axis=1) / counts[:, None]
    mx = np.where(m, y, -np.inf).max(axis=1)
    mn = np.where(m, y, np.inf).min(axis=1)
    blocks = {"triplet": [avg, mx, mn], "maxmin": [mx, mn], "avg": [avg]}[stats]
    return np.concatenate(blocks, axis=1)


# --------------------------------------------------------------------------
# 4. Score
# --------------------------------------------------------------------------

def tile_scores(qhat: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """s[i, j] = qhat_i . khat_j for video query tile i and video key tile j.

    Plain dot product of the tile descriptors, as the heuristic scorer with
    the identity (unit) projection does ("BSAI-ComfyUI-VedaSparse" README,
    scorer modes table, heuristic row). Reading: no 1/sqrt(d) and no softmax
    over tiles, since neither changes the order. Computed in float64 and
    rounded to float32, the precision the ranking uses. Prefix tiles are
    never scored: they are always kept.
    """
    s = np.asarray(qhat, dtype=np.float64) @ np.asarray(khat, dtype=np.float64).T
    return s.astype(np.float32)


# --------------------------------------------------------------------------
# 5. Select
# --------------------------------------------------------------------------

def keep_count(sparsity: float, n_video_tiles: int) -> int:
    """k = number of video key tiles kept per video query tile.

    "75% sparsity" keeps the top 25% of tiles ("From 650 s to 72 s", section
    "Where the time went"). Reading: the kept share is fixed once as integer
    basis points, keep_bp = round_half_up((1 - sparsity) * 10^4), and
    k = max(1, ceil(keep_bp * n / 10^4)) in integer arithmetic, so that
    e.g. 5% of 3780 tiles is exactly 189.
    """
    keep_bp = int(math.floor((1.0 - float(sparsity)) * 10000.0 + 0.5))
    return max(1, -(-(keep_bp * int(n_video_tiles)) // 10000))


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k key tiles per query tile, as ascending index lists.

    Each video query tile keeps its k best-scoring video key tiles
    ("Ref2VA VSA" node news, item 2: top-k pruning applies to generated-video
    key tiles only; "Veda Sparse Attention в ComfyUI", section "Что делает
    Veda": head-aware top-k forms the tile mask). Order: higher score first,
    the lower tile index first among equal scores, i.e. tile j is kept iff
    #{j' : s_j' > s_j} + #{j' < j : s_j' = s_j} < k. A stable sort (a library
    primitive) realises that order. Returns int64 [n_query, k], each row
    ascending.
    """
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[1]
    idx = np.arange(n)
    out = np.empty((s.shape[0], k), dtype=np.int64)
    for i in range(s.shape[0]):
        order = np.lexsort((idx, -s[i]))
        out[i] = np.sort(order[:k])
    return out


# --------------------------------------------------------------------------
# 6. Mask
# --------------------------------------------------------------------------

def allowed_tiles(tmap: TileMap, kv_video) -> np.ndarray:
    """bool [n_tiles, n_tiles]: query tile may attend to key tile.

    Prefix key tiles are never pruned ("Ref2VA VSA" node news, item 1) and
    prefix (conditioning) query rows stay exact, i.e. attend to everything
    ("BSAI-ComfyUI-VedaSparse" README, v3.4 highlights: conditioning rows
    always dense, sink = exact_kv_and_rows). A video query tile attends to
    all prefix tiles plus its selected video key tiles. ``kv_video`` holds,
    per video query tile, video-local key tile indices.
    """
    npf, n = tmap.n_prefix_tiles, tmap.n_tiles
    allow = np.zeros((n, n), dtype=bool)
    allow[:npf, :] = True
    allow[:, :npf] = True
    for i, row in enumerate(kv_video):
        allow[npf + i, npf + np.asarray(row, dtype=np.int64)] = True
    return allow


# --------------------------------------------------------------------------
# 7. Attention
# --------------------------------------------------------------------------

def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Rows of softmax(q k^T * scale) v over the given keys, and their LSE.

    Subtract the row maximum, exponentiate, normalise. float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = (q @ k.T) * scale
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ v) / den
    lse = (mx + np.log(den))[:, 0]
    return out, lse


def sparse_attention(q, k, v, tmap: TileMap, allow: np.ndarray, scale: float,
                     query_tiles=None):
    """Tile-skipping attention: each query tile sees only its allowed tiles.

    Each query tile attends exactly to the key tiles it keeps and skips the
    rest ("Veda Sparse Attention в ComfyUI", section "Что делает Veda";
    "BSAI-ComfyUI-VedaSparse" README, Tile-Skipping row). Pad slots are
    neither queries nor keys. The result for a query token is written at the
    token's own sequence position. Rows of tiles not in ``query_tiles`` stay
    NaN. Returns (out [N, d], lse [N]) in float64.
    """
    N, d = q.shape
    out = np.full((N, v.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    tiles = range(tmap.n_tiles) if query_tiles is None else query_tiles
    for tq in tiles:
        rows = tmap.tile_tokens(tq)
        if rows.size == 0:
            continue
        keys = np.concatenate([tmap.tile_tokens(tk)
                               for tk in np.nonzero(allow[tq])[0]])
        o, l = softmax_attention(q[rows], k[keys], v[keys], scale)
        out[rows] = o
        lse[rows] = l
    return out, lse


def dense_attention(q, k, v, scale: float):
    """Full softmax attention of every token over every token (float64)."""
    return softmax_attention(q, k, v, scale)


def effective_flops(tmap: TileMap, allow: np.ndarray, d: int) -> int:
    """4*d * sum over query tiles of (real queries) x (real allowed keys).

    QK^T and PV, two flops per multiply-add; softmax not counted.
    """
    real = tmap.valid().sum(axis=1).astype(np.int64)
    keys = allow.astype(np.int64) @ real
    return int(4 * d * int((real * keys).sum()))


# --------------------------------------------------------------------------
# 8. Two-stream budget (reference-to-video)
# --------------------------------------------------------------------------

def segment_tiles(prefix, segment: int) -> np.ndarray:
    """Global tile indices of prefix segment ``segment`` (sequence order)."""
    n = [-(-int(L) // TILE) for L in prefix]
    t0 = sum(n[:segment])
    return np.arange(t0, t0 + n[segment], dtype=np.int64)


def allowed_two_stream(tmap: TileMap, kv_video, ref_tiles, kv_ref) -> np.ndarray:
    """bool [n_tiles, n_tiles] under the two-stream budget.

    The reference-to-video predictor keeps, per query tile, a budget of
    reference tiles and a budget of video tiles, while text and audio
    conditioning stay dense ("BSAI-ComfyUI-VedaSparse" README, section
    "v3.4.2 Vendored Official Veda (Pull-and-Go)", R2VA predictor row: two
    streams of 32 tiles each). Reading: the reference stream is one prefix
    segment (the reference image), scored against the video query tiles with
    the same descriptors as the video stream and ranked by the same rule;
    every other prefix tile stays a dense key; prefix (conditioning) query
    rows stay dense, including the reference rows. ``kv_ref`` holds, per
    video query tile, indices into ``ref_tiles``.
    """
    npf, n = tmap.n_prefix_tiles, tmap.n_tiles
    ref_tiles = np.asarray(ref_tiles, dtype=np.int64)
    allow = np.zeros((n, n), dtype=bool)
    allow[:npf, :] = True
    dense_prefix = np.setdiff1d(np.arange(npf), ref_tiles)
    allow[npf:, dense_prefix] = True
    for i, (rv, rr) in enumerate(zip(kv_video, kv_ref)):
        allow[npf + i, npf + np.asarray(rv, dtype=np.int64)] = True
        allow[npf + i, ref_tiles[np.asarray(rr, dtype=np.int64)]] = True
    return allow


# --------------------------------------------------------------------------
# 9. Teacher tile map and tile recall
# --------------------------------------------------------------------------

def teacher_tile_map(q, k, tmap: TileMap, scale: float, query_tiles=None) -> np.ndarray:
    """Full attention max-pooled per (video query tile, video key tile).

    The teacher distribution at tile level comes from full attention with
    max pooling ("Veda Sparse Attention в ComfyUI", section "Что делает
    Veda": the first of the method's three stages). Reading: the attention
    probability of real query q and real key k is softmax over all real keys
    (prefix and video) of q.k * scale; the teacher value of a tile pair is the
    largest such probability over the pair's real queries and keys. Rows are
    the given video query tiles (default: all), columns all video key tiles.
    float64 [n_rows, n_video].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    npf = tmap.n_prefix_tiles
    rows = range(tmap.n_video_tiles) if query_tiles is None else query_tiles
    keys_all = np.concatenate([tmap.tile_tokens(t) for t in range(tmap.n_tiles)])
    video_keys = [tmap.tile_tokens(npf + j) for j in range(tmap.n_video_tiles)]
    out = np.zeros((len(rows), tmap.n_video_tiles))
    for r, i in enumerate(rows):
        qs = tmap.tile_tokens(npf + i)
        logits = (q[qs] @ k[keys_all].T) * scale
        mx = logits.max(axis=1, keepdims=True)
        lse = mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True))
        for j, ks in enumerate(video_keys):
            out[r, j] = np.exp((q[qs] @ k[ks].T) * scale - lse).max()
    return out


def tile_recall(selection, teacher_rows, k: int) -> float:
    """Share of the teacher's top-k tiles that a selection keeps.

    Tile recall against the max-pooled teacher is the measure the pages use
    to compare scorers ("BSAI-ComfyUI-VedaSparse" README, Overview table,
    TripPool row: tile recall of TripPool against mean pooling). Reading: per
    video query tile, |selection ∩ teacher top-k| / k with the teacher ranked
    like the scores (higher first, lower index first among ties), averaged
    over the rows given.
    """
    top = select_topk(np.asarray(teacher_rows, dtype=np.float32), k)
    sel = np.asarray(selection)
    hits = [len(set(a[:k].tolist()) & set(b.tolist())) for a, b in zip(sel, top)]
    return float(np.mean(hits)) / k


# --------------------------------------------------------------------------
# 10. Low-precision attention inputs (fp8 e4m3)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0          # largest finite OCP e4m3 value, 1.75 * 2^8


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest OCP FP8 E4M3 value, ties to even (float64 out).

    E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; normals
    2^-6 .. 448, subnormals in steps of 2^-9. The node runs its attention as
    a quantized kernel ("Veda Sparse Attention в ComfyUI", section "Узел
    ComfyUI": a Triton INT8 kernel); the MI355X analogue is the e4m3 matrix
    core format. Reading: inputs beyond +-448 are an error here (the
    quantizer scales every tile into range first).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round: value outside the finite e4m3 range")
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -6.0)                      # below 2^-6: the subnormal grid
    step = np.exp2(e - 3.0)                      # 3 mantissa bits
    r = np.round(ax / step) * step               # np.round: half to even; exact
    return np.copysign(r, x)


def tile_scale_exponent(amax: float) -> int:
    """Per-tile power-of-two scale: the least e with amax * 2^-e <= 448.

    Reading: one scale per 64-token tile of a head, a power of two so that
    scaling is exact (the OCP microscaling formats use power-of-two scales
    too); e = 0 for an all-zero tile. The scale is kept as a biased 8-bit
    exponent (the microscaling E8M0 byte), so e is clamped to >= -127: a
    tile whose largest |x| is below 448 * 2^-127 keeps e = -127.
    """
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, E = math.frexp(amax)                      # amax = m * 2^E, 0.5 <= m < 1
    e = E - 9 if m <= 0.875 else E - 8           # 448 = 0.875 * 2^9
    return max(e, -127)


def quantize_tiles_e4m3(xt: np.ndarray):
    """Tiled rows [n_tiles, 64, d] -> (dequantized values, exponents).

    Each tile is scaled by 2^-e (tile_scale_exponent of its largest |x|,
    pads are zero), rounded to e4m3, and scaled back: the value the fp8
    path computes with is e4m3_round(x * 2^-e) * 2^e exactly.
    """
    xt = np.asarray(xt, dtype=np.float64)
    exps = np.array([tile_scale_exponent(np.abs(t).max()) for t in xt], dtype=np.int64)
    sc = np.exp2(exps.astype(np.float64))[:, None, None]
    return e4m3_round(xt / sc) * sc, exps


def ungather(xt: np.ndarray, tmap: TileMap, n_tokens: int) -> np.ndarray:
    """Inverse of gather: tile rows back to token order (pads dropped)."""
    s2t = tmap.slot_to_token
    flat = np.asarray(xt).reshape(-1, np.asarray(xt).shape[-1])
    out = np.zeros((n_tokens, flat.shape[1]), dtype=flat.dtype)
    real = s2t >= 0
    out[s2t[real]] = flat[real]
    return out


def fp8_attention_inputs(q, k, v, tmap: TileMap):
    """Q, K, V as the fp8 path sees them: per-tile e4m3 values, token order.

    Attention over these with the same mask (sparse_attention) is what the
    fp8 kernel computes, up to its rounding of the probabilities.
    """
    n = np.asarray(q).shape[0]
    out = []
    for x in (q, k, v):
        xq, _ = quantize_tiles_e4m3(gather(np.asarray(x, dtype=np.float64), tmap))
        out.append(ungather(xq, tmap, n))
    return tuple(out)


# --------------------------------------------------------------------------
# The whole path for one (batch, head)
# --------------------------------------------------------------------------

def head_forward(q, k, v, grid, prefix, shape, sparsity, scorer, wq, wk=None,
                 scale=None, query_tiles=None, kv_video=None, ref_budget=None,
                 kv_ref=None, tripool_mode="triplet"):
    """Map -> gather -> pool -> score -> select -> attention for one head.

    ``scorer`` is "mean_gate" (``wq`` is the gate; ``wk`` defaults to it) or
    "trippool" (``wq``, ``wk`` are the per-head projections; ``tripool_mode``
    picks the statistics, see pool_trippool). ``kv_video``
    overrides the selection (a caller-supplied valid selection).
    ``ref_budget`` = (segment, k_ref) turns on the two-stream budget: that
    prefix segment's tiles are scored and k_ref of them kept per video query
    tile (``kv_ref`` overrides that selection). Returns a dict with every
    intermediate.
    """
    T, Hv, Wv = grid
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    tmap = tile_map(T, Hv, Wv, prefix, shape)
    qt, kt = gather(q, tmap), gather(k, tmap)
    wk = wq if wk is None else wk
    if scorer == "mean_gate":
        pool = pool_mean_gate
    else:
        def pool(xt, tm, w, tiles=None):
            return pool_trippool(xt, tm, w, tiles, stats=tripool_mode)
    qhat, khat = pool(qt, tmap, wq), pool(kt, tmap, wk)
    scores = tile_scores(qhat, khat)
    kk = keep_count(sparsity, tmap.n_video_tiles)
    sel = select_topk(scores, kk) if kv_video is None else np.asarray(kv_video)
    extra = {}
    if ref_budget is None:
        allow = allowed_tiles(tmap, sel)
    else:
        segment, k_ref = ref_budget
        ref_tiles = segment_tiles(prefix, segment)
        khat_ref = pool(kt, tmap, wk, tiles=ref_tiles)
        ref_scores = tile_scores(qhat, khat_ref)
        rsel = select_topk(ref_scores, int(k_ref)) if kv_ref is None else np.asarray(kv_ref)
        allow = allowed_two_stream(tmap, sel, ref_tiles, rsel)
        extra = {"ref_tiles": ref_tiles, "khat_ref": khat_ref, "ref_scores": ref_scores,
                 "kv_ref": rsel}
    out, lse = sparse_attention(q, k, v, tmap, allow, scale, query_tiles)
    return {"tmap": tmap, "qt": qt, "kt": kt, "qhat": qhat, "khat": khat,
            "scores": scores, "k": kk, "kv_video": sel, "allow": allow,
            "out": out, "lse": lse, **extra}
