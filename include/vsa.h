/*
 * vsa.h - tile-sparse video attention on AMD Instinct MI355X (gfx950).
 *
 * The method (one attention layer of a video diffusion transformer):
 *   1. tile map      prefix segments (text, reference image, reference audio)
 *                    go into segment-pure 64-token tiles; video tokens go
 *                    into 3D tiles of (pt, ph, pw), pt*ph*pw = 64.
 *   2. tile scores   each (video query tile, video key tile) pair gets a
 *                    coarse score from pooled Q/K tiles.
 *   3. top-k         each video query tile keeps its k best video key tiles.
 *   4. attention     flash-style softmax attention that visits only the
 *                    prefix tiles and the kept video tiles; prefix query rows
 *                    attend to everything.
 * Sources: "Ref2VA VSA: нода разреженного внимания для H3 reference-to-video"
 * (section "Патч внимания с двумя уровнями"); "Veda Sparse Attention в
 * ComfyUI: ускорение MiniMax H3" (section "Что делает Veda");
 * "BSAI-ComfyUI-VedaSparse" README (Overview table; Implementation);
 * "From 650 s to 72 s: reference-to-video on a single RTX 4090" (section
 * "The method").
 *
 * Conventions for every entry point
 *   - Host-callable, thread-safe, no global state.
 *   - Device pointers are owned by the caller. The library never allocates,
 *     frees or keeps a pointer after it returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). All device work
 *     is enqueued on it; no entry point synchronises.
 *   - Return VSA_OK (0) or a negative vsa_status. Every argument error is
 *     found on the host before anything is launched; nothing falls back to a
 *     slower path silently (the caller decides about a dense fallback).
 *     VSA_ERR_HIP reports a failed launch; faults inside a kernel surface at
 *     the caller's next synchronisation.
 *
 * Sequence layout: Q, K, V and O are [B][H][N][d], d contiguous, with
 * N = sum(prefix_len) + T*Hv*Wv: the prefix segments in caller order, then
 * video tokens row-major in (t, y, x).
 */
#ifndef VSA_H
#define VSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSA_API __attribute__((visibility("default")))

#define VSA_VERSION 100             /* 1.0.0 */
#define VSA_TILE 64                 /* tokens per tile */
#define VSA_MAX_SEGMENTS 8          /* prefix segments */
#define VSA_MAX_SHAPES 16           /* distinct per-head tile shapes */
#define VSA_MAX_VIDEO_TILES 8192    /* video tiles per head (top-k row length) */
#define VSA_MAX_TILES 16383         /* prefix + video tiles per head: keeps every byte
                                       offset inside one head's tiled copy below 2^31 and
                                       every 32-key unit index below 2^15 */
#define VSA_MAX_PROJ 64             /* TripPool projection width */

typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = -1,   /* null pointer, bad geometry, N mismatch,
                                 tile product != 64, sparsity out of range */
  VSA_ERR_UNSUPPORTED = -2,   /* d or dtype the kernels do not implement */
  VSA_ERR_SIZE = -3,          /* a count exceeds a documented limit */
  VSA_ERR_HIP = -4            /* a HIP call or kernel launch failed */
} vsa_status;

typedef enum vsa_dtype { VSA_F32 = 0, VSA_BF16 = 1 } vsa_dtype;

typedef enum vsa_score_mode {
  VSA_SCORE_MEAN_GATE = 0,    /* VSA: mean-pool, then the per-head gate */
  VSA_SCORE_TRIPPOOL = 1,     /* Veda: project tokens, then Avg|Max|Min */
  VSA_SCORE_TRIPPOOL_MAXMIN = 2,  /* Veda tripool_mode maxmin: Max|Min */
  VSA_SCORE_TRIPPOOL_AVG = 3      /* Veda tripool_mode avg: Avg */
} vsa_score_mode;

/* One attention layer's geometry. */
typedef struct vsa_problem {
  int32_t B, H, N, d;         /* batch, heads, tokens, head dim (64 or 128) */
  int32_t T, Hv, Wv;          /* latent video grid */
  int32_t n_prefix;           /* 0..VSA_MAX_SEGMENTS prefix segments */
  int32_t prefix_len[VSA_MAX_SEGMENTS];  /* lengths in sequence order; each
                                 segment fills its own ceil(len/64) tiles,
                                 a zero length gives no tile */
  int32_t n_shapes;           /* 1..VSA_MAX_SHAPES */
  const int32_t *tile_shape;  /* HOST pointer, [n_shapes][3] = (pt, ph, pw),
                                 pt*ph*pw == 64; head h uses shape
                                 h % n_shapes; each grid axis is padded up to a
                                 multiple of the tile edge */
  int32_t dtype;              /* vsa_dtype of Q, K, V, the tiled copies and O */
} vsa_problem;

/* Buffer sizes and per-shape counts, from vsa_query_sizes. */
typedef struct vsa_sizes {
  int64_t map_elems;          /* int32 elements of slot_to_token */
  int64_t tiled_elems;        /* dtype elements of each of qt, kt, vt */
  int64_t pooled_rows;        /* rows of the pooling workspace (see
                                 vsa_pooled_bytes) */
  int64_t score_elems;        /* float elements of scores */
  int64_t idx_elems;          /* int32 elements of kv_idx */
  int64_t out_elems;          /* dtype elements of out: B*H*N*d */
  int32_t n_prefix_tiles;     /* same for every shape */
  int32_t max_tiles;          /* max over shapes of n_tiles */
  int32_t max_video_tiles;    /* max over shapes of n_video_tiles */
  int32_t k_max;              /* max over shapes of k */
  int32_t keep_bp;            /* kept share of video key tiles, basis points */
  int32_t n_tiles[VSA_MAX_SHAPES];        /* prefix + video tiles */
  int32_t n_video_tiles[VSA_MAX_SHAPES];
  int32_t k[VSA_MAX_SHAPES];  /* video key tiles kept per video query tile */
} vsa_sizes;

/*
 * vsa_query_sizes - validate a problem and report buffer sizes. Host only,
 * makes no HIP call.
 *
 * sparsity in [0, 1) is turned into keep_bp = round((1 - sparsity) * 10^4)
 * once; per shape k = max(1, ceil(keep_bp * n_video_tiles / 10^4)) in
 * integer arithmetic ("75% sparsity" keeps the top 25% of video key tiles:
 * "From 650 s to 72 s", section "Where the time went"). sparsity == 0 is
 * the dense path (k = n_video_tiles).
 */
VSA_API int vsa_query_sizes(const vsa_problem *prob, double sparsity,
                            vsa_sizes *sizes);

/*
 * vsa_pooled_bytes - bytes of the pooling workspace of vsa_tile_scores:
 * pooled_rows * r * 8, r = d (mean gate) or 3 * proj_dim (TripPool).
 */
VSA_API int vsa_pooled_bytes(const vsa_problem *prob, int32_t mode,
                             int32_t proj_dim, int64_t *bytes);

/*
 * Tiled layouts (per tile: 64 slots x d channels, dtype elements).
 *
 * qt, kt ("row operand" layout): element (slot s, channel c) at
 *   ((s/32)*(d/16) + c/16)*512 + (((c%16)/8)*32 + s%32)*8 + c%8
 * vt ("column operand" layout): element (s, c) at
 *   ((c/32)*4 + s/16)*512 + (((s%8)/4)*32 + c%32)*8 + ((s%16)/8)*4 + s%4
 * Both are permutations of the tile's 64*d elements; pad slots hold zero.
 * Tile t of head (b, h) starts at element ((b*H + h)*max_tiles + t)*64*d.
 * Tiles beyond the head's own n_tiles are not written.
 *
 * slot_to_token: int32 [n_shapes][max_tiles][64]; the token index held by a
 * slot, -1 for a pad. Prefix segment s (offset o_s, length L_s) fills
 * ceil(L_s/64) tiles, slot j -> o_s + j while j < L_s. Video tile
 * (ti, hi, wi) is tile n_prefix_tiles + (ti*nh + hi)*nw + wi, slot
 * (a*ph + b)*pw + c -> token P + (t*Hv + y)*Wv + x with
 * (t, y, x) = (ti*pt + a, hi*ph + b, wi*pw + c), or -1 outside the grid.
 * Entries of tiles beyond a shape's n_tiles are -1.
 */

/*
 * vsa_map_tiles - step 1: build slot_to_token and gather Q, K, V into the
 * tiled layouts (segment-pure prefix tiles: "Ref2VA VSA" node news, section
 * "Патч внимания с двумя уровнями", item 1; whole-tile row gather:
 * "BSAI-ComfyUI-VedaSparse" README, Implementation section).
 *
 * q, k, v: [B][H][N][d] dtype, device. Any of the three may be NULL together
 * with its tiled output (that tensor is skipped). slot_to_token (device,
 * map_elems) is always written. qt, kt, vt: device, tiled_elems each.
 */
VSA_API int vsa_map_tiles(const vsa_problem *prob, const void *q,
                          const void *k, const void *v, int32_t *slot_to_token,
                          void *qt, void *kt, void *vt, void *stream);

/*
 * vsa_tile_scores - step 2: pooled tile descriptors and their dot products.
 *
 * mode VSA_SCORE_MEAN_GATE (VSA): desc = mean of a video tile's real rows
 *   times the head's gate (to_gate_compress: "From 650 s to 72 s", section
 *   "The method"). wq: float [H][d][d] gate applied to pooled Q; wk: gate for
 *   pooled K, or NULL to use wq for both. proj_dim must equal d.
 * mode VSA_SCORE_TRIPPOOL (Veda): each real token of a video tile is
 *   projected by the head's d x proj_dim matrix, then [Avg | Max | Min] over
 *   the tile's real tokens (TripPool: "BSAI-ComfyUI-VedaSparse" README,
 *   Overview table). wq, wk: float [H][d][proj_dim]; proj_dim a power of two
 *   in 8..VSA_MAX_PROJ.
 * modes VSA_SCORE_TRIPPOOL_MAXMIN / _AVG: the same projection, keeping only
 *   the [Max | Min] or the [Avg] blocks (the README's tripool_mode parameter,
 *   parameter table: triplet, maxmin, avg). Descriptor width is 3, 2 or 1
 *   times proj_dim.
 * Pads never enter a descriptor. Descriptors are accumulated in double.
 *
 * scores: float [B][H][max_video_tiles][max_video_tiles], row = video query
 *   tile i, column = video key tile j (video-local indices), the double dot
 *   product of the two descriptors rounded once to float. Only the head's
 *   n_video_tiles x n_video_tiles block is written. Prefix tiles are never
 *   scored.
 * pooled_ws: device workspace of vsa_pooled_bytes bytes (holds the double
 *   descriptors, Q rows first, then K rows).
 * qt, kt, slot_to_token: as written by vsa_map_tiles.
 */
VSA_API int vsa_tile_scores(const vsa_problem *prob, int32_t mode,
                            int32_t proj_dim, const void *qt, const void *kt,
                            const int32_t *slot_to_token, const float *wq,
                            const float *wk, void *pooled_ws, float *scores,
                            void *stream);

/*
 * vsa_map_tiles_scores - vsa_map_tiles followed by vsa_tile_scores in one call;
 * for the mean gate the pooling is done in the gather pass, so the tiled Q and
 * K are not read back (the pages' engine gathers whole tiles in one pass: "BSAI-ComfyUI-VedaSparse"
 * README, Implementation section). Mean gate: the gather takes each video
 * tile's channel means, then the gate product follows. TripPool modes: the
 * gather, then the pooling kernel, as the two calls run them (the projection
 * needs every token's row, which the pooling reads once). Writes exactly what
 * the two calls write: slot_to_token, qt, kt, vt, the workspace's
 * descriptors and the scores, bit for bit.
 *
 * Arguments as the two calls: mode and proj_dim as vsa_tile_scores; q, k
 * (and v, or v = vt = NULL) device inputs; wq, wk as vsa_tile_scores
 * (mean gate: wk may be NULL for wq); pooled_ws of
 * vsa_pooled_bytes(prob, mode, proj_dim) bytes.
 */
VSA_API int vsa_map_tiles_scores(const vsa_problem *prob, int32_t mode,
                                 int32_t proj_dim, const void *q, const void *k,
                                 const void *v, int32_t *slot_to_token, void *qt,
                                 void *kt, void *vt, const float *wq,
                                 const float *wk, void *pooled_ws, float *scores,
                                 void *stream);

/*
 * vsa_tile_scores_noalloc - vsa_tile_scores for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It takes no workspace: the double descriptors go to
 * a fixed array of VSA_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends, and the (batch, head) pairs are
 * pooled and scored in chunks that fit it. Same arguments, rules and results
 * as vsa_tile_scores; no hipMalloc, hipFree or allocating call is made.
 *
 * Returns VSA_ERR_SIZE when the Q and K descriptors of one (batch, head),
 * 2 * max_video_tiles * width * 8 bytes, exceed the array (not possible within
 * VSA_MAX_VIDEO_TILES and VSA_MAX_PROJ). Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialized by the caller. Calls on one stream are ordered.
 */
#define VSA_NOALLOC_SCRATCH_BYTES (32ll << 20)
VSA_API int vsa_tile_scores_noalloc(const vsa_problem *prob, int32_t mode,
                                    int32_t proj_dim, const void *qt, const void *kt,
                                    const int32_t *slot_to_token, const float *wq,
                                    const float *wk, float *scores, void *stream);

/*
 * vsa_select_topk - step 3: per (b, h, video query tile i), keep the k best
 * video key tiles: higher score first, lower tile index first among equal
 * scores (-0.0 equals +0.0); tile j is kept iff
 * #{j' : s_j' > s_j} + #{j' < j : s_j' = s_j} < k. Top-k pruning applies to
 * video key tiles only ("Ref2VA VSA" node news, item 2).
 *
 * kv_idx: int32 [B][H][max_video_tiles][k_max]; row i holds the k kept
 * video-local tile indices in ascending order, then -1 up to k_max.
 * Scores must be finite.
 */
VSA_API int vsa_select_topk(const vsa_problem *prob, const float *scores,
                            double sparsity, int32_t *kv_idx, void *stream);

/*
 * vsa_tile_select - steps 2 and 3 in one call: the pooled descriptors of
 * vsa_tile_scores, then the top-k of vsa_select_topk, without writing the
 * score matrix (the pages' engine keeps its intermediates bounded by working
 * in chunks: "BSAI-ComfyUI-VedaSparse" README, Implementation section). Each
 * score is the same double dot product, accumulated in the same order and
 * rounded once to float, so kv_idx equals that of vsa_tile_scores followed
 * by vsa_select_topk.
 *
 * Arguments as vsa_tile_scores (pooled_ws: device, vsa_pooled_bytes bytes,
 * overwritten) plus sparsity (> 0) and kv_idx (device) of vsa_select_topk.
 * Needs max_video_tiles <= VSA_FUSED_MAX_TILES and a descriptor width that is
 * a multiple of 32 and at most VSA_FUSED_MAX_R: the mean gate with d = 64 or
 * 128; TripPool with proj_dim 32 or 64 (any mode) or 16 (maxmin). Otherwise
 * returns VSA_ERR_UNSUPPORTED before any launch; the two separate calls cover
 * every size.
 */
#define VSA_FUSED_MAX_TILES 4096
#define VSA_FUSED_MAX_R 192
VSA_API int vsa_tile_select(const vsa_problem *prob, int32_t mode,
                            int32_t proj_dim, const void *qt, const void *kt,
                            const int32_t *slot_to_token, const float *wq,
                            const float *wk, double sparsity, void *pooled_ws,
                            int32_t *kv_idx, void *stream);

/*
 * vsa_sparse_attn_fwd - step 4: for every real query token t,
 *   O_t = softmax_u(q_t . k_u * scale) V_u over its allowed real keys u.
 * A video query tile is allowed every prefix tile and its kv_idx video
 * tiles (tile skipping: "Veda Sparse Attention в ComfyUI", section "Что
 * делает Veda"); a prefix query tile is allowed every tile (conditioning rows
 * stay exact: "BSAI-ComfyUI-VedaSparse" README, v3.4 highlights). Pad slots
 * are neither queries nor keys.
 *
 * qt, kt, vt, slot_to_token: from vsa_map_tiles. kv_idx: from
 * vsa_select_topk with the same sparsity; may be NULL when sparsity == 0
 * (dense: every tile allowed). softmax_scale <= 0 selects 1/sqrt(d).
 * out: [B][H][N][d] dtype, each token's row written at its own position.
 * lse: float [B][H][N] natural-log sum of exp of the scaled logits, or NULL.
 * VSA_BF16: bf16 inputs, fp32 accumulation and softmax, bf16 output.
 * VSA_F32: fp32 throughout.
 */
VSA_API int vsa_sparse_attn_fwd(const vsa_problem *prob, const void *qt,
                                const void *kt, const void *vt,
                                const int32_t *slot_to_token,
                                const int32_t *kv_idx, double sparsity,
                                float softmax_scale, void *out, float *lse,
                                void *stream);

/*
 * vsa_kept_stats - host only: tile pairs the attention visits and their
 * share of full attention's tile pairs (the "attention computed: x% of full
 * attention" report of "Veda Sparse Attention в ComfyUI", section "Узел
 * ComfyUI").
 */
VSA_API int vsa_kept_stats(const vsa_problem *prob, double sparsity,
                           int64_t *kept_tile_pairs, double *frac_of_full);

/*
 * vsa_count_flops - host only: effective FLOPs of vsa_sparse_attn_fwd,
 * 4*d * sum over real query tokens of their allowed real keys (QK^T and PV,
 * two flops per multiply-add; softmax not counted).
 * slot_to_token_host, kv_idx_host: HOST copies of the device arrays
 * (kv_idx_host may be NULL when sparsity == 0).
 */
VSA_API int vsa_count_flops(const vsa_problem *prob, double sparsity,
                            const int32_t *slot_to_token_host,
                            const int32_t *kv_idx_host, double *flops);

/*
 * Two-stream budget (reference-to-video). One prefix segment, the reference
 * image, becomes a second sparse stream: its tiles are pooled and scored
 * against the video query tiles the same way as the video key tiles, and
 * each video query tile keeps its k_ref best of them (higher score first,
 * lower tile index first among equal scores). The other prefix segments
 * stay dense keys and every prefix query row stays dense
 * ("BSAI-ComfyUI-VedaSparse" README, section "v3.4.2 Vendored Official
 * Veda (Pull-and-Go)", R2VA predictor row: 32 reference tiles and 32 video
 * tiles per query, text and audio conditioning dense).
 */
typedef struct vsa_ref_budget {
  int32_t segment;            /* index into prefix_len of the reference segment */
  int32_t k_ref;              /* reference tiles kept, 1 .. that segment's tiles */
} vsa_ref_budget;

/*
 * vsa_ref_sizes - host only: tiles of the reference segment, and the
 * elements of ref_scores ([B][H][max_video_tiles][n_ref] float) and of
 * ref_idx ([B][H][max_video_tiles][k_ref] int32).
 */
VSA_API int vsa_ref_sizes(const vsa_problem *prob, const vsa_ref_budget *budget,
                          int32_t *n_ref_tiles, int64_t *ref_score_elems,
                          int64_t *ref_idx_elems);

/* vsa_ref_pooled_bytes - host only: bytes of ref_pooled_ws (double
 * [B][H][n_ref][r], r as for vsa_pooled_bytes). */
VSA_API int vsa_ref_pooled_bytes(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                                 const vsa_ref_budget *budget, int64_t *bytes);

/*
 * vsa_ref_scores - the reference stream's scores. Pools the reference tiles
 * of kt (wk for TripPool; the gate wk, or wq when wk is NULL, for the mean
 * gate) into ref_pooled_ws, then ref_scores[b][h][i][j] = the double dot
 * product of video query tile i's descriptor and reference tile j's,
 * rounded once to float. pooled_ws must hold the query descriptors written
 * by vsa_tile_scores with the same mode and proj_dim (it is only read).
 */
VSA_API int vsa_ref_scores(const vsa_problem *prob, int32_t mode, int32_t proj_dim,
                           const void *kt, const int32_t *slot_to_token, const float *wq,
                           const float *wk, const vsa_ref_budget *budget,
                           const void *pooled_ws, void *ref_pooled_ws, float *ref_scores,
                           void *stream);

/*
 * vsa_ref_select - per video query tile, the k_ref best reference tiles:
 * ref_idx[b][h][i][0..k_ref) ascending indices into the reference segment's
 * tiles (0 = its first tile). Same ranking rule as vsa_select_topk.
 */
VSA_API int vsa_ref_select(const vsa_problem *prob, const vsa_ref_budget *budget,
                           const float *ref_scores, int32_t *ref_idx, void *stream);

/*
 * vsa_sparse_attn_fwd_ref - vsa_sparse_attn_fwd under the two-stream budget:
 * a video query tile is allowed the non-reference prefix tiles, its ref_idx
 * reference tiles and its kv_idx video tiles; a prefix query tile is allowed
 * every tile. sparsity must be > 0. Other arguments as vsa_sparse_attn_fwd.
 */
VSA_API int vsa_sparse_attn_fwd_ref(const vsa_problem *prob, const void *qt, const void *kt,
                                    const void *vt, const int32_t *slot_to_token,
                                    const int32_t *kv_idx, double sparsity,
                                    const vsa_ref_budget *budget, const int32_t *ref_idx,
                                    float softmax_scale, void *out, float *lse,
                                    void *stream);

/* vsa_kept_stats_ref / vsa_count_flops_ref - host only: as vsa_kept_stats
 * and vsa_count_flops under the two-stream budget (ref_idx_host: HOST copy
 * of ref_idx). */
VSA_API int vsa_kept_stats_ref(const vsa_problem *prob, double sparsity,
                               const vsa_ref_budget *budget, int64_t *kept_tile_pairs,
                               double *frac_of_full);
VSA_API int vsa_count_flops_ref(const vsa_problem *prob, double sparsity,
                                const vsa_ref_budget *budget,
                                const int32_t *slot_to_token_host,
                                const int32_t *kv_idx_host, const int32_t *ref_idx_host,
                                double *flops);

/*
 * vsa_teacher_map - the teacher tile map, a measurement aid: teacher[b][h][i][j]
 * is the largest full-attention probability (softmax over all real keys of
 * q.k * scale) over the real queries of video tile i and the real keys of
 * video tile j ("Veda Sparse Attention в ComfyUI", section "Что делает Veda":
 * full attention max-pooled per tile is the teacher). Same layout as the
 * scores of vsa_tile_scores, so vsa_select_topk on it gives the teacher's
 * top-k. lse_ws: device float workspace of B*H*max_video_tiles*64 elements
 * (per-query log-sum-exp, base 2). softmax_scale <= 0 selects 1/sqrt(d).
 * Costs two dense passes of Q K^T.
 */
VSA_API int vsa_teacher_map(const vsa_problem *prob, const void *qt, const void *kt,
                            const int32_t *slot_to_token, float softmax_scale, float *lse_ws,
                            float *teacher, void *stream);

/*
 * vsa_quantize_fp8 - inputs of the low-precision (fp8) attention variant.
 * The node runs its attention as a quantized kernel ("Veda Sparse Attention
 * в ComfyUI", section "Узел ComfyUI"); here the format is OCP FP8 E4M3,
 * the MI355X matrix core's 8-bit type.
 *
 * Every tile of every head of qt, kt, vt (bf16, as written by vsa_map_tiles)
 * gets one power-of-two scale 2^e: e is the least integer with
 * max|x| * 2^-e <= 448 (e = 0 for an all-zero tile; e >= -127). The tile's
 * values x * 2^-e are rounded to E4M3 (nearest, ties to even).
 *
 * q8, k8, v8: device, tiled_elems BYTES each (same tile order as qt), in the
 *   fp8 operand layouts: Q and K tiles are 2 KB blocks of 32 slots x 64
 *   channels, block (s/32)*(d/64) + c/64; V tiles are 2 KB blocks of
 *   64 keys x 32 channels, block c/32. Inside a block, lane L (0..63) holds
 *   32 bytes as two 16-byte halves at half*1024 + L*16:
 *     Q/K: L = s%32 + 32*g, byte e (half e/16, e%16 within it) is channel
 *          64*(c/64) + 32*g + e;
 *     V:   L = c%32 + 32*g, byte e is key (e/16)*32 + 8*((e%16)/4) + 4*g + e%4.
 * scales: device uint8 [B][H][max_tiles][4], byte 0/1/2 = e + 127 of the Q/K/V
 *   tile, byte 3 unused; 4-byte aligned.
 * Only tiles that exist for the head's shape are written. dtype must be
 * VSA_BF16 (VSA_ERR_UNSUPPORTED otherwise). Inputs must be finite: a tile
 * holding an infinity or NaN has no scale, and its codes are unspecified.
 */
VSA_API int vsa_quantize_fp8(const vsa_problem *prob, const void *qt, const void *kt,
                             const void *vt, void *q8, void *k8, void *v8, void *scales,
                             void *stream);

/*
 * vsa_map_tiles_fp8 - vsa_map_tiles and vsa_quantize_fp8 in one pass: the
 * same slot_to_token, bf16 tiles (for scoring) and E4M3 tiles plus scale
 * bytes (for vsa_sparse_attn_fwd_fp8), bit for bit, without reading the
 * bf16 tiles back. q, k, v and every output are required; bf16 only.
 */
VSA_API int vsa_map_tiles_fp8(const vsa_problem *prob, const void *q, const void *k,
                              const void *v, int32_t *slot_to_token, void *qt, void *kt,
                              void *vt, void *q8, void *k8, void *v8, void *scales,
                              void *stream);

/*
 * vsa_sparse_attn_fwd_fp8 - step 4 on the fp8 copies: the same key-tile
 * lists, mask and outputs as vsa_sparse_attn_fwd (budget == NULL) or
 * vsa_sparse_attn_fwd_ref (budget and ref_idx given), computed from the E4M3
 * values times their tile scales. Probabilities are rounded to E4M3 before
 * the PV product (the row max is kept 8 below the true max, so they lie in
 * (0, 256]); row sums use the same rounded values. out: bf16 [B][H][N][d];
 * lse: float [B][H][N] or NULL. dtype must be VSA_BF16.
 */
VSA_API int vsa_sparse_attn_fwd_fp8(const vsa_problem *prob, const void *q8, const void *k8,
                                    const void *v8, const void *scales,
                                    const int32_t *slot_to_token, const int32_t *kv_idx,
                                    double sparsity, const vsa_ref_budget *budget,
                                    const int32_t *ref_idx, float softmax_scale, void *out,
                                    float *lse, void *stream);

/*
 * Measurement aids for the rooflines; neither is a step of the method.
 *
 * vsa_device_clocks - the current HIP device's compute-unit count, the
 * engine clock the runtime reports for it (kHz; its maximum, the clock the
 * published matrix-core peaks assume) and the rate of its constant
 * real-time counter (kHz). The dense bf16 peak at a clock f is
 * CUs x f x 4096 flop per clock (twice that for fp8). Any pointer may be
 * NULL. VSA_ERR_HIP if the runtime call fails (for instance, no device).
 *
 * vsa_mfma_probe - a pure matrix-core load, to measure the rate and clock
 * the chip sustains under it. n_workgroups workgroups of 256 threads (4
 * waves); every wave runs `iters` trips of 4 independent MFMAs:
 *   kind 0: bf16 32x32x16   (32768 flop each, the bf16 attention's type)
 *   kind 1: E4M3 32x32x64 with unit block scales (131072 flop each)
 * so one launch performs n_workgroups * 16 * iters MFMAs. Kinds 2-4 run
 * workgroups of 512 threads (8 waves, two on every SIMD) of kind 1's trips:
 *   kind 2: every wave runs the trips (32 MFMAs per workgroup and trip)
 *   kind 3: every wave adds 16 exponentials (v_exp_f32) per trip (32 MFMAs)
 *   kind 4: waves 0-3 run the trips, waves 4-7 only the 16 exponentials per
 *           trip (16 MFMAs per workgroup and trip). ticks: device
 * uint64 [n_workgroups][4] or NULL, 8-byte aligned; workgroup w writes the
 * span of its waves' loops on the shader tick counter (earliest start
 * ticks[w][0], latest end [1]) and on the real-time counter ([2], [3]).
 * Nothing else is written. 1 <= iters <= 2^22 and 1 <= n_workgroups <= 2^16
 * (VSA_ERR_SIZE above, VSA_ERR_INVALID_ARG below or for a kind outside 0..4).
 */
VSA_API int vsa_device_clocks(int32_t *cu_count, int32_t *clock_khz, int32_t *wall_khz);
VSA_API int vsa_mfma_probe(int32_t kind, int32_t iters, int32_t n_workgroups, uint64_t *ticks,
                           void *stream);

/* Static text for a vsa_status value. */
VSA_API const char *vsa_status_string(int status);

/* VSA_VERSION of the built library. */
VSA_API int vsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
