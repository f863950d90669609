"""CPU oracle for tile-sparse video attention (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding. It shares
no code with the HIP path. See vsa_oracle.py for the steps and their sources.
"""
from .vsa_oracle import (  # noqa: F401
    TILE, TileMap, tile_map, gather, pool_mean_gate, pool_trippool, TRIPOOL_MODES,
    tile_scores, keep_count, select_topk, allowed_tiles, softmax_attention,
    sparse_attention, dense_attention, effective_flops, head_forward,
    segment_tiles, allowed_two_stream, teacher_tile_map, tile_recall,
    E4M3_MAX, e4m3_round, tile_scale_exponent, quantize_tiles_e4m3, ungather,
    fp8_attention_inputs,
)
