"""The synthetic workloads: raw parameters only, no arithmetic of the method.

Each entry restates one benchmark shape of tile-sparse video attention:
batch, heads, head dim, the latent video grid (T, H, W), the prefix segment
lengths in sequence order (text, reference image, reference audio), the tile
shapes that heads cycle through, the tile scorer, the sparsity and the seed.

Shapes follow the workloads the pages talk about: a 1344x768 clip is a
48x84 latent frame ("Veda Sparse Attention в ComfyUI", section
"Производительность": one attention layer at about 104k tokens), 64-token
tiles of 4x4x4 ("From 650 s to 72 s", section "The method") and per-head
(pt, ph, pw) shapes with pt*ph*pw = 64 ("BSAI-ComfyUI-VedaSparse" README,
section "一、插件说明 / Overview", Head-Aware Tiling row).

Nothing here derives tile counts, k or any other quantity of the method:
the oracle and the library each do that on their own.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

VSA_SHAPE = ((4, 4, 4),)
HEAD_AWARE_CYCLE = ((4, 4, 4), (1, 8, 8), (16, 2, 2))
SHORT_PREFIX = (40, 64, 24)          # text, ref-image, ref-audio
REF2VA_PREFIX = (512, 4032, 128)     # text, one 48x84 ref frame, ref-audio


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16"
    B: int
    H: int
    d: int
    grid: Tuple[int, int, int]      # (T, Hv, Wv) latent video grid
    prefix: Tuple[int, ...]         # prefix segment lengths, sequence order
    tile_shapes: Tuple[Tuple[int, int, int], ...]
    scorer: str                     # "mean_gate" or "trippool"
    sparsity: float
    seed: int
    proj_dim: int = 32              # TripPool per-head projection width
    tripool_mode: str = "triplet"   # TripPool statistics: triplet, maxmin, avg
    note: str = field(default="", compare=False)

    @property
    def n_video_tokens(self) -> int:
        T, Hv, Wv = self.grid
        return T * Hv * Wv

    @property
    def N(self) -> int:
        return sum(self.prefix) + self.n_video_tokens


WORKLOADS = {
    "1": Workload("tiny-f32", "f32", 1, 2, 64, (4, 8, 8), SHORT_PREFIX,
                  VSA_SHAPE, "mean_gate", 0.75, 1001,
                  note="256 video tokens, 4 tiles, top-1 of 4"),
    "2": Workload("short-clip-bf16", "bf16", 1, 24, 128, (8, 48, 84),
                  REF2VA_PREFIX, VSA_SHAPE, "mean_gate", 0.75, 1002,
                  note="32,256 video tokens, keep 25%"),
    "3a": Workload("full-clip-bf16", "bf16", 1, 24, 128, (28, 48, 84),
                   SHORT_PREFIX, VSA_SHAPE, "mean_gate", 0.75, 1003,
                   note="112,896 video tokens, 75% sparsity (headline)"),
    "3b": Workload("full-clip-ref2va-bf16", "bf16", 1, 24, 128, (28, 48, 84),
                   REF2VA_PREFIX, VSA_SHAPE, "mean_gate", 0.75, 1003,
                   note="3a with the long reference prefix"),
    "4a": Workload("veda-short-bf16", "bf16", 1, 24, 128, (8, 48, 84),
                   REF2VA_PREFIX, HEAD_AWARE_CYCLE, "trippool", 0.90, 1004,
                   note="TripPool, head-aware tiles, keep 10%"),
    "4b": Workload("veda-full-bf16", "bf16", 1, 24, 128, (28, 48, 84),
                   REF2VA_PREFIX, HEAD_AWARE_CYCLE, "trippool", 0.90, 1004,
                   note="TripPool at the full-clip grid"),
    "5": Workload("long-clip-bf16", "bf16", 1, 24, 128, (60, 48, 84),
                  REF2VA_PREFIX, HEAD_AWARE_CYCLE, "trippool", 0.95, 1005,
                  note="241,920 video tokens, keep 5%"),
}

# The workload the headline metric is quoted on.
HEADLINE = "3a"
