"""Workload shapes for the AB-Attention sparse attention layer.

The AB-Attention page evaluates Wan2.1 (81 frames) and HunyuanVideo (129 frames)
at 720p (section "Как мерили и что вышло"); the latent grids below (21 and 33
frames) are the shapes of those video layers.  No model weights or prompts are
used: inputs are synthetic (see ``synth.py``).

Budget: the page quotes sparsity as a share of attention skipped (89-92%, lede
and "Как мерили и что вышло").  A density d becomes an expected number of kept
key blocks per query block K = round-half-up(d * NB), at least 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

BLOCK = 128          # tokens per query block and per key block
FINE_BLOCK = 4       # tokens per key block of the fine-grained selection
CLUSTERS = 8         # IBCS clusters per query block
KMEANS_ITERS = 10    # Lloyd iterations


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    grid: tuple                     # latent grid (frames, height, width), flattened frame-major
    n_centres: int                  # Gaussian mixture centres per head
    densities: tuple                # target key-block densities
    tiles: int = 4                  # spatial tiles per frame side in the token -> centre map
    temporal_group: int = 1         # frames sharing one centre group (temporal locality)
    steps: int = 1                  # denoising steps (the sweep)
    drift: float = 0.0              # Euclidean drift of every centre per step
    description: str = field(default="", compare=False)

    @property
    def seq_len(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def n_blocks(self) -> int:
        return (self.seq_len + BLOCK - 1) // BLOCK

    @property
    def seq_pad(self) -> int:
        return self.n_blocks * BLOCK

    def budget(self, density: float | None = None) -> int:
        d = self.densities[0] if density is None else density
        return budget_for(d, self.n_blocks)

    @property
    def n_fine_blocks(self) -> int:
        return (self.seq_len + FINE_BLOCK - 1) // FINE_BLOCK

    def fine_budget(self, density: float | None = None) -> int:
        """Budget in 4-token key blocks with the same number of 128-key tiles as the
        128-token budget (the page's kernel paragraph compares the two at a fixed
        number of tiles)."""
        return (BLOCK // FINE_BLOCK) * self.budget(density)

    @property
    def dense_flops(self) -> float:
        """4 * B * H * N^2 * D: QK^T and PV of full attention over the valid tokens."""
        return 4.0 * self.batch * self.heads * float(self.seq_len) ** 2 * self.head_dim


def budget_for(density: float, n_blocks: int) -> int:
    return max(1, int(math.floor(density * n_blocks + 0.5)))


TINY = Workload("tiny", 1, 2, 64, "f32", (4, 16, 16), 16, (0.25,), tiles=2,
                description="batch 1, 2 heads, 1024 tokens (8 blocks of 128), head_dim 64, fp32, 16 centres")
SINGLE = Workload("single_layer", 1, 12, 128, "bf16", (21, 30, 52), 64, (0.10,),
                  description="batch 1, 12 heads, head_dim 128, bf16, 21x30x52 grid (32760 tokens), 64 centres")
WIDE = Workload("wide_head", 1, 40, 128, "bf16", (21, 30, 52), 64, (0.08, 0.10, 0.20), temporal_group=3,
                description="batch 1, 40 heads, head_dim 128, bf16, 21x30x52 grid, centres shared by 3 frames")
HIGHRES = Workload("high_res", 1, 24, 128, "bf16", (33, 45, 80), 128, (0.08,),
                   description="batch 1, 24 heads, head_dim 128, bf16, 33x45x80 grid (118800 tokens), 128 centres")
SWEEP = Workload("sweep", 1, 12, 128, "bf16", (21, 30, 52), 64, (0.10,), steps=30, drift=0.05,
                 description="single layer x 30 steps, fresh q/k/v per step, centres drifting by 0.05 per step")

ALL = {w.name: w for w in (TINY, SINGLE, WIDE, HIGHRES, SWEEP)}
