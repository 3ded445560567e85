"""Seeded synthetic video-token inputs (q, k, v) for the attention layer.

This module draws inputs only; it holds none of the layer's arithmetic, and
both the HIP path and the CPU oracle consume exactly the tensors it returns.

The AB-Attention page measures on real Wan2.1 / HunyuanVideo activations over
the Penguin Video prompts (section "Как мерили и что вышло"); those are not
available, so these inputs stand in for them with the layer's shapes and a
spatially and temporally structured token distribution:

* centres: mu_m = 3 * g_m / |g_m|, g_m ~ N(0, I_D), one set of M centres per head;
* token (t, y, x) of the frame-major latent grid maps to centre
  z = (tiles^2 * floor(t / temporal_group) + tiles * floor(tiles*y/Y) + floor(tiles*x/X)) mod M;
* keys k = mu_z + N(0, 1), queries q = mu_z + N(0, 0.5^2), values v ~ N(0, 1);
* the sweep drifts every centre by a Euclidean step of ``drift`` per denoising
  step: mu <- 3 * normalize(mu + drift * u), u a random unit vector, with fresh
  q/k/v per step;
* rows >= N (padding to a whole number of 128-token blocks) are zero.
"""
from __future__ import annotations

import torch

from .workloads import Workload

Q_STD = 0.5
K_STD = 1.0
CENTRE_NORM = 3.0

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def token_centres(w: Workload) -> torch.Tensor:
    """Centre index of every valid token, in frame-major order: int64 [N]."""
    T, Y, X = w.grid
    t = torch.arange(T).view(T, 1, 1)
    y = torch.arange(Y).view(1, Y, 1)
    x = torch.arange(X).view(1, 1, X)
    tiles = w.tiles
    region = tiles * ((tiles * y) // Y) + (tiles * x) // X
    z = (tiles * tiles * (t // w.temporal_group) + region) % w.n_centres
    return z.expand(T, Y, X).reshape(-1).contiguous()


def centres(w: Workload, seed: int, step: int = 0) -> torch.Tensor:
    """Mixture centres [H, M, D] (float64) after ``step`` drift steps."""
    g = torch.Generator().manual_seed(seed)
    mu = torch.randn(w.heads, w.n_centres, w.head_dim, generator=g, dtype=torch.float64)
    mu = CENTRE_NORM * mu / mu.norm(dim=-1, keepdim=True)
    for s in range(step):
        gs = torch.Generator().manual_seed(seed * 1_000_003 + 7919 * (s + 1))
        u = torch.randn(mu.shape, generator=gs, dtype=torch.float64)
        u = u / u.norm(dim=-1, keepdim=True)
        mu = mu + w.drift * u
        mu = CENTRE_NORM * mu / mu.norm(dim=-1, keepdim=True)
    return mu


def make_inputs(w: Workload, seed: int, step: int = 0):
    """q, k, v as CPU tensors [B, H, N_pad, D] in the workload's dtype, rows >= N zero."""
    H = w.heads
    N, N_pad, D, B = w.seq_len, w.seq_pad, w.head_dim, w.batch
    mu = centres(w, seed, step)                              # [H, M, D]
    z = token_centres(w)                                     # [N]
    g = torch.Generator().manual_seed(seed * 7 + 1 + 104729 * step)
    base = mu[:, z, :].to(torch.float32).unsqueeze(0)        # [1, H, N, D]
    out = {}
    for name in ("k", "q", "v"):
        noise = torch.randn(B, H, N, D, generator=g, dtype=torch.float32)
        if name == "k":
            val = base + K_STD * noise
        elif name == "q":
            val = base + Q_STD * noise
        else:
            val = noise
        full = torch.zeros(B, H, N_pad, D, dtype=torch.float32)
        full[:, :, :N, :] = val
        out[name] = full.to(torch_dtype(w.dtype)).contiguous()
        del noise, val, full
    return out["q"], out["k"], out["v"]


def random_scores(B: int, H: int, NBq: int, NBk: int, seed: int, peak: float = 4.0) -> torch.Tensor:
    """Random positive fp32 rows normalised to sum to about one, with a spread of
    magnitudes set by ``peak`` (inputs for tests of the sampling stage alone)."""
    g = torch.Generator().manual_seed(seed)
    logits = peak * torch.randn(B, H, NBq, NBk, generator=g, dtype=torch.float64)
    e = torch.exp(logits - logits.amax(dim=-1, keepdim=True))
    return (e / e.sum(dim=-1, keepdim=True)).to(torch.float32).contiguous()
