"""Helpers for the GPU parity tests: run a HIP stage and its oracle counterpart
on the same seeded inputs and measure the disagreement."""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_attention_38_amd import synth
from block_sparse_attention_38_amd.workloads import CLUSTERS, KMEANS_ITERS, Workload

# Tolerances (the floating-point bars are stated with their derivation in the
# design notes):
SCORE_RTOL = 1e-4          # scores, relative per element
ATT_ATOL_BF16 = 2e-2       # attention outputs, bf16 inputs, fp32 accumulation
ATT_ATOL_F32 = 1e-4        # attention outputs, fp32 inputs
CENT_RTOL = 1e-5           # centroids, relative to the block's largest |centroid|
POOL_RTOL = 1e-5           # pooled keys, relative to the layer's largest |kbar|
NEAR_TIE = 1e-4            # k-means blocks whose two best distances are closer are not compared


def device():
    return torch.device("cuda:0")


def inputs(w: Workload, seed: int, step: int = 0):
    q, k, v = synth.make_inputs(w, seed, step)
    dev = device()
    return (q, k, v), (q.to(dev), k.to(dev), v.to(dev))


def make_plan(aba, w: Workload, density: float | None = None, budget: int | None = None):
    K = w.budget(density) if budget is None else budget
    return aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS, K)


def make_fine_plan(aba, w: Workload, density: float | None = None, budget: int | None = None):
    """A plan with 4-token key blocks, at the 128-token budget's number of tiles unless given."""
    K = w.fine_budget(density) if budget is None else budget
    return aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, CLUSTERS, KMEANS_ITERS, K,
                    key_block=aba.FINE_BLOCK)


def att_tol(w: Workload) -> float:
    return ATT_ATOL_BF16 if w.dtype == "bf16" else ATT_ATOL_F32


def gpu_rows(out: torch.Tensor, items, blk: int = 128) -> np.ndarray:
    """Rows of the listed (b, h, query block) items of a [B,H,N_pad,D] output, as fp64 [n, blk, D]."""
    o = out.float().cpu()
    return np.stack([o[b, h, qb * blk:(qb + 1) * blk].numpy() for b, h, qb in items]).astype(np.float64)


def sample_items(w: Workload, n: int, seed: int = 0, include_last: bool = True):
    rng = np.random.default_rng(seed)
    items = {(int(rng.integers(w.batch)), int(rng.integers(w.heads)), int(rng.integers(w.n_blocks)))
             for _ in range(n)}
    if include_last:
        items.add((0, w.heads - 1, w.n_blocks - 1))
        items.add((0, 0, 0))
    return sorted(items)


def compare_lists(g_idx, g_cnt, g_w, o_idx, o_cnt, o_w):
    """Number of rows whose (cnt, idx[:cnt], w[:cnt]) differ bit for bit."""
    g_idx, g_cnt, g_w = g_idx.cpu().numpy(), g_cnt.cpu().numpy(), g_w.cpu().numpy()
    if not np.array_equal(g_cnt, o_cnt):
        return int((g_cnt != o_cnt).sum())
    bad = 0
    flat_g = g_idx.reshape(-1, g_idx.shape[-1]), g_w.reshape(-1, g_w.shape[-1])
    flat_o = o_idx.reshape(-1, o_idx.shape[-1]), o_w.reshape(-1, o_w.shape[-1])
    for r, c in enumerate(o_cnt.reshape(-1)):
        if not (np.array_equal(flat_g[0][r, :c], flat_o[0][r, :c])
                and np.array_equal(flat_g[1][r, :c].view(np.uint32), flat_o[1][r, :c].view(np.uint32))):
            bad += 1
    return bad
