"""Pins for the oracle with fine-grained key blocks (CPU only).

The AB-Attention page (section "Три приёма AB-Attention", the kernel paragraph)
selects key/value blocks of only 4 tokens while the query blocks stay at 128
tokens, and gathers the selected small blocks into full matrix-core tiles.  The
oracle takes this as a key-block size kblk = 4 in pooling, scoring, sampling,
attention and the attention mass.  These pins tie the fine-grained results to
torch's fp64 softmax attention, to the coarse (128-token) results they must
agree with, and to exact enumeration of the sampling distribution.
"""
import itertools

import numpy as np
import pytest
import torch

BLK, FINE = 128, 4
TWO32 = float(2**32)


def _qkv(seed, H=1, N=300, D=16, spread=1.5):
    g = torch.Generator().manual_seed(seed)
    NB = (N + BLK - 1) // BLK
    pad = NB * BLK
    q, k, v = (torch.zeros(1, H, pad, D) for _ in range(3))
    q[:, :, :N] = torch.randn(1, H, N, D, generator=g) * spread
    k[:, :, :N] = torch.randn(1, H, N, D, generator=g)
    v[:, :, :N] = torch.randn(1, H, N, D, generator=g)
    return q, k, v, NB


def _sdpa(q_rows, k_rows, v_rows, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        q_rows.double()[None, None], k_rows.double()[None, None], v_rows.double()[None, None], scale=scale)[0, 0]


def _group_rows(x, h, groups, N):
    return torch.cat([x[0, h, g * FINE:min(g * FINE + FINE, N)] for g in groups], 0)


@pytest.mark.parametrize("N", [256, 301])
def test_fine_pool_is_group_mean(oracle_mod, N):
    _, k, _, _ = _qkv(1, H=2, N=N)
    kbar = oracle_mod.pool(k, N, blk=FINE)
    NBk = (N + FINE - 1) // FINE
    assert kbar.shape == (1, 2, NBk, 16)
    for g in range(NBk):
        ref = k[:, :, g * FINE:min(g * FINE + FINE, N)].double().mean(dim=2)
        assert torch.allclose(torch.from_numpy(kbar[:, :, g]), ref, rtol=0, atol=1e-14)


def test_fine_pool_averages_to_coarse_pool(oracle_mod):
    """A full 128-token block's mean is the mean of its 32 group means."""
    N = 3 * BLK
    _, k, _, _ = _qkv(2, N=N)
    fine = oracle_mod.pool(k, N, blk=FINE)
    coarse = oracle_mod.pool(k, N)
    assert np.allclose(fine.reshape(1, 1, 3, 32, -1).mean(3), coarse, rtol=0, atol=1e-14)


def test_fine_scores_are_distributions_and_one_cluster_is_meanpool(oracle_mod):
    N, D = 2 * BLK - 6, 16
    q, k, _, NB = _qkv(3, N=N, D=D, spread=2.0)
    scale = 1.0 / np.sqrt(D)
    kbar = oracle_mod.pool(k, N, blk=FINE)
    cent, w, _ = oracle_mod.kmeans(q, N, C=8, T=10)
    s = oracle_mod.score(cent, w, kbar, scale)
    assert s.shape == (1, 1, NB, kbar.shape[2])
    assert np.all(s >= 0) and np.allclose(s.sum(-1), 1.0, rtol=0, atol=1e-12)
    # one cluster: the block-mean query's softmax over the group means (torch)
    c1, w1, _ = oracle_mod.kmeans(q, N, C=1, T=10)
    s1 = oracle_mod.score(c1, w1, kbar, scale)
    qbar = torch.stack([q[0, 0, j * BLK:min(j * BLK + BLK, N)].double().mean(0) for j in range(NB)])
    ref = torch.softmax(scale * qbar @ torch.from_numpy(kbar[0, 0]).T, dim=-1)
    assert torch.allclose(torch.from_numpy(s1[0, 0]), ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("N", [256, 299])
def test_fine_every_group_kept_is_dense(oracle_mod, N):
    D = 16
    q, k, v, NB = _qkv(4, H=2, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    NBk = (N + FINE - 1) // FINE
    idx = np.tile(np.arange(NBk, dtype=np.int32), (1, 2, NB, 1))
    cnt = np.full((1, 2, NB), NBk, np.int32)
    w = np.ones_like(idx, dtype=np.float32)
    items = oracle_mod.layer_items(1, 2, NB)
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=items, scale=scale, kblk=FINE)
    for it, (b, h, qb) in enumerate(items):
        nq = min(BLK, N - qb * BLK)
        ref = _sdpa(q[b, h, qb * BLK:qb * BLK + nq], k[b, h, :N], v[b, h, :N], scale)
        assert torch.allclose(torch.from_numpy(out[it, :nq]), ref, rtol=0, atol=1e-12)
        assert np.all(out[it, nq:] == 0.0)


def test_fine_integer_weights_are_group_replication(oracle_mod):
    """A 4-token block of weight c counts as its keys and values repeated c times."""
    N, D = 2 * BLK - 2, 16
    q, k, v, NB = _qkv(5, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    NBk = (N + FINE - 1) // FINE
    rng = np.random.default_rng(5)
    idx = np.zeros((1, 1, NB, NBk), np.int32)
    cnt = np.zeros((1, 1, NB), np.int32)
    w = np.zeros((1, 1, NB, NBk), np.float32)
    lists = []
    for qb in range(NB):
        groups = sorted(rng.choice(NBk, size=int(rng.integers(1, 20)), replace=False).tolist())
        if qb == NB - 1:
            groups = sorted(set(groups) | {NBk - 1})      # the partial last group
        reps = rng.integers(1, 5, size=len(groups))
        idx[0, 0, qb, :len(groups)] = groups
        w[0, 0, qb, :len(groups)] = reps
        cnt[0, 0, qb] = len(groups)
        lists.append((groups, reps))
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=[(0, 0, qb) for qb in range(NB)], scale=scale, kblk=FINE)
    for qb, (groups, reps) in enumerate(lists):
        rep = [g for g, c in zip(groups, reps) for _ in range(int(c))]
        nq = min(BLK, N - qb * BLK)
        ref = _sdpa(q[0, 0, qb * BLK:qb * BLK + nq], _group_rows(k, 0, rep, N), _group_rows(v, 0, rep, N), scale)
        assert torch.allclose(torch.from_numpy(out[qb, :nq]), ref, rtol=0, atol=1e-12)


def test_fine_mass_matches_torch_and_sums_to_coarse(oracle_mod):
    N, D = 3 * BLK - 10, 16
    q, k, _, NB = _qkv(6, N=N, D=D, spread=2.0)
    scale = 1.0 / np.sqrt(D)
    items = [(0, 0, j) for j in range(NB)]
    fine = oracle_mod.block_mass(q, k, N, items=items, scale=scale, kblk=FINE)
    coarse = oracle_mod.block_mass(q, k, N, items=items, scale=scale)
    NBk = (N + FINE - 1) // FINE
    assert fine.shape == (NB, NBk)
    p = torch.softmax(scale * q[0, 0, :N].double() @ k[0, 0, :N].double().T, dim=-1)
    for j in range(NB):
        rows = p[j * BLK:min(j * BLK + BLK, N)]
        ref = torch.stack([rows[:, g * FINE:min(g * FINE + FINE, N)].sum(1).mean() for g in range(NBk)])
        assert torch.allclose(torch.from_numpy(fine[j]), ref, rtol=0, atol=1e-13)
    padded = np.zeros((NB, NB * 32))
    padded[:, :NBk] = fine
    assert np.allclose(padded.reshape(NB, NB, 32).sum(2), coarse, rtol=0, atol=1e-13)


def test_fine_ideal_topk_keeps_at_least_the_coarse_mass(oracle_mod):
    """Every set of K coarse blocks is a set of 32K fine blocks, so the ideal fine
    top-32K mass is never below the ideal coarse top-K mass (the page's 59% -> 69%
    comparison at an equal number of tiles)."""
    N, D = 8 * BLK, 32
    q, k, _, NB = _qkv(7, H=2, N=N, D=D, spread=3.0)
    items = oracle_mod.layer_items(1, 2, NB)
    fine = oracle_mod.block_mass(q, k, N, items=items, kblk=FINE)
    coarse = oracle_mod.block_mass(q, k, N, items=items)
    for f_row, c_row in zip(fine, coarse):
        for K in range(1, NB + 1):
            assert oracle_mod.topk_mass(f_row, 32 * K) >= oracle_mod.topk_mass(c_row, K) - 1e-14


def test_fine_ht_estimator_is_unbiased_by_enumeration(oracle_mod):
    """32 tokens in 8 groups of 4: the probability-weighted sum over every kept /
    not-kept pattern of the free groups equals the dense numerator and normaliser."""
    N, D, K = 32, 8, 3
    q, k, v, _ = _qkv(8, N=N, D=D, spread=2.0)
    scale = 1.0 / np.sqrt(D)
    NBk = N // FINE
    kbar = oracle_mod.pool(k, N, blk=FINE)
    cent, w, _ = oracle_mod.kmeans(q, N, C=4, T=5)
    scores = oracle_mod.score(cent, w, kbar, scale).astype(np.float32)
    theta, t = oracle_mod.thresholds(scores[0, 0, 0], K)
    assert abs(theta.astype(np.float64).sum() / TWO32 - K) <= NBk / TWO32
    pi = theta.astype(np.float64) / TWO32
    wts = (TWO32 / theta.astype(np.float64)).astype(np.float32)
    free = [j for j in range(NBk) if theta[j] < 2**32]
    forced = [j for j in range(NBk) if theta[j] == 2**32]
    patterns = [[j for b, j in enumerate(free) if (mask >> b) & 1] for mask in range(1 << len(free))]
    P = len(patterns)
    qq, kk, vv = (x.expand(1, P, BLK, D).contiguous() for x in (q, k, v))
    idx = np.zeros((1, P, 1, NBk), np.int32)
    cnt = np.zeros((1, P, 1), np.int32)
    wl = np.zeros((1, P, 1, NBk), np.float32)
    prob = np.zeros(P)
    for p, sub in enumerate(patterns):
        kept = sorted(forced + sub)
        idx[0, p, 0, :len(kept)] = kept
        wl[0, p, 0, :len(kept)] = wts[kept]
        cnt[0, p, 0] = len(kept)
        prob[p] = np.prod([pi[j] if j in sub else 1 - pi[j] for j in free])
    assert abs(prob.sum() - 1) < 1e-12
    logits = scale * q[0, 0, :N].double() @ k[0, 0, :N].double().T
    M = logits.max(1).values.numpy()
    shift = np.zeros((P, BLK))
    shift[:, :N] = M
    _, num, den = oracle_mod.attend(qq, kk, vv, N, idx, cnt, wl, items=[(0, p, 0) for p in range(P)],
                                    scale=scale, shift=shift, kblk=FINE)
    e = torch.exp(logits - torch.from_numpy(M)[:, None])
    exp_den = prob @ den[:, :N]
    exp_num = np.tensordot(prob, num[:, :N], axes=1)
    assert np.allclose(exp_den, e.sum(1).numpy(), rtol=2.0**-23, atol=0)
    assert np.allclose(exp_num, (e @ v[0, 0, :N].double()).numpy(), rtol=2.0**-23,
                       atol=2.0**-23 * e.sum(1).max().item())


def test_fine_sampling_budget_on_a_long_row(oracle_mod):
    """8190 groups and a budget of 832 (26 coarse blocks of 32 groups): inclusion
    probabilities sum to K, the always-kept blocks are the top of the sorted order,
    and the kept lists of many seeds average K blocks."""
    rng = np.random.default_rng(9)
    NBk, K = 8190, 832
    s = rng.gamma(0.3, size=NBk)
    s[rng.choice(NBk, 40, replace=False)] *= 500.0          # a few heavy groups that cap
    s = (s / s.sum()).astype(np.float32)
    theta, t = oracle_mod.thresholds(s, K)
    assert abs(theta.astype(np.float64).sum() / TWO32 - K) <= NBk / TWO32
    capped = np.flatnonzero(theta == 2**32)
    assert len(capped) == t and t > 1
    sigma = np.floor(s.astype(np.float64) * TWO32)
    order = np.lexsort((np.arange(NBk), -sigma))
    assert set(order[:t].tolist()) == set(capped.tolist())
    counts = []
    for seed in range(20):
        idx, cnt, w, _ = oracle_mod.sample(s.reshape(1, 1, 1, NBk), K, seed=seed)
        c = int(cnt[0, 0, 0])
        assert np.all(np.diff(idx[0, 0, 0, :c]) > 0) and set(capped.tolist()) <= set(idx[0, 0, 0, :c].tolist())
        counts.append(c)
    sd = np.sqrt((theta.astype(np.float64) / TWO32 * (1 - theta.astype(np.float64) / TWO32)).sum())
    assert abs(np.mean(counts) - K) <= 5 * sd / np.sqrt(len(counts))
