"""Pins for the oracle's IBCS stages: clustering, key pooling, block scores (CPU only).

IBCS, per the AB-Attention page (section "Три приёма AB-Attention", IBCS
paragraph): each 128-query block is grouped into 8 clusters with a centroid and
a weight equal to the cluster's share of the block's queries; a key block's
score is the weighted attention of the centroids to its averaged keys.  The page
contrasts this with averaging the whole query block into one vector (section
"Где ломаются прежние разреженные схемы"), which is IBCS with a single cluster.
"""
import itertools

import numpy as np
import pytest
import torch

BLK = 128


def _qk(seed, B=1, H=2, N=300, D=16, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    NB = (N + BLK - 1) // BLK
    q = torch.zeros(B, H, NB * BLK, D)
    k = torch.zeros(B, H, NB * BLK, D)
    q[:, :, :N] = torch.randn(B, H, N, D, generator=g) * spread
    k[:, :, :N] = torch.randn(B, H, N, D, generator=g)
    return q, k, NB


def test_pool_is_block_mean(oracle_mod):
    N = 3 * BLK - 50
    _, k, NB = _qk(1, N=N)
    kbar = oracle_mod.pool(k, N)
    for j in range(NB):
        ref = k[:, :, j * BLK:min(j * BLK + BLK, N)].double().mean(dim=2)
        assert torch.allclose(torch.from_numpy(kbar[:, :, j]), ref, rtol=0, atol=1e-14)


def test_scores_are_distributions(oracle_mod):
    N, D = 5 * BLK - 3, 16
    q, k, NB = _qk(2, N=N, D=D, spread=2.0)
    cent, w, _ = oracle_mod.kmeans(q, N, C=8, T=10)
    s = oracle_mod.score(cent, w, oracle_mod.pool(k, N), 1.0 / np.sqrt(D))
    assert s.shape == (1, 2, NB, NB)
    assert np.all(s >= 0)
    assert np.allclose(s.sum(-1), 1.0, rtol=0, atol=1e-12)


def _meanpool_scores(q, k, N, scale):
    """Mean-pool scorer of the page's earlier methods: softmax_j(s * qbar . kbar_j) (torch)."""
    NB = (N + BLK - 1) // BLK
    qbar = torch.stack([q[:, :, j * BLK:min(j * BLK + BLK, N)].double().mean(2) for j in range(NB)], 2)
    kbar = torch.stack([k[:, :, j * BLK:min(j * BLK + BLK, N)].double().mean(2) for j in range(NB)], 2)
    return torch.softmax(scale * qbar @ kbar.transpose(-1, -2), dim=-1)


def test_one_cluster_is_meanpool_scorer(oracle_mod):
    N, D = 4 * BLK - 77, 32
    q, k, NB = _qk(3, N=N, D=D, spread=3.0)
    scale = 1.0 / np.sqrt(D)
    cent, w, _ = oracle_mod.kmeans(q, N, C=1, T=10)
    assert np.all(w == 1.0)
    s = oracle_mod.score(cent, w, oracle_mod.pool(k, N), scale)
    assert torch.allclose(torch.from_numpy(s), _meanpool_scores(q, k, N, scale), rtol=0, atol=1e-13)


def test_identical_queries_collapse_to_meanpool(oracle_mod):
    """All queries of a block equal: one cluster holds every query (ties go to the first)."""
    N, D = 3 * BLK, 16
    q, k, NB = _qk(4, H=1, N=N, D=D)
    for j in range(NB):
        q[0, 0, j * BLK:(j + 1) * BLK] = q[0, 0, j * BLK]
    scale = 1.0 / np.sqrt(D)
    cent, w, _ = oracle_mod.kmeans(q, N, C=8, T=10)
    assert np.all(w[..., 0] == 1.0) and np.all(w[..., 1:] == 0.0)
    s = oracle_mod.score(cent, w, oracle_mod.pool(k, N), scale)
    assert torch.allclose(torch.from_numpy(s), _meanpool_scores(q, k, N, scale), rtol=0, atol=1e-13)


def test_key_block_seen_by_one_cluster_scores_its_share(oracle_mod):
    """Two well-separated query groups, and key blocks that only one group attends
    to: with the logits saturated, each centroid's softmax is one-hot on its own
    block, so that block's score is the group's share of the block's queries
    (IBCS paragraph: the weight of a centroid is its cluster's share).  Group B
    is exactly the 8 strided seed rows (share 8/128), so a scorer that weighted
    the centroids uniformly would give 1/8 and 7/8 instead of 120/128 and 8/128."""
    D = 16
    N = 3 * BLK
    u = torch.zeros(D)
    u[0] = 1.0
    v = torch.zeros(D)
    v[1] = 1.0
    alpha, beta = 40.0, 40.0                 # s * alpha * beta = 400: every softmax saturates
    q = torch.zeros(1, 1, N, D)
    k = torch.zeros(1, 1, N, D)
    q[0, 0, :] = alpha * u                   # group A everywhere ...
    for qb in range(3):
        q[0, 0, qb * BLK + 16 * torch.arange(8)] = alpha * v   # ... but the seed rows m * 128 / 8 are group B
    k[0, 0, 0:BLK] = beta * u                # key block 0: attended by group A only
    k[0, 0, BLK:2 * BLK] = beta * v          # key block 1: attended by group B only
    # key block 2 stays zero: logit 0 for every centroid, far below the saturated ones
    scale = 1.0 / np.sqrt(D)
    cent, w, _ = oracle_mod.kmeans(q, N, C=8, T=10)
    assert np.allclose(np.sort(w[0, 0], axis=-1)[..., ::-1][..., :2], [120 / 128, 8 / 128], rtol=0, atol=0)
    s = oracle_mod.score(cent, w, oracle_mod.pool(k, N), scale)
    for qb in range(3):
        assert abs(s[0, 0, qb, 0] - 120 / 128) < 1e-12
        assert abs(s[0, 0, qb, 1] - 8 / 128) < 1e-12
        assert s[0, 0, qb, 2] < 1e-12


def test_kmeans_invariants_and_monotone_objective(oracle_mod):
    rng = np.random.default_rng(5)
    for trial in range(6):
        n = [128, 120, 16, 77, 9, 128][trial]
        D = [16, 64, 128, 8, 32, 128][trial]
        x = (rng.normal(size=(n, D)) + rng.normal(size=(1, D)) * 2).astype(np.float32)
        prev = np.inf
        for T in range(0, 11):
            cent, w, a, _ = oracle_mod.kmeans_block(x, C=8, T=T)
            # Lloyd objective with the final centroids is non-increasing in T
            d2 = ((x[:, None, :].astype(np.float64) - cent[None]) ** 2).sum(-1)
            obj = d2.min(1).sum()
            assert obj <= prev * (1 + 1e-12)
            prev = obj
            if T == 0:
                continue
            assert abs(w.sum() - 1.0) < 1e-12
            assert np.allclose(np.bincount(a, minlength=8) / n, w, rtol=0, atol=0)
            # weights are cluster shares of the last assignment, centroids its means
            assert np.allclose((w[:, None] * cent).sum(0), x.astype(np.float64).mean(0), rtol=0, atol=1e-12)


def test_kmeans_with_fewer_rows_than_clusters(oracle_mod):
    """n < C distinct rows: the strided initial centroids x[floor(m n / C)] repeat
    rows, every row sits at distance 0 from its own copies and goes to the first
    of them, m = ceil(r C / n), so each such cluster holds one row (weight 1/n),
    the others stay empty and keep their copy, and nothing moves in later rounds.
    Copies tie exactly, so the smallest gap to a different centroid is 1."""
    rng = np.random.default_rng(8)
    for n, D in [(1, 128), (2, 64), (3, 16), (4, 128), (5, 64), (7, 32)]:
        x = rng.normal(size=(n, D)).astype(np.float32)
        cent, w, a, gap = oracle_mod.kmeans_block(x, C=8, T=10)
        first = [-(-r * 8 // n) for r in range(n)]                # ceil(r C / n)
        assert a.tolist() == first
        ref_w = np.zeros(8)
        ref_w[first] = 1.0 / n
        assert np.array_equal(w, ref_w)
        for m in range(8):
            assert np.array_equal(cent[m], x[m * n // 8].astype(np.float64))
        assert gap == 1.0
    # a row exactly halfway between two different centroids is a true tie: it
    # goes to the smaller index, and the gap says the assignment is fragile (0)
    x = np.zeros((3, 4), np.float32)
    x[0, 0], x[1, 0] = -1.0, 1.0                             # initial centroids rows 0 and 1; row 2 halfway
    _, w, a, gap = oracle_mod.kmeans_block(x, C=2, T=1)
    assert a.tolist() == [0, 1, 0] and gap == 0.0 and np.array_equal(w, [2 / 3, 1 / 3])


def test_kmeans_recovers_separated_blobs(oracle_mod):
    rng = np.random.default_rng(6)
    D = 32
    centres = np.zeros((2, D))
    centres[0, 0], centres[1, 0] = -20.0, 20.0
    labels = np.array([0] * 40 + [1] * 88)
    rng.shuffle(labels)
    x = (centres[labels] + rng.normal(size=(128, D))).astype(np.float32)
    cent, w, a, gap = oracle_mod.kmeans_block(x, C=2, T=10)
    mean0 = x[labels == 0].astype(np.float64).mean(0)
    mean1 = x[labels == 1].astype(np.float64).mean(0)
    got = sorted([cent[0], cent[1]], key=lambda c: c[0])
    assert np.allclose(got[0], mean0, atol=1e-12) and np.allclose(got[1], mean1, atol=1e-12)
    assert sorted(w.tolist()) == [40 / 128, 88 / 128]
    assert gap > 0.5


def test_kmeans_matches_sklearn_lloyd(oracle_mod):
    """scikit-learn's Lloyd k-means with the same initial centroids, when no cluster empties."""
    sklearn_cluster = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(7)
    compared = 0
    for trial in range(12):
        n, D = 128, [16, 64, 128][trial % 3]
        means = rng.normal(size=(8, D)) * 1.5
        x = (means[rng.integers(0, 8, size=n)] + rng.normal(size=(n, D))).astype(np.float32)
        cent, w, a, gap = oracle_mod.kmeans_block(x, C=8, T=10)
        if np.any(np.bincount(a, minlength=8) == 0) or gap < 1e-6:
            continue
        init = x[[m * n // 8 for m in range(8)]].astype(np.float64)
        km = sklearn_cluster.KMeans(n_clusters=8, init=init, n_init=1, max_iter=10, tol=0.0, algorithm="lloyd")
        km.fit(x.astype(np.float64))
        # scikit-learn relocates empty clusters during the run; only compare runs where it never did
        if np.any(np.bincount(km.labels_, minlength=8) == 0):
            continue
        assert np.allclose(km.cluster_centers_, cent, rtol=0, atol=1e-10)
        compared += 1
    assert compared >= 6


def test_block_mass_rows_and_torch(oracle_mod):
    N, D = 4 * BLK - 20, 16
    q, k, NB = _qk(8, H=1, N=N, D=D, spread=2.0)
    scale = 1.0 / np.sqrt(D)
    items = [(0, 0, j) for j in range(NB)]
    mass = oracle_mod.block_mass(q, k, N, items=items, scale=scale)
    p = torch.softmax(scale * q[0, 0, :N].double() @ k[0, 0, :N].double().T, dim=-1)
    for j in range(NB):
        rows = p[j * BLK:min(j * BLK + BLK, N)]
        ref = torch.stack([rows[:, t * BLK:min(t * BLK + BLK, N)].sum(1).mean() for t in range(NB)])
        assert torch.allclose(torch.from_numpy(mass[j]), ref, rtol=0, atol=1e-13)
    assert np.allclose(mass.sum(1), 1.0, atol=1e-12)


def test_topk_mass_brute_force(oracle_mod):
    """Ideal top-k retention equals the best mass over all C(NB, K) block subsets."""
    N, D = 8 * BLK, 64
    q, k, NB = _qk(9, H=2, N=N, D=D, spread=3.0)
    items = oracle_mod.layer_items(1, 2, NB)
    mass = oracle_mod.block_mass(q, k, N, items=items)
    for row in mass:
        for K in range(1, NB + 1):
            best = max(sum(row[list(c)]) for c in itertools.combinations(range(NB), K))
            assert abs(oracle_mod.topk_mass(row, K) - best) < 1e-14
