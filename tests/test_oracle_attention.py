"""Pins for the oracle's attention routines (CPU only).

Pinned against torch's scaled_dot_product_attention in fp64 (textbook softmax
attention) and against the AB-Attention page's worked example for the
inverse-inclusion weight: a block kept with probability 25% counts as four
(section "Три приёма AB-Attention", SIP paragraph), i.e. an integer weight is
the same as repeating that block's keys and values.
"""
import json
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
BLK = 128


def _case(seed, B=1, H=2, N=300, D=16, logit_std=1.5):
    g = torch.Generator().manual_seed(seed)
    NB = (N + BLK - 1) // BLK
    pad = NB * BLK
    q = torch.zeros(B, H, pad, D)
    k = torch.zeros(B, H, pad, D)
    v = torch.zeros(B, H, pad, D)
    q[:, :, :N] = torch.randn(B, H, N, D, generator=g) * logit_std
    k[:, :, :N] = torch.randn(B, H, N, D, generator=g)
    v[:, :, :N] = torch.randn(B, H, N, D, generator=g)
    return q, k, v, NB


def _sdpa(q_rows, k_rows, v_rows, scale):
    """Reference: torch SDPA in fp64 on explicit key/value rows."""
    return torch.nn.functional.scaled_dot_product_attention(
        q_rows.double()[None, None], k_rows.double()[None, None], v_rows.double()[None, None], scale=scale
    )[0, 0]


def _rows(x, b, h, blocks, N):
    parts = [x[b, h, j * BLK:min(j * BLK + BLK, N)] for j in blocks]
    return torch.cat(parts, 0)


def _item_out(out, it, qb, N):
    nq = min(BLK, N - qb * BLK)
    return torch.from_numpy(out[it, :nq])


@pytest.mark.parametrize("N,D", [(300, 16), (256, 64), (129, 128)])
def test_dense_matches_sdpa(oracle_mod, N, D):
    q, k, v, NB = _case(1, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    items = oracle_mod.layer_items(1, 2, NB)
    out = oracle_mod.attend_full(q, k, v, N, items=items, scale=scale)
    for it, (b, h, qb) in enumerate(items):
        nq = min(BLK, N - qb * BLK)
        ref = _sdpa(q[b, h, qb * BLK:qb * BLK + nq], k[b, h, :N], v[b, h, :N], scale)
        assert torch.allclose(_item_out(out, it, qb, N), ref, rtol=0, atol=1e-12)
        assert np.all(out[it, nq:] == 0.0)  # padded query rows are zero


def test_full_list_unit_weights_is_dense(oracle_mod):
    N, D = 300, 16
    q, k, v, NB = _case(2, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    idx = np.tile(np.arange(NB, dtype=np.int32), (1, 2, NB, 1))
    cnt = np.full((1, 2, NB), NB, np.int32)
    w = np.ones_like(idx, dtype=np.float32)
    items = oracle_mod.layer_items(1, 2, NB)
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=items, scale=scale)
    for it, (b, h, qb) in enumerate(items):
        nq = min(BLK, N - qb * BLK)
        ref = _sdpa(q[b, h, qb * BLK:qb * BLK + nq], k[b, h, :N], v[b, h, :N], scale)
        assert torch.allclose(_item_out(out, it, qb, N), ref, rtol=0, atol=1e-12)


def _plan(NB, lists):
    """idx/cnt/w arrays [1, 1, NB, NB] with the given per-query-block (blocks, weights)."""
    idx = np.zeros((1, 1, NB, NB), np.int32)
    cnt = np.zeros((1, 1, NB), np.int32)
    w = np.zeros((1, 1, NB, NB), np.float32)
    for qb, (blocks, weights) in enumerate(lists):
        cnt[0, 0, qb] = len(blocks)
        idx[0, 0, qb, :len(blocks)] = blocks
        w[0, 0, qb, :len(blocks)] = weights
    return idx, cnt, w


def test_page_example_weight_four_is_replication(oracle_mod):
    """The page's worked example: a block with inclusion probability 25% counts as four."""
    ex = json.load(open(os.path.join(HERE, "golden", "ht_weight_example.json")))
    assert ex["weight"] == 1.0 / ex["inclusion_probability"]
    N, D = 4 * BLK, 32
    q, k, v, NB = _case(3, H=1, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    kept = [0, 2, 3]
    weights = [1.0, ex["weight"], 1.0]      # block 2 was drawn with probability 25%
    idx, cnt, w = _plan(NB, [(kept, weights)] * NB)
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=[(0, 0, qb) for qb in range(NB)], scale=scale)
    rep = [0] + [2] * ex["replication_factor"] + [3]
    for qb in range(NB):
        ref = _sdpa(q[0, 0, qb * BLK:qb * BLK + BLK], _rows(k, 0, 0, rep, N), _rows(v, 0, 0, rep, N), scale)
        assert torch.allclose(torch.from_numpy(out[qb]), ref, rtol=0, atol=1e-12)


def test_integer_weights_are_replication(oracle_mod):
    N, D = 5 * BLK - 37, 16
    q, k, v, NB = _case(4, H=1, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(4)
    lists = []
    for qb in range(NB):
        blocks = sorted(rng.choice(NB, size=rng.integers(1, NB + 1), replace=False).tolist())
        lists.append((blocks, rng.integers(1, 6, size=len(blocks)).astype(np.float32).tolist()))
    idx, cnt, w = _plan(NB, lists)
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=[(0, 0, qb) for qb in range(NB)], scale=scale)
    for qb, (blocks, weights) in enumerate(lists):
        rep = [j for j, c in zip(blocks, weights) for _ in range(int(c))]
        nq = min(BLK, N - qb * BLK)
        ref = _sdpa(q[0, 0, qb * BLK:qb * BLK + nq], _rows(k, 0, 0, rep, N), _rows(v, 0, 0, rep, N), scale)
        assert torch.allclose(_item_out(out, qb, qb, N), ref, rtol=0, atol=1e-12)


def test_uniform_weights_cancel(oracle_mod):
    """Equal weights over the kept list give plain block-sparse softmax attention."""
    N, D = 6 * BLK, 16
    q, k, v, NB = _case(5, H=1, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    lists = [([0, 3, 5], [7.5] * 3), ([1], [3.0]), ([0, 1, 2, 3, 4, 5], [2.0] * 6)] + [([qb], [1.0]) for qb in range(3, NB)]
    idx, cnt, w = _plan(NB, lists)
    out = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=[(0, 0, qb) for qb in range(NB)], scale=scale)
    for qb, (blocks, _) in enumerate(lists):
        ref = _sdpa(q[0, 0, qb * BLK:qb * BLK + BLK], _rows(k, 0, 0, blocks, N), _rows(v, 0, 0, blocks, N), scale)
        assert torch.allclose(torch.from_numpy(out[qb]), ref, rtol=0, atol=1e-12)


def test_shifted_numerator_and_denominator(oracle_mod):
    """With an explicit logit shift M, num/den are the shifted sums and out = num/den."""
    N, D = 2 * BLK, 16
    q, k, v, NB = _case(6, H=1, N=N, D=D)
    scale = 1.0 / np.sqrt(D)
    idx, cnt, w = _plan(NB, [([0, 1], [1.0, 2.0]), ([1], [4.0])])
    items = [(0, 0, 0), (0, 0, 1)]
    shift = np.full((2, BLK), 0.75)
    out, num, den = oracle_mod.attend(q, k, v, N, idx, cnt, w, items=items, scale=scale, shift=shift)
    assert np.allclose(out, num / den[..., None], rtol=1e-14, atol=0)
    # block weights multiply the shifted exponentials: compare against torch on replicated keys
    for it, rep in enumerate([[0, 1, 1], [1, 1, 1, 1]]):
        qq = q[0, 0, it * BLK:(it + 1) * BLK].double()
        kk, vv = _rows(k, 0, 0, rep, N).double(), _rows(v, 0, 0, rep, N).double()
        e = torch.exp(scale * qq @ kk.T - 0.75)
        assert torch.allclose(torch.from_numpy(den[it]), e.sum(1), rtol=1e-13, atol=0)
        assert torch.allclose(torch.from_numpy(num[it]), e @ vv, rtol=1e-12, atol=1e-13)
