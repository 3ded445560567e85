"""GPU parity: every HIP stage against the CPU oracle on the same seeded inputs.

Stages are compared one at a time, each fed identical inputs, so errors do not
compound: k-means (centroids and weights), key pooling, scores (re-scored by the
oracle from the GPU's own centroids, weights and pooled keys), sampling (bit for
bit from the GPU's scores and the same seed), attention (from the oracle's own
lists), and dense attention.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_38_amd import synth
from block_sparse_attention_38_amd.workloads import SINGLE, TINY, Workload

from parity_utils import (CENT_RTOL, NEAR_TIE, POOL_RTOL, SCORE_RTOL, check_attention, compare_lists, device,
                          gpu_rows, inputs, make_plan, sample_items)

pytestmark = pytest.mark.gpu

# Small layers that still span several tiles and end in a ragged block.
RAGGED = Workload("ragged_bf16", 1, 3, 128, "bf16", (3, 10, 43), 16, (0.25,),
                  description="1290 tokens: 11 blocks, the last with 10 valid")
RAGGED64 = Workload("ragged_bf16_d64", 2, 2, 64, "bf16", (2, 9, 50), 16, (0.3,),
                    description="batch 2, 900 tokens: 8 blocks, the last with 4 valid")
ONE_TAIL = Workload("one_token_tail", 1, 2, 128, "bf16", (1, 1, 257), 4, (0.5,),
                    description="257 tokens: the last block holds a single token")
BATCH2 = Workload("batch2_bf16", 2, 2, 128, "bf16", (2, 9, 37), 16, (0.3,),
                  description="batch 2, head_dim 128, 666 tokens: 6 blocks, the last with 26 valid")
ONE_TOKEN = Workload("one_token", 1, 2, 128, "bf16", (1, 1, 1), 1, (0.5,), tiles=1,
                     description="a single token: one query block (one row, fewer than clusters), one key block")
SMALL = [TINY, RAGGED, RAGGED64, ONE_TAIL, BATCH2, ONE_TOKEN]


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def _score_stage(aba, w, seed):
    (q, k, v), (qd, kd, vd) = inputs(w, seed)
    p = make_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    torch.cuda.synchronize()
    return p, (q, k, v), (qd, kd, vd), s, cent, wgt, kbar


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_kmeans_matches_oracle(aba, w):
    p, (q, k, v), _, s, cent, wgt, kbar = _score_stage(aba, w, seed=101)
    o_cent, o_w, gap = oracle.kmeans(q, w.seq_len, C=p.n_clusters, T=p.kmeans_iters)
    g_cent, g_w = cent.cpu().numpy().astype(np.float64), wgt.cpu().numpy()
    ok = gap >= NEAR_TIE
    assert ok.mean() > 0.5, f"too many near-tie blocks ({(~ok).sum()} of {ok.size})"
    if 0 < w.seq_len % 128 < p.n_clusters:
        # a last block with fewer rows than clusters starts from repeated rows,
        # whose copies tie exactly: it is compared like any other
        assert ok[..., -1].all()
    scale = np.abs(o_cent).max(axis=(-1, -2), keepdims=True)
    err = (np.abs(g_cent - o_cent) / scale).max(axis=(-1, -2))
    print(f"[{w.name}] kmeans: {ok.sum()}/{ok.size} blocks compared, centroid rel err {err[ok].max():.3g}")
    assert err[ok].max() <= CENT_RTOL, f"centroid rel err {err[ok].max():.3g}"
    assert np.array_equal(g_w[ok].view(np.uint32), o_w[ok].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_pool_matches_oracle(aba, w):
    p, (q, k, v), _, s, cent, wgt, kbar = _score_stage(aba, w, seed=102)
    ref = oracle.pool(k, w.seq_len)
    got = kbar.cpu().numpy().astype(np.float64)
    print(f"[{w.name}] pool: rel err {np.abs(got - ref).max() / np.abs(ref).max():.3g}")
    assert np.abs(got - ref).max() <= POOL_RTOL * np.abs(ref).max()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_scores_match_oracle_from_gpu_parts(aba, w):
    p, _, _, s, cent, wgt, kbar = _score_stage(aba, w, seed=103)
    ref = oracle.score(cent.cpu().double().numpy(), wgt.cpu().double().numpy(), kbar.cpu().double().numpy(),
                       p.softmax_scale)
    got = s.cpu().numpy().astype(np.float64)
    rel = np.abs(got - ref) / np.abs(ref)
    print(f"[{w.name}] scores: max rel err {rel.max():.3g}")
    assert rel.max() <= SCORE_RTOL, f"score rel err {rel.max():.3g}"
    assert np.allclose(got.sum(-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_sampling_bit_exact(aba, w):
    p, _, _, s, *_ = _score_stage(aba, w, seed=104)
    for seed in (0, 7, 0xDEADBEEFCAFEF00D):
        g = aba.sample(p, s, seed)
        torch.cuda.synchronize()
        o_idx, o_cnt, o_w, _ = oracle.sample(s.cpu().numpy(), p.budget, seed)
        assert compare_lists(*g, o_idx, o_cnt, o_w) == 0


@pytest.mark.parametrize("NB,K,peak", [(8, 1, 3.0), (8, 8, 3.0), (8, 20, 3.0), (256, 26, 5.0), (929, 74, 8.0),
                                       (1024, 100, 2.0), (37, 5, 30.0)])
def test_sampling_bit_exact_on_varied_rows(aba, NB, K, peak):
    """Sharp and flat rows, budgets of one and beyond every block, the largest block count."""
    p = aba.plan(1, 2, NB * 128, 128, "bf16", 8, 10, K)
    s = synth.random_scores(1, 2, NB, NB, seed=NB + K, peak=peak)
    s[0, 0, 0, :] = 0.0                    # underflowed row: every sigma is 1
    s[0, 1, 0, :] = 1.0 / NB               # exact ties everywhere
    sd = s.to(device())
    g = aba.sample(p, sd, 99)
    torch.cuda.synchronize()
    o_idx, o_cnt, o_w, theta = oracle.sample(s.numpy(), K, 99)
    assert compare_lists(*g, o_idx, o_cnt, o_w) == 0
    if 1 < K < NB and NB != 8:
        # both ways of finding the stopping point t (the first t blocks capped) run:
        # rows where only the top block is forced and rows with a longer capped top
        t = (theta == 2**32).sum(axis=-1)
        assert (t == 1).any() and (t > 1).any()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_attend_matches_oracle_on_oracle_lists(aba, w):
    (q, k, v), (qd, kd, vd) = inputs(w, 105)
    p = make_plan(aba, w)
    scores = synth.random_scores(w.batch, w.heads, w.n_blocks, w.n_blocks, seed=5, peak=2.0)
    idx, cnt, wt, _ = oracle.sample(scores.numpy(), p.budget, 11)
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (idx, cnt, wt)))
    torch.cuda.synchronize()
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, idx, cnt, wt, items=items, scale=p.softmax_scale)
    err = check_attention(gpu_rows(out, items), ref, w.dtype, "attend_matches_oracle_on_oracle_lists")
    print(f"[{w.name}] attend: max abs err {err:.3g} (mean |out| {np.abs(ref).mean():.3g})")
    assert torch.all(out[:, :, w.seq_len:] == 0)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_attend_empty_lists_give_zeros(aba, w):
    """A query block with nothing to attend (cnt 0, a negative cnt, or only invalid
    entries) gets zeros, the call's stated convention (the attention formula is 0/0
    there); every other row still matches the oracle."""
    (q, k, v), (qd, kd, vd) = inputs(w, 108)
    p = make_plan(aba, w)
    NB = w.n_blocks
    scores = synth.random_scores(w.batch, w.heads, NB, NB, seed=9, peak=2.0)
    idx, cnt, wt, _ = oracle.sample(scores.numpy(), p.budget, 13)
    idx, cnt, wt = idx.copy(), cnt.copy(), wt.copy()
    empty = [(0, 0, 0), (w.batch - 1, w.heads - 1, NB - 1), (0, w.heads - 1, NB // 2)]
    cnt[empty[0]] = 0
    cnt[empty[1]] = -3
    idx[empty[2]] = -1                     # every entry invalid
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (idx, cnt, wt)))
    torch.cuda.synchronize()
    clean_cnt = cnt.copy()
    for e in empty:
        clean_cnt[e] = 0
    items = oracle.layer_items(w.batch, w.heads, NB)
    got = gpu_rows(out, items)
    is_empty = np.array([it in empty for it in items])
    assert np.all(got[is_empty] == 0.0)
    ref = oracle.attend(q, k, v, w.seq_len, idx, clean_cnt, wt, items=[it for it in items if it not in empty],
                        scale=p.softmax_scale)
    check_attention(got[~is_empty], ref, w.dtype, "attend_empty_lists_give_zeros")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_attend_full_matches_oracle(aba, w):
    (q, k, v), (qd, kd, vd) = inputs(w, 106)
    p = make_plan(aba, w)
    out = aba.attend_full(p, qd, kd, vd)
    torch.cuda.synchronize()
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend_full(q, k, v, w.seq_len, items=items, scale=p.softmax_scale)
    err = check_attention(gpu_rows(out, items), ref, w.dtype, "attend_full_matches_oracle")
    print(f"[{w.name}] attend_full: max abs err {err:.3g}")


def test_attend_skips_malformed_list_entries(aba):
    """Entries outside [0, NB), weights <= 0 and cnt beyond the capacity are ignored."""
    w = RAGGED
    (q, k, v), (qd, kd, vd) = inputs(w, 107)
    p = make_plan(aba, w)
    NB = w.n_blocks
    idx = np.zeros((1, w.heads, NB, NB), np.int32)
    wt = np.ones((1, w.heads, NB, NB), np.float32)
    cnt = np.full((1, w.heads, NB), 4, np.int32)
    idx[..., :4] = [1, NB + 3, -2, NB - 1]
    wt[..., 3] = 2.5
    wt[0, 0, 0, 0] = 0.0                   # zero weight: skipped
    cnt[0, 1, 1] = NB + 50                 # clamped to the capacity (entries past 4 are block 0, weight 1)
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (idx, cnt, wt)))
    torch.cuda.synchronize()
    clean_idx = np.zeros_like(idx)
    clean_w = np.ones_like(wt)
    clean_cnt = np.zeros_like(cnt)
    for h in range(w.heads):
        for qb in range(NB):
            c = min(int(cnt[0, h, qb]), NB)
            keep = [(j, x) for j, x in zip(idx[0, h, qb, :c], wt[0, h, qb, :c]) if 0 <= j < NB and x > 0]
            clean_cnt[0, h, qb] = len(keep)
            for e, (j, x) in enumerate(keep):
                clean_idx[0, h, qb, e], clean_w[0, h, qb, e] = j, x
    items = oracle.layer_items(1, w.heads, NB)
    ref = oracle.attend(q, k, v, w.seq_len, clean_idx, clean_cnt, clean_w, items=items, scale=p.softmax_scale)
    check_attention(gpu_rows(out, items), ref, w.dtype, "attend_skips_malformed_list_entries")


@pytest.mark.parametrize("w", [RAGGED, BATCH2], ids=lambda w: w.name)
def test_every_block_kept_equals_dense(aba, w):
    """Budget >= NB: every inclusion probability is 1 and sparse attention is dense attention
    (an odd number of query blocks per head: one query block per dense workgroup; an even
    number, batch 2: two per workgroup)."""
    (q, k, v), (qd, kd, vd) = inputs(w, 108)
    p = make_plan(aba, w, budget=w.n_blocks)
    out, (s, idx, cnt, wt) = aba.layer(p, qd, kd, vd, seed=3)
    dense = aba.attend_full(p, qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.all(cnt == w.n_blocks) and torch.all(wt == 1.0)
    assert (out.float() - dense.float()).abs().max().item() <= 1e-2


def test_layer_is_deterministic(aba):
    w = RAGGED
    _, (qd, kd, vd) = inputs(w, 109)
    p = make_plan(aba, w)
    a = aba.layer(p, qd, kd, vd, seed=5)
    b = aba.layer(p, qd, kd, vd, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    (sa, ia, ca, wa), (sb, ib, cb, wb) = a[1], b[1]
    assert torch.equal(sa, sb)
    # list entries at or past cnt are unspecified; the kept prefix must agree bit for bit
    assert compare_lists(ia, ca, wa, ib.cpu().numpy(), cb.cpu().numpy(), wb.cpu().numpy()) == 0


def test_full_pipeline_tiny_stagewise(aba):
    """The whole layer on the fp32 workload, each stage checked against the oracle."""
    w = TINY
    (q, k, v), (qd, kd, vd) = inputs(w, 1000)
    p = make_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    idx, cnt, wt = aba.sample(p, s, 7)
    out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
    torch.cuda.synchronize()
    o_idx, o_cnt, o_w, _ = oracle.sample(s.cpu().numpy(), p.budget, 7)
    assert compare_lists(idx, cnt, wt, o_idx, o_cnt, o_w) == 0
    items = oracle.layer_items(1, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, o_idx, o_cnt, o_w, items=items, scale=p.softmax_scale)
    check_attention(gpu_rows(out, items), ref, w.dtype, "full_pipeline_tiny_stagewise")


# ---------------------------------------------------------------------------
# The 32K-token single layer, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def single(aba):
    w = SINGLE
    (q, k, v), (qd, kd, vd) = inputs(w, 1001)
    p = make_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    idx, cnt, wt = aba.sample(p, s, 7)
    out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
    torch.cuda.synchronize()
    return dict(w=w, p=p, cpu=(q, k, v), gpu=(qd, kd, vd), s=s, cent=cent, wgt=wgt, kbar=kbar, idx=idx, cnt=cnt,
                wt=wt, out=out)


def test_single_layer_scores_pool_and_sampling(aba, single):
    w, p = single["w"], single["p"]
    q, k, v = single["cpu"]
    ref_kbar = oracle.pool(k, w.seq_len)
    assert np.abs(single["kbar"].cpu().double().numpy() - ref_kbar).max() <= POOL_RTOL * np.abs(ref_kbar).max()
    ref = oracle.score(single["cent"].cpu().double().numpy(), single["wgt"].cpu().double().numpy(),
                       single["kbar"].cpu().double().numpy(), p.softmax_scale)
    got = single["s"].cpu().double().numpy()
    print(f"[single] scores: max rel err {(np.abs(got - ref) / ref).max():.3g}")
    assert (np.abs(got - ref) / ref).max() <= SCORE_RTOL
    o_idx, o_cnt, o_w, _ = oracle.sample(single["s"].cpu().numpy(), p.budget, 7)
    assert compare_lists(single["idx"], single["cnt"], single["wt"], o_idx, o_cnt, o_w) == 0
    density = single["cnt"].float().mean().item() / w.n_blocks
    print(f"[single] lists bit-exact over {o_cnt.size} rows; realised density {density:.4f}")
    assert abs(density - p.budget / w.n_blocks) < 0.02


def test_single_layer_kmeans_sampled(aba, single):
    w, p = single["w"], single["p"]
    q = single["cpu"][0]
    items = sample_items(w, 40, seed=1)
    g_cent = single["cent"].cpu().double().numpy()
    g_w = single["wgt"].cpu().numpy()
    compared = 0
    for b, h, qb in items:
        n = min(128, w.seq_len - qb * 128)
        cent, wt, _, gap = oracle.kmeans_block(q[b, h, qb * 128:qb * 128 + n], C=p.n_clusters, T=p.kmeans_iters)
        if gap < NEAR_TIE:
            continue
        assert np.abs(g_cent[b, h, qb] - cent).max() <= CENT_RTOL * np.abs(cent).max()
        assert np.array_equal(g_w[b, h, qb].view(np.uint32), wt.astype(np.float32).view(np.uint32))
        compared += 1
    print(f"[single] kmeans: {compared}/{len(items)} sampled blocks compared")
    assert compared >= len(items) // 2


def test_single_layer_attention_sampled(aba, single):
    w, p = single["w"], single["p"]
    q, k, v = single["cpu"]
    items = sample_items(w, 32, seed=2)
    idx, cnt, wt = (x.cpu().numpy() for x in (single["idx"], single["cnt"], single["wt"]))
    ref = oracle.attend(q, k, v, w.seq_len, idx, cnt, wt, items=items, scale=p.softmax_scale)
    err = check_attention(gpu_rows(single["out"], items), ref, w.dtype, "single_layer_attention_sampled")
    print(f"[single] attend: {len(items)} query blocks, max abs err {err:.3g}")


def test_single_layer_dense_sampled(aba, single):
    w, p = single["w"], single["p"]
    q, k, v = single["cpu"]
    qd, kd, vd = single["gpu"]
    dense = aba.attend_full(p, qd, kd, vd)
    torch.cuda.synchronize()
    items = sample_items(w, 6, seed=3)
    ref = oracle.attend_full(q, k, v, w.seq_len, items=items, scale=p.softmax_scale)
    err = check_attention(gpu_rows(dense, items), ref, w.dtype, "single_layer_dense_sampled")
    print(f"[single] attend_full: {len(items)} query blocks, max abs err {err:.3g}")


@pytest.mark.parametrize("w", [RAGGED, BATCH2], ids=lambda w: w.name)
@pytest.mark.parametrize("key_block", [128, 4])
def test_padding_rows_are_ignored(aba, key_block, w):
    """Rows >= N of q, k and v may hold anything (NaN, inf, huge values): scores,
    lists, sparse and dense outputs are bitwise those of zero padding (both dense
    workgroup shapes: an odd and an even number of query blocks per head)."""
    (q, k, v), (qd, kd, vd) = inputs(w, 17)
    N = w.seq_len
    p = aba.plan(w.batch, w.heads, N, w.head_dim, w.dtype, 8, 10, w.budget() if key_block == 128 else 64,
                 key_block=key_block)

    def run(qx, kx, vx):
        s = aba.score(p, qx, kx)
        lists = aba.sample(p, s, 5)
        o = aba.attend(p, qx, kx, vx, *lists)
        of = aba.attend_full(p, qx, kx, vx)
        torch.cuda.synchronize()
        return [x.cpu() for x in (s, *lists, o, of)]

    clean = run(qd, kd, vd)
    dirty = []
    for x in (qd, kd, vd):
        y = x.clone()
        y[:, :, N:] = float("nan")
        y[:, :, N::2] = float("inf")
        y[:, 1:, N:] = -3.0e38
        dirty.append(y)
    got = run(*dirty)
    names = ("scores", "idx", "cnt", "w", "attend", "attend_full")
    for name, a, b in zip(names, clean, got):
        if name == "idx" or name == "w":   # entries past cnt are unspecified
            cnt = clean[2]
            for r in np.ndindex(*cnt.shape):
                n = int(cnt[r])
                assert torch.equal(a[r][:n], b[r][:n]), f"{name} differs in row {r}"
            continue
        assert torch.equal(a, b), f"{name} differs with garbage padding rows"
