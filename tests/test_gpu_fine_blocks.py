"""GPU parity with 4-token key blocks (the page's kernel paragraph: the unit of
selection is smaller than the compute tile, and kept blocks are gathered by
index into full matrix-core tiles).

Each stage is checked against the oracle with key blocks of 4 tokens, fed the
same inputs: pooling, scores (re-scored by the oracle from the GPU's own
centroids, weights and pooled keys), sampling (bit for bit from the GPU's
scores; rows of up to 32768 blocks exercise the long-row sampler), attention
(from the oracle's own lists), and the attention mass per 4-token block."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_38_amd import synth
from block_sparse_attention_38_amd.workloads import SINGLE, TINY, Workload

from parity_utils import (POOL_RTOL, SCORE_RTOL, check_attention, compare_lists, device, gpu_rows, inputs,
                          make_fine_plan, sample_items)

pytestmark = pytest.mark.gpu

FINE = 4
MASS_ATOL = 2e-5

RAGGED = Workload("ragged_bf16", 1, 3, 128, "bf16", (3, 10, 43), 16, (0.25,),
                  description="1290 tokens: 11 query blocks, 323 key blocks, the last with 2 valid tokens")
ONE_TAIL = Workload("one_token_tail", 1, 2, 128, "bf16", (1, 1, 257), 4, (0.5,),
                    description="257 tokens: the last key block holds a single token")
BATCH2 = Workload("batch2_bf16", 2, 2, 128, "bf16", (2, 9, 37), 16, (0.3,),
                  description="batch 2, 666 tokens: 6 query blocks (the last with 26 valid), 167 key blocks "
                              "(the last with 2 valid tokens)")
ONE_TOKEN = Workload("one_token", 1, 2, 128, "bf16", (1, 1, 1), 1, (0.5,), tiles=1,
                     description="a single token: one query block, one 4-token key block with one valid token")
SMALL = [TINY, RAGGED, ONE_TAIL, BATCH2, ONE_TOKEN]


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def _score_stage(aba, w, seed):
    (q, k, v), (qd, kd, vd) = inputs(w, seed)
    p = make_fine_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    torch.cuda.synchronize()
    return p, (q, k, v), (qd, kd, vd), s, cent, wgt, kbar


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fine_pool_and_scores_match_oracle(aba, w):
    p, (q, k, v), _, s, cent, wgt, kbar = _score_stage(aba, w, 201)
    assert s.shape == (w.batch, w.heads, w.n_blocks, w.n_fine_blocks)
    ref_kbar = oracle.pool(k, w.seq_len, blk=FINE)
    err = np.abs(kbar.cpu().double().numpy() - ref_kbar).max() / np.abs(ref_kbar).max()
    print(f"[{w.name}] fine pool: rel err {err:.3g}")
    assert err <= POOL_RTOL
    ref = oracle.score(cent.cpu().double().numpy(), wgt.cpu().double().numpy(), kbar.cpu().double().numpy(),
                       p.softmax_scale)
    got = s.cpu().double().numpy()
    rel = (np.abs(got - ref) / ref).max()
    print(f"[{w.name}] fine scores: max rel err {rel:.3g}; row sums {got.sum(-1).min():.6f}..{got.sum(-1).max():.6f}")
    assert rel <= SCORE_RTOL, f"score rel err {rel:.3g}"


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fine_sampling_bit_exact(aba, w):
    p, _, _, s, *_ = _score_stage(aba, w, 202)
    for seed in (0, 7, 0xDEADBEEFCAFEF00D):
        g = aba.sample(p, s, seed)
        torch.cuda.synchronize()
        o_idx, o_cnt, o_w, _ = oracle.sample(s.cpu().numpy(), p.budget, seed)
        assert compare_lists(*g, o_idx, o_cnt, o_w) == 0


@pytest.mark.parametrize("NB,K,peak", [(1025, 1, 3.0), (1025, 32, 30.0), (2000, 700, 1.0), (8190, 832, 4.0),
                                       (8190, 832, 0.3), (8190, 8190, 2.0), (8190, 9000, 2.0), (29700, 2368, 5.0),
                                       (32768, 2048, 8.0), (32768, 1, 0.5)])
def test_fine_sampling_bit_exact_on_long_rows(aba, NB, K, peak):
    """Rows longer than the short-row sampler holds: budgets of one, the page's
    4-token budgets, budgets at and beyond every block, the largest row."""
    p = aba.plan(1, 1, FINE * NB, 128, "bf16", 8, 10, K, key_block=FINE)
    NBq = p.n_blocks
    s = synth.random_scores(1, 1, NBq, NB, seed=NB + K, peak=peak)
    s[0, 0, 0, :] = 0.0                          # underflowed row: every sigma is 1
    if NBq > 1:
        s[0, 0, 1, :] = 1.0 / NB                 # exact ties everywhere
    if NBq > 2:
        s[0, 0, 2, : NB // 2] = 2.0 / NB         # two tie levels
        s[0, 0, 2, NB // 2:] = 0.0
    if NBq > 3:
        s[0, 0, 3, :] = 0.0
        s[0, 0, 3, ::97] = 1.0                   # a few blocks that all cap
    g = aba.sample(p, s.to(device()), 1234)
    torch.cuda.synchronize()
    o_idx, o_cnt, o_w, theta = oracle.sample(s.numpy(), K, 1234)
    assert compare_lists(*g, o_idx, o_cnt, o_w) == 0
    if 1 < K < NB:
        # rows where only the top block is forced (the two-key test) and rows with
        # a longer capped top (the gathered, sorted top) both occur
        t = (theta == 2**32).sum(axis=-1)
        assert (t == 1).any() and (t > 1).any()
    print(f"[long rows NB={NB} K={K}] {NBq} rows bit-exact; mean kept {o_cnt.mean():.1f}")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fine_attend_matches_oracle_on_oracle_lists(aba, w):
    (q, k, v), (qd, kd, vd) = inputs(w, 203)
    p = make_fine_plan(aba, w)
    NBk = p.n_key_blocks
    scores = synth.random_scores(w.batch, w.heads, w.n_blocks, NBk, seed=6, peak=2.0)
    idx, cnt, wt, _ = oracle.sample(scores.numpy(), p.budget, 13)
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (idx, cnt, wt)))
    torch.cuda.synchronize()
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, idx, cnt, wt, items=items, scale=p.softmax_scale, kblk=FINE)
    err = check_attention(gpu_rows(out, items), ref, w.dtype, "fine_attend_matches_oracle_on_oracle_lists")
    print(f"[{w.name}] fine attend: max abs err {err:.3g}; kept blocks per row {cnt.mean():.1f} of {NBk}")
    assert torch.all(out[:, :, w.seq_len:] == 0)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fine_attend_empty_lists_give_zeros(aba, w):
    """4-token lists: a query block with nothing to attend (cnt 0, a negative cnt,
    or only invalid entries) gets zeros; every other row still matches the oracle."""
    (q, k, v), (qd, kd, vd) = inputs(w, 208)
    p = make_fine_plan(aba, w)
    NB, NBk = w.n_blocks, p.n_key_blocks
    scores = synth.random_scores(w.batch, w.heads, NB, NBk, seed=10, peak=2.0)
    idx, cnt, wt, _ = oracle.sample(scores.numpy(), p.budget, 17)
    idx, cnt, wt = idx.copy(), cnt.copy(), wt.copy()
    empty = [(0, 0, 0), (w.batch - 1, w.heads - 1, NB - 1), (0, w.heads - 1, NB // 2)]
    cnt[empty[0]] = 0
    cnt[empty[1]] = -3
    idx[empty[2]] = NBk + 7                # every entry past the last key block
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
                        scale=p.softmax_scale, kblk=FINE)
    check_attention(got[~is_empty], ref, w.dtype, "fine_attend_empty_lists_give_zeros")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fine_every_block_kept_is_dense(aba, w):
    """A budget of every block caps them all (weight 1): the layer is dense attention."""
    (q, k, v), (qd, kd, vd) = inputs(w, 204)
    p = make_fine_plan(aba, w, budget=w.n_fine_blocks)
    s = aba.score(p, qd, kd)
    idx, cnt, wt = aba.sample(p, s, 3)
    out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
    torch.cuda.synchronize()
    assert torch.all(cnt == w.n_fine_blocks) and torch.all(wt == 1.0)
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend_full(q, k, v, w.seq_len, items=items, scale=p.softmax_scale)
    err = check_attention(gpu_rows(out, items), ref, w.dtype, "fine_every_block_kept_is_dense")
    print(f"[{w.name}] fine, every block kept vs dense: max abs err {err:.3g}")


@pytest.mark.parametrize("w", [TINY, RAGGED], ids=lambda w: w.name)
def test_fine_attend_skips_malformed_list_entries(aba, w):
    """Entries outside [0, NBk), weights that are not positive and finite, and cnt
    beyond the capacity are ignored; whole 16-entry groups of invalid entries too."""
    (q, k, v), (qd, kd, vd) = inputs(w, 205)
    p = make_fine_plan(aba, w)
    NBk, cap = p.n_key_blocks, p.list_cap
    scores = synth.random_scores(w.batch, w.heads, w.n_blocks, NBk, seed=7, peak=1.0)
    idx, cnt, wt, _ = oracle.sample(scores.numpy(), p.budget, 17)
    bad_idx, bad_cnt, bad_w = idx.copy(), cnt.copy(), wt.copy()
    rng = np.random.default_rng(5)
    for r in np.ndindex(*cnt.shape):
        c = int(cnt[r])
        for e in rng.choice(c, size=min(c, 6), replace=False):
            kind = rng.integers(4)
            if kind == 0:
                bad_idx[r + (e,)] = -1 - int(rng.integers(5))
            elif kind == 1:
                bad_idx[r + (e,)] = NBk + int(rng.integers(5))
            elif kind == 2:
                bad_w[r + (e,)] = 0.0
            else:
                bad_w[r + (e,)] = np.inf
    b0 = (0, 0, 0)
    c0 = int(cnt[b0])
    if c0 > 40:   # a whole sub-tile of invalid entries in the middle of a list
        bad_idx[b0 + (slice(16, 32),)] = -7
    bad_cnt[0, 0, 1] = cap + 1000               # beyond the capacity: clamped
    clean_idx = np.zeros_like(idx)
    clean_w = np.zeros_like(wt)
    clean_cnt = np.zeros_like(cnt)
    for r in np.ndindex(*cnt.shape):
        c = min(int(bad_cnt[r]), cap)
        keep = [(j, x) for j, x in zip(bad_idx[r][:c], bad_w[r][:c]) if 0 <= j < NBk and 0 < x < np.inf]
        clean_cnt[r] = len(keep)
        for e, (j, x) in enumerate(keep):
            clean_idx[r + (e,)] = j
            clean_w[r + (e,)] = x
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (bad_idx, bad_cnt, bad_w)))
    torch.cuda.synchronize()
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, clean_idx, clean_cnt, clean_w, items=items, scale=p.softmax_scale,
                        kblk=FINE)
    err = check_attention(gpu_rows(out, items), ref, w.dtype, "fine_attend_skips_malformed_list_entries")
    print(f"[{w.name}] fine attend with malformed entries: max abs err {err:.3g}")


def test_fine_full_pipeline_tiny_stagewise(aba):
    w = TINY
    (q, k, v), (qd, kd, vd) = inputs(w, 1000)
    p = make_fine_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    idx, cnt, wt = aba.sample(p, s, 7)
    out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
    torch.cuda.synchronize()
    o_idx, o_cnt, o_w, _ = oracle.sample(s.cpu().numpy(), p.budget, 7)
    assert compare_lists(idx, cnt, wt, o_idx, o_cnt, o_w) == 0
    items = oracle.layer_items(1, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, o_idx, o_cnt, o_w, items=items, scale=p.softmax_scale, kblk=FINE)
    check_attention(gpu_rows(out, items), ref, w.dtype, "fine_full_pipeline_tiny_stagewise")


@pytest.mark.parametrize("w", [RAGGED, ONE_TAIL], ids=lambda w: w.name)
def test_fine_block_mass_matches_oracle(aba, w):
    (q, k, _), (qd, kd, _) = inputs(w, 206)
    p = make_fine_plan(aba, w)
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    got = aba.block_mass(p, qd, kd, items).cpu().double().numpy()
    ref = oracle.block_mass(q, k, w.seq_len, items=items, scale=p.softmax_scale, kblk=FINE)
    assert got.shape == ref.shape == (len(items), w.n_fine_blocks)
    err = np.abs(got - ref).max()
    print(f"[{w.name}] fine block mass: max abs err {err:.3g}")
    assert err <= MASS_ATOL
    assert np.allclose(got.sum(1), 1.0, atol=1e-4)


# ---------------------------------------------------------------------------
# The 32K-token single layer with 4-token key blocks, as the benchmark runs it
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def single_fine(aba):
    w = SINGLE
    (q, k, v), (qd, kd, vd) = inputs(w, 1001)
    p = make_fine_plan(aba, w)
    s, cent, wgt, kbar = aba.score(p, qd, kd, return_parts=True)
    idx, cnt, wt = aba.sample(p, s, 7)
    out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
    torch.cuda.synchronize()
    return dict(w=w, p=p, cpu=(q, k, v), gpu=(qd, kd, vd), s=s, cent=cent, wgt=wgt, kbar=kbar, idx=idx, cnt=cnt,
                wt=wt, out=out)


def test_single_layer_fine_pool_scores_and_sampling(aba, single_fine):
    L, w, p = single_fine, SINGLE, single_fine["p"]
    k = L["cpu"][1]
    ref_kbar = oracle.pool(k, w.seq_len, blk=FINE)
    assert np.abs(L["kbar"].cpu().double().numpy() - ref_kbar).max() <= POOL_RTOL * np.abs(ref_kbar).max()
    items = sample_items(w, 24, seed=4)
    cent = L["cent"].cpu().double().numpy()
    wgt = L["wgt"].cpu().double().numpy()
    kbar = L["kbar"].cpu().double().numpy()
    got = L["s"].cpu().double().numpy()
    worst = 0.0
    for b, h, qb in items:   # the oracle re-scores one query block at a time
        ref = oracle.score(cent[b:b + 1, h:h + 1, qb:qb + 1], wgt[b:b + 1, h:h + 1, qb:qb + 1],
                           kbar[b:b + 1, h:h + 1], p.softmax_scale)[0, 0, 0]
        worst = max(worst, (np.abs(got[b, h, qb] - ref) / ref).max())
    print(f"[single fine] scores: {len(items)} rows of {got.shape[-1]}, max rel err {worst:.3g}")
    assert worst <= SCORE_RTOL
    o_idx, o_cnt, o_w, _ = oracle.sample(L["s"].cpu().numpy(), p.budget, 7)
    assert compare_lists(L["idx"], L["cnt"], L["wt"], o_idx, o_cnt, o_w) == 0
    kept = L["cnt"].float().mean().item()
    print(f"[single fine] lists bit-exact over {o_cnt.size} rows; mean kept {kept:.1f} of {p.n_key_blocks} "
          f"(budget {p.budget})")
    assert abs(kept - p.budget) < 0.05 * p.budget


def test_single_layer_fine_attention_sampled(aba, single_fine):
    L, w, p = single_fine, SINGLE, single_fine["p"]
    q, k, v = L["cpu"]
    items = sample_items(w, 16, seed=5)
    idx, cnt, wt = (x.cpu().numpy() for x in (L["idx"], L["cnt"], L["wt"]))
    ref = oracle.attend(q, k, v, w.seq_len, idx, cnt, wt, items=items, scale=p.softmax_scale, kblk=FINE)
    err = check_attention(gpu_rows(L["out"], items), ref, w.dtype, "single_layer_fine_attention_sampled")
    print(f"[single fine] attend: {len(items)} query blocks, max abs err {err:.3g}")


@pytest.mark.parametrize("key_block,n_tokens,heads", [(4, 2048, 2), (4, 2049, 2), (4, 2052, 2), (128, 65536, 1),
                                                      (128, 65409, 1), (128, 65664, 1), (128, 131072, 1)])
def test_scores_at_the_one_pass_limit(aba, key_block, n_tokens, heads):
    """Rows of exactly 512 key blocks take the one-pass scorer with its largest LDS
    rows; 513 or more take the two-pass scorer (up to the largest 128-token row,
    1024 blocks); both against the oracle, re-scored from the GPU's own centroids,
    weights and pooled keys."""
    g = torch.Generator().manual_seed(n_tokens + key_block)
    NB = (n_tokens + 127) // 128
    shape = (1, heads, 128 * NB, 128)
    centres = torch.randn(heads, 16, 128, generator=g)
    z = torch.randint(0, 16, (n_tokens,), generator=g)
    base = torch.zeros(shape)
    base[0, :, :n_tokens] = centres[:, z, :]
    q = (base + 0.5 * torch.randn(shape, generator=g)).to(torch.bfloat16)
    k = (base + torch.randn(shape, generator=g)).to(torch.bfloat16)
    q[0, :, n_tokens:] = 0
    k[0, :, n_tokens:] = 0
    p = aba.plan(1, heads, n_tokens, 128, "bf16", 8, 10, 8, key_block=key_block)
    NBk = p.n_key_blocks
    assert NBk == (n_tokens + key_block - 1) // key_block
    s, cent, wgt, kbar = aba.score(p, q.to(device()), k.to(device()), return_parts=True)
    torch.cuda.synchronize()
    ref = oracle.score(cent.cpu().double().numpy(), wgt.cpu().double().numpy(), kbar.cpu().double().numpy(),
                       p.softmax_scale)
    got = s.cpu().double().numpy()
    rel = (np.abs(got - ref) / ref).max()
    sums = got.sum(-1)
    print(f"[one-pass limit kb={key_block} N={n_tokens} NBk={NBk}] max rel err {rel:.3g}; "
          f"row sums {sums.min():.6f}..{sums.max():.6f}")
    assert rel <= SCORE_RTOL
    ref_kbar = oracle.pool(k.float().numpy(), n_tokens, blk=key_block)
    assert np.abs(kbar.cpu().double().numpy() - ref_kbar).max() / np.abs(ref_kbar).max() <= POOL_RTOL
