"""GPU parity on peaked attention, where the comparison can fail.

The synthetic layers give nearly flat attention (outputs of a few 1e-2), so the
peaked variant runs the same inputs with the softmax scale 1 instead of
1/sqrt(D) (logits x sqrt(D)): a row's logits span ~100 log2 units and the
outputs are O(1).  The lists carry Horvitz-Thompson weights of 2^0..2^4 on their
first half and 2^16..2^20 on their second (the SIP paragraph of the
AB-Attention page: a block's weight enters numerator and normaliser as a logit
shift), so the shifted logits jump upward part-way through every list.  Each
case also emulates, on its inputs, the kernels' lazy rescale and asserts that it
runs after the first sub-tile, so the rescale path is exercised, not only the
first-tile path.  Both key block sizes, the small ragged layers and the 32K-token
layer in the benchmark's launch configuration.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_38_amd.workloads import SINGLE, TINY, Workload

from parity_utils import (PEAKED_SCALE, check_attention, device, gpu_rows, inputs, peaked_lists,
                          rescales_after_first_subtile, sample_items)

pytestmark = pytest.mark.gpu

RAGGED = Workload("ragged_bf16", 1, 3, 128, "bf16", (3, 10, 43), 16, (0.25,),
                  description="1290 tokens: 11 blocks, the last with 10 valid")
RAGGED64 = Workload("ragged_bf16_d64", 2, 2, 64, "bf16", (2, 9, 50), 16, (0.3,),
                    description="batch 2, 900 tokens: 8 blocks, the last with 4 valid")
ONE_TAIL = Workload("one_token_tail", 1, 2, 128, "bf16", (1, 1, 257), 4, (0.5,),
                    description="257 tokens: the last block holds a single token")


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def _plan(aba, w, key_block, budget):
    return aba.plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, 8, 10, budget, softmax_scale=PEAKED_SCALE,
                    key_block=key_block)


def _run_lists(aba, w, key_block, per_row, seed, items=None):
    (q, k, v), (qd, kd, vd) = inputs(w, seed)
    NBk = w.n_blocks if key_block == 128 else w.n_fine_blocks
    p = _plan(aba, w, key_block, min(per_row, NBk))
    idx, cnt, wt = peaked_lists(w.batch, w.heads, w.n_blocks, NBk, per_row, seed=seed + 1)
    out = aba.attend(p, qd, kd, vd, *(torch.from_numpy(a).to(device()) for a in (idx, cnt, wt)))
    torch.cuda.synchronize()
    if items is None:
        items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend(q, k, v, w.seq_len, idx, cnt, wt, items=items, scale=PEAKED_SCALE, kblk=key_block)
    label = f"{w.name} peaked, {key_block}-token key blocks"
    check_attention(gpu_rows(out, items), ref, w.dtype, label)
    scale = float(np.abs(ref).max())
    n = rescales_after_first_subtile(q, k, w.seq_len, items, idx, cnt, wt, PEAKED_SCALE, key_block)
    print(f"[{label}] output scale {scale:.3g}; rescales after the first sub-tile: {n}")
    assert scale > 0.5, "peaked attention should give O(1) outputs"
    assert n > 0, "the case must drive the lazy rescale past the first sub-tile"
    assert torch.all(out[:, :, w.seq_len:] == 0)


@pytest.mark.parametrize("w", [TINY, RAGGED, RAGGED64, ONE_TAIL], ids=lambda w: w.name)
def test_peaked_attention_128_token_blocks(aba, w):
    _run_lists(aba, w, 128, per_row=6, seed=301)


@pytest.mark.parametrize("w,per_row", [(TINY, 64), (RAGGED, 64), (ONE_TAIL, 48)], ids=lambda x: getattr(x, "name", ""))
def test_peaked_attention_4_token_blocks(aba, w, per_row):
    _run_lists(aba, w, 4, per_row=per_row, seed=311)


def test_peaked_attention_single_layer_sampled(aba):
    """The whole 32K-token layer launched with peaked lists of the benchmark's size
    (26 blocks per query block); 24 sampled query blocks compared, the ragged last
    one included."""
    w = SINGLE
    _run_lists(aba, w, 128, per_row=w.budget(), seed=321, items=sample_items(w, 22, seed=31))


def test_peaked_attention_single_layer_4_token_sampled(aba):
    w = SINGLE
    _run_lists(aba, w, 4, per_row=w.fine_budget(), seed=331, items=sample_items(w, 14, seed=33))


def _dense(aba, w, seed, items=None):
    (q, k, v), (qd, kd, vd) = inputs(w, seed)
    p = _plan(aba, w, 128, 1)
    out = aba.attend_full(p, qd, kd, vd)
    torch.cuda.synchronize()
    if items is None:
        items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    ref = oracle.attend_full(q, k, v, w.seq_len, items=items, scale=PEAKED_SCALE)
    check_attention(gpu_rows(out, items), ref, w.dtype, f"{w.name} peaked dense")
    NB = w.n_blocks
    idx = np.broadcast_to(np.arange(NB, dtype=np.int32), (w.batch, w.heads, NB, NB))
    cnt = np.full((w.batch, w.heads, NB), NB, np.int32)
    wt = np.ones((w.batch, w.heads, NB, NB), np.float32)
    n = rescales_after_first_subtile(q, k, w.seq_len, items, idx, cnt, wt, PEAKED_SCALE, 128)
    print(f"[{w.name} peaked dense] output scale {np.abs(ref).max():.3g}; rescales after the first sub-tile: {n}")
    assert np.abs(ref).max() > 0.5
    assert n > 0


@pytest.mark.parametrize("w", [TINY, RAGGED, RAGGED64, ONE_TAIL], ids=lambda w: w.name)
def test_peaked_dense_small(aba, w):
    _dense(aba, w, 341)


def test_peaked_dense_single_layer_sampled(aba):
    w = SINGLE
    _dense(aba, w, 351, items=sample_items(w, 3, seed=35))
