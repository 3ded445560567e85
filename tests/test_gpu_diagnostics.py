"""GPU parity of the selection diagnostic (aba_block_mass) against the oracle's
dense attention mass per key block, on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_38_amd.workloads import SINGLE, Workload

from parity_utils import inputs, make_plan, sample_items

pytestmark = pytest.mark.gpu

# Masses are probabilities summed over up to N keys: bf16 products are exact in
# fp32, logits carry fp32 rounding of a 128-term sum (relative ~1e-6), so a
# mass of m is off by about m * 1e-5 at worst; rows hold masses up to ~0.5.
MASS_ATOL = 2e-5

RAGGED = Workload("ragged_bf16", 1, 3, 128, "bf16", (3, 10, 43), 16, (0.25,),
                  description="1290 tokens: 11 blocks, the last with 10 valid")
RAGGED64 = Workload("ragged_bf16_d64", 2, 2, 64, "bf16", (2, 9, 50), 16, (0.3,),
                    description="batch 2, 900 tokens: 8 blocks, the last with 4 valid")


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


@pytest.mark.parametrize("w", [RAGGED, RAGGED64], ids=lambda w: w.name)
def test_block_mass_matches_oracle_every_block(aba, w):
    (q, k, _), (qd, kd, _) = inputs(w, 31)
    p = make_plan(aba, w)
    items = oracle.layer_items(w.batch, w.heads, w.n_blocks)
    got = aba.block_mass(p, qd, kd, items).cpu().double().numpy()
    ref = oracle.block_mass(q, k, w.seq_len, items=items, scale=p.softmax_scale)
    err = np.abs(got - ref).max()
    print(f"[{w.name}] block mass: {len(items)} rows, max abs err {err:.3g}")
    assert err <= MASS_ATOL
    assert np.abs(got.sum(axis=1) - 1.0).max() <= 1e-4


def test_block_mass_single_layer_sampled(aba):
    w = SINGLE
    (q, k, _), (qd, kd, _) = inputs(w, 1001)
    p = make_plan(aba, w)
    items = sample_items(w, 6, seed=5)
    got = aba.block_mass(p, qd, kd, items).cpu().double().numpy()
    ref = oracle.block_mass(q, k, w.seq_len, items=items, scale=p.softmax_scale)
    err = np.abs(got - ref).max()
    print(f"[single] block mass: {len(items)} rows, max abs err {err:.3g}")
    assert err <= MASS_ATOL
    # ideal top-K mass from the GPU rows equals the oracle's brute-force selection
    for r in range(len(items)):
        assert abs(np.sort(got[r])[::-1][:p.budget].sum() - oracle.topk_mass(ref[r], p.budget)) <= 1e-4


def test_block_mass_outside_items_give_zero_rows(aba):
    w = RAGGED
    (_, _, _), (qd, kd, _) = inputs(w, 31)
    p = make_plan(aba, w)
    got = aba.block_mass(p, qd, kd, [(0, 0, w.n_blocks), (0, w.heads, 0), (1, 0, 0), (0, 0, 0)]).cpu().numpy()
    assert not got[:3].any()
    assert abs(got[3].sum() - 1.0) <= 1e-4
