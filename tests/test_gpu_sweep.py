"""Plan reuse across denoising steps (the page refreshes the sampling plan every
4 steps and attends every step): attention on a later step's q/k/v with an
earlier step's lists matches the oracle given the same lists."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_38_amd.workloads import SWEEP

from parity_utils import (check_attention, compare_lists, gpu_rows, inputs, make_plan, sample_items)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def test_plan_reused_on_later_steps(aba):
    w = SWEEP
    p = make_plan(aba, w)
    (_, _, _), (q0, k0, _) = inputs(w, 1001, step=0)
    s0 = aba.score(p, q0, k0)
    idx, cnt, wt = aba.sample(p, s0, 7)
    lists = tuple(x.cpu().numpy() for x in (idx, cnt, wt))
    items = sample_items(w, 8, seed=21)
    for step in (1, 3):
        (q, k, v), (qd, kd, vd) = inputs(w, 1001, step=step)
        out = aba.attend(p, qd, kd, vd, idx, cnt, wt)
        torch.cuda.synchronize()
        ref = oracle.attend(q, k, v, w.seq_len, *lists, items=items, scale=p.softmax_scale)
        err = check_attention(gpu_rows(out, items), ref, w.dtype, "plan_reused_on_later_steps")
        print(f"[sweep] step {step} with the step-0 plan: max abs err {err:.3g}")
    # a refreshed plan follows the drifted inputs: the lists change, and stay bit-exact
    (_, _, _), (q4, k4, _) = inputs(w, 1001, step=4)
    s4 = aba.score(p, q4, k4)
    idx4, cnt4, wt4 = aba.sample(p, s4, 7 + 4)
    o_idx, o_cnt, o_w, _ = oracle.sample(s4.cpu().numpy(), p.budget, 7 + 4)
    assert compare_lists(idx4, cnt4, wt4, o_idx, o_cnt, o_w) == 0
    assert compare_lists(idx4, cnt4, wt4, *lists) > 0
