"""The layer step (aba_score, aba_sample, aba_attend) launched into a captured
HIP graph: the library allocates, clears and synchronises nothing on these
paths, so a caller may capture a step and replay it.  Every replay, with eager
work and synchronisations between replays, must give the eager step's scores,
lists and output bit for bit; the graph is also replayed after its inputs are
overwritten in place (a plan refresh on new activations), against a fresh eager
step on the new inputs."""
import pytest
import torch

from block_sparse_attention_38_amd.workloads import SINGLE, TINY, Workload

from parity_utils import compare_lists, inputs, make_fine_plan, make_plan

pytestmark = pytest.mark.gpu

RAGGED = Workload("ragged_bf16", 1, 3, 128, "bf16", (3, 10, 43), 16, (0.25,),
                  description="1290 tokens: 11 blocks, the last with 10 valid")


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def _buffers(aba, p, q):
    dev = q.device
    B, H, NB, cap = p.batch, p.heads, p.n_blocks, p.list_cap
    return (aba.workspace(p, dev), torch.empty(B, H, NB, p.n_key_blocks, device=dev),
            (torch.empty(B, H, NB, cap, dtype=torch.int32, device=dev),
             torch.empty(B, H, NB, dtype=torch.int32, device=dev), torch.empty(B, H, NB, cap, device=dev)),
            torch.empty_like(q))


def _state(scores, lists, out):
    return [scores.clone(), *(x.clone() for x in lists), out.clone()]


def _same(a, b):
    """Scores and outputs bit for bit; the lists on their valid prefixes (the
    sampler writes the first cnt entries of a row and leaves the rest)."""
    ref = tuple(x.cpu().numpy() for x in b[1:4])
    return torch.equal(a[0], b[0]) and torch.equal(a[4], b[4]) and compare_lists(*a[1:4], *ref) == 0


@pytest.mark.parametrize("w,key_block", [(TINY, 128), (RAGGED, 128), (RAGGED, 4), (SINGLE, 128)],
                         ids=["tiny", "ragged", "ragged_4token", "single_layer"])
def test_step_replays_from_a_graph(aba, w, key_block):
    (_, _, _), (q, k, v) = inputs(w, 601)
    p = make_plan(aba, w) if key_block == 128 else make_fine_plan(aba, w)
    ws, scores, lists, out = _buffers(aba, p, q)

    def step():
        aba.score(p, q, k, out=scores, ws=ws)
        aba.sample(p, scores, 11, out=lists, ws=ws)
        aba.attend(p, q, k, v, *lists, out=out, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = _state(scores, lists, out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (scores, out, *lists):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_state(scores, lists, out), eager), f"replay {r} differs from the eager step"
        step()                       # eager work between replays
        torch.cuda.synchronize()
    # new activations in the captured buffers: the replay follows them
    (_, _, _), (q2, k2, v2) = inputs(w, 602)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    fresh = _state(scores, lists, out)
    assert not torch.equal(fresh[-1], eager[-1])
    g.replay()
    torch.cuda.synchronize()
    assert _same(_state(scores, lists, out), fresh)
    print(f"[{w.name}, {key_block}-token] 4 graph replays bit-identical to the eager step")
