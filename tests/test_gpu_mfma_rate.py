"""The matrix-core rate loop (aba_mfma_rate, measurement support): it runs, its
products are real (zeros give zeros, random operands a checksum that scales with
the number of rounds), and a timed call reports a rate below the quoted peak."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod.load_library()
    return mod


def test_mfma_rate_products(aba):
    dev = torch.device("cuda:0")
    out = torch.full((aba.MFMA_RATE_THREADS,), float("nan"), device=dev)
    aba.mfma_rate(3, False, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    one = torch.empty_like(out)
    two = torch.empty_like(out)
    aba.mfma_rate(1, True, one)
    aba.mfma_rate(2, True, two)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all() and torch.isfinite(two).all()
    assert (one.abs() > 0).float().mean().item() > 0.99
    # every round adds the same products: two rounds give twice the checksum
    # (to fp32 rounding, measured against the largest checksum: single sums can cancel)
    rel = ((two - 2 * one).abs().max() / (2 * one).abs().max()).item()
    print(f"[mfma_rate] checksum linearity: max rel err {rel:.2e}")
    assert rel < 1e-4


def test_mfma_rate_is_timed_below_the_quoted_peak(aba):
    dev = torch.device("cuda:0")
    out = torch.empty(aba.MFMA_RATE_THREADS, device=dev)
    iters = 2000
    aba.mfma_rate(iters, True, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    aba.mfma_rate(iters, True, out)
    e1.record()
    torch.cuda.synchronize()
    tflops = iters * aba.MFMA_RATE_FLOP_PER_ITER / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"[mfma_rate] random operands: {tflops:.0f} TFLOP/s")
    assert 100 < tflops < 2600
