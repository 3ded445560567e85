"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/aba.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aba.h")


@pytest.fixture(scope="module")
def aba():
    from block_sparse_attention_38_amd import aba as mod

    if not os.path.exists(mod.LIB_PATH):
        pytest.fail("libaba.so is not built (run __graft_entry__.build() or python -m block_sparse_attention_38_amd.build)")
    mod.load_library()
    return mod


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aba_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("aba_plan", "aba_score", "aba_sample", "aba_attend", "aba_attend_full", "aba_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(aba):
    lib = aba.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), f"libaba.so does not export {name}"
    assert set(aba.EXPORTS) <= set(_declared_functions())


def test_plan_struct_matches_header_layout(aba):
    # aba_plan_t: 16 int32/float fields then a uint64 -> 72 bytes
    assert ctypes.sizeof(aba.PlanStruct) == 72
    assert aba.PlanStruct.key_block.offset == 52 and aba.PlanStruct.n_key_blocks.offset == 56
    assert aba.PlanStruct.workspace_bytes.offset == 64


def test_plan_fills_the_layer_sizes(aba):
    p = aba.plan(1, 12, 32760, 128, "bf16", 8, 10, 26)
    assert (p.n_blocks, p.seq_pad, p.list_cap, p.block) == (256, 32768, 256, 128)
    assert abs(p.softmax_scale - 128 ** -0.5) < 1e-7
    rows = 12 * 256
    assert p.workspace_bytes >= 4 * rows * (8 * 128 + 8 + 128)
    assert p.workspace_bytes >= 4 * rows                       # the attention work order
    p64 = aba.plan(1, 12, 32760, 64, "bf16", 8, 10, 26)
    assert p64.workspace_bytes >= 12 * 32768 * 64 * 2         # head_dim 64: the transposed copy of v
    p = aba.plan(1, 24, 118800, 128, "bf16", 8, 10, 74)
    assert (p.n_blocks, p.seq_pad) == (929, 118912)
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2, softmax_scale=0.5)
    assert p.softmax_scale == 0.5 and p.dtype == aba.ABA_F32
    assert (p.key_block, p.n_key_blocks) == (128, 8)


def test_fine_plan_fills_the_key_block_sizes(aba):
    p = aba.plan(1, 12, 32760, 128, "bf16", 8, 10, 832, key_block=aba.FINE_BLOCK)
    assert (p.key_block, p.n_key_blocks, p.list_cap, p.n_blocks, p.seq_pad) == (4, 8190, 8190, 256, 32768)
    coarse = aba.plan(1, 12, 32760, 128, "bf16", 8, 10, 26)
    # the pooled keys are 32x more, plus the scoring statistics
    assert p.workspace_bytes >= coarse.workspace_bytes
    assert p.workspace_bytes >= 4 * 12 * 8190 * 128
    p = aba.plan(1, 24, 118800, 128, "bf16", 8, 10, 74 * 32, key_block=4)
    assert (p.n_key_blocks, p.list_cap) == (29700, 29700)
    p = aba.plan(1, 2, 1023, 64, "f32", 8, 10, 64, key_block=4)
    assert p.n_key_blocks == 256                        # a partial last block of 3 tokens


@pytest.mark.parametrize("args,status", [
    ((0, 1, 128, 128, "bf16", 8, 10, 1), 1),          # batch < 1
    ((1, 1, 0, 128, "bf16", 8, 10, 1), 1),            # no tokens
    ((1, 1, 128, 128, "bf16", 8, 10, 0), 1),          # budget < 1
    ((1, 1, 128, 128, "bf16", 0, 10, 1), 1),          # no clusters
    ((1, 1, 128, 128, "bf16", 8, -1, 1), 1),          # negative rounds
    ((1, 1, 128, 96, "bf16", 8, 10, 1), 2),           # head_dim without kernels
    ((1, 1, 128, 128, "f32", 8, 10, 1), 2),           # fp32 only at head_dim 64
    ((1, 1, 128, 128, "bf16", 9, 10, 1), 2),          # more than 8 clusters
    ((1, 1, 1024 * 128 + 1, 128, "bf16", 8, 10, 1), 2),  # more than 1024 blocks
    ((1, 1, 128, 128, "bf16", 8, 10, 1, 0.0, 8), 1),      # key blocks of neither 128 nor 4 tokens
    ((1, 1, 128, 128, "bf16", 8, 10, 1, 0.0, 0), 1),
    ((1, 1, 128, 64, "bf16", 8, 10, 1, 0.0, 4), 2),       # 4-token blocks with bf16 need head_dim 128
    ((1, 1, 131072, 128, "bf16", 8, 10, 20000, 0.0, 4), 2),  # sampling state beyond the LDS of a CU
])
def test_plan_rejects_bad_sizes(aba, args, status):
    with pytest.raises(aba.AbaError) as ei:
        aba.plan(*args)
    assert ei.value.status == status
    assert aba.load_library().aba_last_error()


def test_entry_points_reject_null_pointers_before_launch(aba):
    lib = aba.load_library()
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2)
    pp = ctypes.byref(p.raw)
    nul = None
    assert lib.aba_score(pp, nul, nul, nul, nul, nul, nul, nul, nul) == aba.ABA_E_INVALID
    assert lib.aba_sample(pp, nul, 1, 0, 0, nul, nul, nul, nul, nul) == aba.ABA_E_INVALID
    assert lib.aba_attend(pp, nul, nul, nul, nul, nul, nul, nul, nul, nul) == aba.ABA_E_INVALID
    assert lib.aba_attend_full(pp, nul, nul, nul, nul, nul, nul) == aba.ABA_E_INVALID
    assert b"NULL" in lib.aba_last_error()
    assert lib.aba_attend_full(None, nul, nul, nul, nul, nul, nul) == aba.ABA_E_INVALID


def test_mfma_rate_rejects_bad_arguments_before_launch(aba):
    lib = aba.load_library()
    assert lib.aba_mfma_rate(0, 1, ctypes.c_void_p(16), None) == aba.ABA_E_INVALID
    assert lib.aba_mfma_rate(1000001, 1, ctypes.c_void_p(16), None) == aba.ABA_E_INVALID
    assert lib.aba_mfma_rate(10, 1, None, None) == aba.ABA_E_INVALID
    assert b"null" in lib.aba_last_error()


@pytest.mark.parametrize("h0,b0", [(-1, 0), (0, -1), (2**31 - 2, 0), (0, 2**31 - 1)])
def test_sample_rejects_offsets_outside_the_counter_range(aba, h0, b0):
    """The draws are addressed by the global (batch, head) indices b0 + b and h0 + h;
    offsets that are negative or push them past 2^31 - 1 are refused before launch."""
    lib = aba.load_library()
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2)
    fake = ctypes.c_void_p(1)
    assert lib.aba_sample(ctypes.byref(p.raw), fake, 1, h0, b0, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"offset" in lib.aba_last_error()


def test_block_mass_checks_dtype_and_pointers(aba):
    lib = aba.load_library()
    fake = ctypes.c_void_p(1)
    p32 = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2)
    assert lib.aba_block_mass(ctypes.byref(p32.raw), fake, fake, fake, 1, fake, None) == aba.ABA_E_UNSUPPORTED
    p = aba.plan(1, 2, 1024, 128, "bf16", 8, 10, 2)
    assert lib.aba_block_mass(ctypes.byref(p.raw), fake, fake, None, 1, fake, None) == aba.ABA_E_INVALID
    assert lib.aba_block_mass(ctypes.byref(p.raw), fake, fake, fake, -1, fake, None) == aba.ABA_E_INVALID
    assert lib.aba_block_mass(ctypes.byref(p.raw), None, None, None, 0, None, None) == aba.ABA_OK   # nothing to do


def test_bf16_attention_requires_a_workspace(aba):
    lib = aba.load_library()
    p = aba.plan(1, 2, 1024, 128, "bf16", 8, 10, 2)
    fake = ctypes.c_void_p(1)
    assert lib.aba_attend(ctypes.byref(p.raw), fake, fake, fake, fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"workspace" in lib.aba_last_error()
    assert lib.aba_attend_full(ctypes.byref(p.raw), fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"workspace" in lib.aba_last_error()


def test_tampered_plan_is_rejected(aba):
    lib = aba.load_library()
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2)
    p.raw.n_blocks = 9          # not what aba_plan computes for 1024 tokens
    fake = ctypes.c_void_p(1)
    assert lib.aba_attend_full(ctypes.byref(p.raw), fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"inconsistent" in lib.aba_last_error()
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 64, key_block=4)
    p.raw.n_key_blocks = 8      # the 128-token count under a 4-token plan
    assert lib.aba_attend_full(ctypes.byref(p.raw), fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 64, key_block=4)
    p.raw.key_block = 128       # fields of the other key block size
    assert lib.aba_attend_full(ctypes.byref(p.raw), fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID


def test_long_rows_sample_needs_a_workspace(aba):
    """Rows of more than 8192 4-token key blocks are sampled in chunks whose state
    lives in the workspace; shorter rows need none."""
    lib = aba.load_library()
    fake = ctypes.c_void_p(1)
    p = aba.plan(1, 2, 118800, 128, "bf16", 8, 10, 2368, key_block=4)
    assert lib.aba_sample(ctypes.byref(p.raw), fake, 1, 0, 0, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"workspace" in lib.aba_last_error()
    short = aba.plan(1, 2, 32760, 128, "bf16", 8, 10, 832, key_block=4)   # 8190 blocks: one workgroup per row
    assert short.workspace_bytes < p.workspace_bytes


@pytest.mark.parametrize("key_block", [128, 4])
def test_scores_always_need_a_workspace(aba, key_block):
    lib = aba.load_library()
    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2 if key_block == 128 else 64, key_block=key_block)
    fake = ctypes.c_void_p(1)
    # every optional output given, still no workspace: the two scoring passes keep their statistics there
    assert lib.aba_score(ctypes.byref(p.raw), fake, fake, fake, fake, fake, fake, None, None) == aba.ABA_E_INVALID
    assert b"workspace" in lib.aba_last_error()


def test_binding_refuses_cpu_tensors(aba):
    import torch

    p = aba.plan(1, 2, 1024, 64, "f32", 8, 10, 2)
    x = torch.zeros(1, 2, 1024, 64)
    with pytest.raises(ValueError):
        aba.attend_full(p, x, x, x)
