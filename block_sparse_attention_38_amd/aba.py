"""Python binding of libaba.so (include/aba.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels; this module checks
tensor shapes/dtypes/devices, allocates outputs with PyTorch (device memory and
streams are all PyTorch is used for) and passes raw pointers and the current
HIP stream across the C ABI.  It raises if the library has not been built: there
is no fallback.

Steps (AB-Attention page, section "Три приёма AB-Attention"):
    score(plan, q, k)              IBCS block scores               -> aba_score
    sample(plan, scores, seed)     SIP sampling plan (idx, cnt, w) -> aba_sample
    attend(plan, q, k, v, ...)     HT-weighted block-sparse attn   -> aba_attend
    attend_full(plan, q, k, v)     dense attention                 -> aba_attend_full
    attend_noalloc(plan, ...)      aba_attend without a workspace  -> aba_attend_noalloc
    block_mass(plan, q, k, items)  attention mass per key block    -> aba_block_mass (diagnostic)
    mfma_rate(iters, random, out)  sustained matrix-core rate     -> aba_mfma_rate (measurement)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaba.so")

ABA_OK, ABA_E_INVALID, ABA_E_UNSUPPORTED, ABA_E_HIP = 0, 1, 2, 3
ABA_F32, ABA_BF16 = 0, 1
BLOCK = 128
FINE_BLOCK = 4
MAX_BLOCKS = 1024
MAX_KEY_BLOCKS = 32768
MAX_CLUSTERS = 8

_DT = {"f32": ABA_F32, "bf16": ABA_BF16, torch.float32: ABA_F32, torch.bfloat16: ABA_BF16}
_TORCH = {ABA_F32: torch.float32, ABA_BF16: torch.bfloat16}


class AbaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"aba status {status}: {msg}")
        self.status = status


class PlanStruct(ctypes.Structure):
    """Mirror of aba_plan_t."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
        ("seq_pad", ctypes.c_int32), ("n_clusters", ctypes.c_int32), ("kmeans_iters", ctypes.c_int32),
        ("budget", ctypes.c_int32), ("list_cap", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("key_block", ctypes.c_int32), ("n_key_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
    ]


EXPORTS = ("aba_plan", "aba_score", "aba_sample", "aba_attend", "aba_attend_full", "aba_attend_noalloc",
           "aba_block_mass", "aba_mfma_rate", "aba_last_error", "aba_version")
# aba_mfma_rate: workgroups x threads of its checksum buffer, and floating-point
# operations per round of its loop (512 x 4 wavefronts x 16 MFMAs x 32*32*16*2)
MFMA_RATE_THREADS = 512 * 256
MFMA_RATE_FLOP_PER_ITER = 512 * 4 * 16 * 32 * 32 * 16 * 2
# Query blocks (B * H * NB) the static scratch of aba_attend_noalloc holds.
NOALLOC_MAX_QUERY_BLOCKS = (1 << 20) // 4

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libaba.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_attention_38_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, i32, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
    PP = ctypes.POINTER(PlanStruct)
    lib.aba_plan.argtypes = [PP, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32]
    lib.aba_score.argtypes = [PP, P, P, P, P, P, P, P, P]
    lib.aba_sample.argtypes = [PP, P, u64, i32, i32, P, P, P, P, P]
    lib.aba_attend.argtypes = [PP, P, P, P, P, P, P, P, P, P]
    lib.aba_attend_full.argtypes = [PP, P, P, P, P, P, P]
    lib.aba_attend_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P]
    lib.aba_block_mass.argtypes = [PP, P, P, P, ctypes.c_int32, P, P]
    lib.aba_mfma_rate.argtypes = [i32, i32, P, P]
    for name in ("aba_plan", "aba_score", "aba_sample", "aba_attend", "aba_attend_full", "aba_attend_noalloc",
                 "aba_block_mass", "aba_mfma_rate"):
        getattr(lib, name).restype = ctypes.c_int
    lib.aba_last_error.argtypes = []
    lib.aba_last_error.restype = ctypes.c_char_p
    lib.aba_version.argtypes = []
    lib.aba_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != ABA_OK:
        msg = load_library().aba_last_error().decode(errors="replace")
        raise AbaError(status, msg)


@dataclass
class Plan:
    """A filled aba_plan_t plus convenience fields."""
    raw: PlanStruct

    def __getattr__(self, name):
        return getattr(self.raw, name)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH[self.raw.dtype]


def plan(batch: int, heads: int, seq_len: int, head_dim: int, dtype="bf16", n_clusters: int = 8,
         kmeans_iters: int = 10, budget: int = 1, softmax_scale: float = 0.0, key_block: int = BLOCK) -> Plan:
    """aba_plan: validate the layer's sizes and fill a plan (host only).  key_block is
    BLOCK (128-token key blocks) or FINE_BLOCK (4-token key blocks); budget counts
    key blocks of that size."""
    raw = PlanStruct()
    _check(load_library().aba_plan(ctypes.byref(raw), batch, heads, seq_len, head_dim, _DT[dtype], n_clusters,
                                   kmeans_iters, budget, key_block, float(softmax_scale)))
    return Plan(raw)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _qkv_shape(p: Plan):
    return (p.batch, p.heads, p.seq_pad, p.head_dim)


def workspace(p: Plan, device) -> torch.Tensor:
    """Device scratch of p.workspace_bytes; one buffer serves every call ordered on a stream."""
    return torch.empty(max(int(p.workspace_bytes), 1), dtype=torch.uint8, device=device)


def _ws(p: Plan, ws, device) -> torch.Tensor:
    if ws is None:
        return workspace(p, device)
    if ws.device != device or ws.numel() * ws.element_size() < int(p.workspace_bytes) or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous {int(p.workspace_bytes)}-byte buffer on {device}")
    return ws


def score(p: Plan, q: torch.Tensor, k: torch.Tensor, *, return_parts: bool = False, out: torch.Tensor | None = None,
          ws: torch.Tensor | None = None):
    """aba_score: IBCS scores [B,H,NB,NBk] (float32).  With return_parts also the
    centroids [B,H,NB,C,D], cluster weights [B,H,NB,C] and pooled keys [B,H,NBk,D]."""
    dev = q.device
    _need(q, "q", _qkv_shape(p), p.torch_dtype, dev)
    _need(k, "k", _qkv_shape(p), p.torch_dtype, dev)
    B, H, NB, NBk, C, D = p.batch, p.heads, p.n_blocks, p.n_key_blocks, p.n_clusters, p.head_dim
    if out is None:
        out = torch.empty(B, H, NB, NBk, dtype=torch.float32, device=dev)
    _need(out, "scores", (B, H, NB, NBk), torch.float32, dev)
    cent = wgt = kbar = None
    if return_parts:
        cent = torch.empty(B, H, NB, C, D, dtype=torch.float32, device=dev)
        wgt = torch.empty(B, H, NB, C, dtype=torch.float32, device=dev)
        kbar = torch.empty(B, H, NBk, D, dtype=torch.float32, device=dev)
    ws = _ws(p, ws, dev)
    _check(load_library().aba_score(ctypes.byref(p.raw), _ptr(q), _ptr(k), _ptr(out), _ptr(cent), _ptr(wgt),
                                    _ptr(kbar), _ptr(ws), _stream()))
    return (out, cent, wgt, kbar) if return_parts else out


def sample(p: Plan, scores: torch.Tensor, seed: int, *, out=None, head_offset: int = 0, batch_offset: int = 0,
           ws: torch.Tensor | None = None):
    """aba_sample: (idx [B,H,NB,cap] int32, cnt [B,H,NB] int32, w [B,H,NB,cap] float32).
    head_offset / batch_offset: global indices of this call's head 0 and batch entry 0
    when it covers a slice of a larger layer (the draws are addressed by them)."""
    dev = scores.device
    B, H, NB, cap = p.batch, p.heads, p.n_blocks, p.list_cap
    _need(scores, "scores", (B, H, NB, p.n_key_blocks), torch.float32, dev)
    if out is None:
        out = (torch.empty(B, H, NB, cap, dtype=torch.int32, device=dev),
               torch.empty(B, H, NB, dtype=torch.int32, device=dev),
               torch.empty(B, H, NB, cap, dtype=torch.float32, device=dev))
    idx, cnt, w = out
    _need(idx, "idx", (B, H, NB, cap), torch.int32, dev)
    _need(cnt, "cnt", (B, H, NB), torch.int32, dev)
    _need(w, "w", (B, H, NB, cap), torch.float32, dev)
    ws = _ws(p, ws, dev)
    _check(load_library().aba_sample(ctypes.byref(p.raw), _ptr(scores), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                     int(head_offset), int(batch_offset), _ptr(idx), _ptr(cnt), _ptr(w), _ptr(ws),
                                     _stream()))
    return idx, cnt, w


def attend(p: Plan, q, k, v, idx, cnt, w, *, out=None, ws=None) -> torch.Tensor:
    """aba_attend: HT-weighted block-sparse attention, [B,H,N_pad,D] in the plan's dtype."""
    dev = q.device
    shp = _qkv_shape(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, shp, p.torch_dtype, dev)
    B, H, NB, cap = p.batch, p.heads, p.n_blocks, p.list_cap
    _need(idx, "idx", (B, H, NB, cap), torch.int32, dev)
    _need(cnt, "cnt", (B, H, NB), torch.int32, dev)
    _need(w, "w", (B, H, NB, cap), torch.float32, dev)
    if out is None:
        out = torch.empty(shp, dtype=p.torch_dtype, device=dev)
    _need(out, "out", shp, p.torch_dtype, dev)
    ws = _ws(p, ws, dev)
    _check(load_library().aba_attend(ctypes.byref(p.raw), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(cnt), _ptr(w),
                                     _ptr(out), _ptr(ws), _stream()))
    return out


def attend_noalloc(p: Plan, q, k, v, idx, cnt, w, *, out: torch.Tensor) -> torch.Tensor:
    """aba_attend_noalloc: aba_attend with the library's static scratch instead of a
    workspace; the caller passes the output, and nothing is allocated."""
    dev = q.device
    shp = _qkv_shape(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, shp, p.torch_dtype, dev)
    B, H, NB, cap = p.batch, p.heads, p.n_blocks, p.list_cap
    _need(idx, "idx", (B, H, NB, cap), torch.int32, dev)
    _need(cnt, "cnt", (B, H, NB), torch.int32, dev)
    _need(w, "w", (B, H, NB, cap), torch.float32, dev)
    _check(load_library().aba_attend_noalloc(ctypes.byref(p.raw), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(cnt),
                                             _ptr(w), _ptr(out), _stream()))
    return out


def attend_full(p: Plan, q, k, v, *, out=None, ws=None) -> torch.Tensor:
    """aba_attend_full: dense softmax attention, [B,H,N_pad,D] in the plan's dtype."""
    dev = q.device
    shp = _qkv_shape(p)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, shp, p.torch_dtype, dev)
    if out is None:
        out = torch.empty(shp, dtype=p.torch_dtype, device=dev)
    _need(out, "out", shp, p.torch_dtype, dev)
    ws = _ws(p, ws, dev)
    _check(load_library().aba_attend_full(ctypes.byref(p.raw), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                          _stream()))
    return out


def block_mass(p: Plan, q, k, items) -> torch.Tensor:
    """aba_block_mass: dense attention mass per key block (of the plan's key_block
    tokens) for the listed (b, h, query block) items, float32 [n_items, NBk]; each
    row sums to one."""
    dev = q.device
    _need(q, "q", _qkv_shape(p), p.torch_dtype, dev)
    _need(k, "k", _qkv_shape(p), p.torch_dtype, dev)
    it = torch.as_tensor(items, dtype=torch.int32).reshape(-1, 3).contiguous().to(dev)
    mass = torch.empty(it.shape[0], p.n_key_blocks, dtype=torch.float32, device=dev)
    _check(load_library().aba_block_mass(ctypes.byref(p.raw), _ptr(q), _ptr(k), _ptr(it), it.shape[0], _ptr(mass),
                                         _stream()))
    return mass


def mfma_rate(iters: int, random: bool, out: torch.Tensor) -> None:
    """aba_mfma_rate: iters x MFMA_RATE_FLOP_PER_ITER bf16 matrix-core operations on
    register operands (random bits or zeros), on the current stream; out is a
    float32 cuda tensor of MFMA_RATE_THREADS elements.  Timing is the caller's."""
    if not (out.is_cuda and out.dtype == torch.float32 and out.numel() >= MFMA_RATE_THREADS):
        raise ValueError(f"out must be a float32 cuda tensor of {MFMA_RATE_THREADS} elements")
    _check(load_library().aba_mfma_rate(int(iters), 1 if random else 0, _ptr(out), _stream()))


def layer(p: Plan, q, k, v, seed: int, *, ws=None):
    """One pass of the whole hot path: score -> sample -> attend."""
    ws = _ws(p, ws, q.device)
    s = score(p, q, k, ws=ws)
    idx, cnt, w = sample(p, s, seed, ws=ws)
    return attend(p, q, k, v, idx, cnt, w, ws=ws), (s, idx, cnt, w)


def version() -> str:
    return load_library().aba_version().decode()
