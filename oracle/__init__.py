"""CPU oracle for the AB-Attention sparse attention layer (test infrastructure).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library and
its Python binding) never imports, links or runs anything here.

This module is argument marshalling over ``aba_oracle.c``: plain C loops in fp64,
built with gcc.  Every function cites the passage of the AB-Attention page
("AB-Attention ускорил генерацию видео до 2,23× и пропускает 92% внимания",
section "Три приёма AB-Attention") that it follows; the C file states each
reading taken where the page is silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aba_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK = 128


def build(force: bool = True) -> str:
    """Compile aba_oracle.c into oracle/liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64, u64 = ctypes.c_int, ctypes.c_long, ctypes.c_double, ctypes.c_uint64
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    lib.oracle_n_blocks.argtypes = [i32, i32]
    lib.oracle_n_blocks.restype = i32
    lib.oracle_kmeans_block.argtypes = [P, i64, i32, i32, i32, i32, P, P, P]
    lib.oracle_kmeans_block.restype = f64
    lib.oracle_kmeans.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.oracle_kmeans.restype = None
    lib.oracle_pool.argtypes = [P, i32, i32, i32, i32, i32, i32, P]
    lib.oracle_pool.restype = None
    lib.oracle_score.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f64, P]
    lib.oracle_score.restype = None
    lib.oracle_thresholds.argtypes = [P, i32, i32, P]
    lib.oracle_thresholds.restype = i32
    lib.oracle_philox4x32_10.argtypes = [P, P, P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_draw.argtypes = [u64, i32, i32, i32, i32]
    lib.oracle_draw.restype = ctypes.c_uint32
    lib.oracle_sample.argtypes = [P, i32, i32, i32, i32, i32, u64, i32, i32, i32, P, P, P, P]
    lib.oracle_sample.restype = None
    lib.oracle_attend.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, P, P, i32, P, i32, P, P, P, P]
    lib.oracle_attend.restype = None
    lib.oracle_attend_full.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f64, P, i32, P]
    lib.oracle_attend_full.restype = None
    lib.oracle_block_mass.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, i32, P]
    lib.oracle_block_mass.restype = None
    lib.oracle_topk_mass.argtypes = [P, i32, i32]
    lib.oracle_topk_mass.restype = f64
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f32(a) -> np.ndarray:
    """Widen a tensor or array to a C-contiguous float32 numpy array (exact for bf16/fp32)."""
    try:  # torch tensor
        import torch

        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _items(items, B, H, NB) -> np.ndarray:
    if items is None:
        items = [(b, h, j) for b in range(B) for h in range(H) for j in range(NB)]
    arr = np.ascontiguousarray(np.asarray(items, dtype=np.int32).reshape(-1, 3))
    assert np.all(arr[:, 0] < B) and np.all(arr[:, 1] < H) and np.all(arr[:, 2] < NB)
    return arr


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def default_scale(head_dim: int) -> float:
    return 1.0 / float(np.sqrt(head_dim))


def n_blocks(n_valid: int, blk: int = BLOCK) -> int:
    return _load().oracle_n_blocks(n_valid, blk)


def kmeans_block(x, C: int = 8, T: int = 10):
    """IBCS clustering of one block's query rows x [n, D] (IBCS paragraph).

    Returns (centroids [C, D], weights [C], last assignment [n], min relative gap)."""
    x = _f32(x)
    n, D = x.shape
    cent = np.zeros((C, D), np.float64)
    w = np.zeros(C, np.float64)
    a = np.zeros(max(n, 1), np.int32)
    gap = _load().oracle_kmeans_block(_ptr(x), D, n, D, C, T, _ptr(cent), _ptr(w), _ptr(a))
    return cent, w, a[:n], gap


def kmeans(q, n_valid: int, C: int = 8, T: int = 10, blk: int = BLOCK):
    """Per-(b, h, query block) clustering of q [B,H,N_pad,D] (IBCS paragraph).

    Returns centroids [B,H,NB,C,D], weights [B,H,NB,C], min relative gap [B,H,NB]."""
    q = _f32(q)
    B, H, N_pad, D = q.shape
    NB = n_blocks(n_valid, blk)
    cent = np.zeros((B, H, NB, C, D), np.float64)
    w = np.zeros((B, H, NB, C), np.float64)
    gap = np.zeros((B, H, NB), np.float64)
    _load().oracle_kmeans(_ptr(q), B, H, n_valid, N_pad, D, blk, C, T, _ptr(cent), _ptr(w), _ptr(gap))
    return cent, w, gap


def pool(k, n_valid: int, blk: int = BLOCK) -> np.ndarray:
    """Mean of the valid keys of every key block of ``blk`` tokens (IBCS paragraph,
    "averaged keys"; 4-token key blocks: the kernel paragraph)."""
    k = _f32(k)
    B, H, N_pad, D = k.shape
    NB = n_blocks(n_valid, blk)
    kbar = np.zeros((B, H, NB, D), np.float64)
    _load().oracle_pool(_ptr(k), B, H, n_valid, N_pad, D, blk, _ptr(kbar))
    return kbar


def score(cent, weight, kbar, scale: float) -> np.ndarray:
    """Cluster-weighted attention of centroids to pooled keys (IBCS paragraph).

    cent [B,H,NBq,C,D], weight [B,H,NBq,C], kbar [B,H,NBk,D] -> fp64 scores [B,H,NBq,NBk]."""
    cent = np.ascontiguousarray(cent, np.float64)
    weight = np.ascontiguousarray(weight, np.float64)
    kbar = np.ascontiguousarray(kbar, np.float64)
    B, H, NBq, C, D = cent.shape
    NBk = kbar.shape[2]
    out = np.zeros((B, H, NBq, NBk), np.float64)
    _load().oracle_score(_ptr(cent), _ptr(weight), _ptr(kbar), B, H, NBq, NBk, C, D, scale, _ptr(out))
    return out


def thresholds(scores_row, K: int):
    """SIP inclusion thresholds of one row (SIP paragraph): (theta uint64 [NB], n always-kept)."""
    s = np.ascontiguousarray(np.asarray(scores_row, np.float32))
    theta = np.zeros(s.shape[0], np.uint64)
    t = _load().oracle_thresholds(_ptr(s), s.shape[0], K, _ptr(theta))
    return theta, t


def philox4x32_10(counter, key):
    """Philox4x32-10 (Salmon et al., SC'11) of one 4-word counter and 2-word key."""
    c = np.ascontiguousarray(np.asarray(counter, np.uint32))
    k = np.ascontiguousarray(np.asarray(key, np.uint32))
    out = np.zeros(4, np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def draw(seed: int, b: int, h: int, qb: int, j: int) -> int:
    """The 32-bit uniform draw addressed by (seed, batch, head, query block, key block)."""
    return int(_load().oracle_draw(seed, b, h, qb, j))


def sample(scores, K: int, seed: int, cap: int | None = None, head_offset: int = 0, batch_offset: int = 0):
    """SIP sampling plan (SIP paragraph): idx/w [B,H,NBq,cap], cnt [B,H,NBq], theta [B,H,NBq,NBk].
    The scores may be heads head_offset.. and batch entries batch_offset.. of a larger
    layer; draws are addressed by those global indices."""
    s = np.ascontiguousarray(np.asarray(scores, np.float32))
    B, H, NBq, NBk = s.shape
    cap = NBk if cap is None else cap
    idx = np.full((B, H, NBq, cap), -1, np.int32)
    cnt = np.zeros((B, H, NBq), np.int32)
    w = np.zeros((B, H, NBq, cap), np.float32)
    theta = np.zeros((B, H, NBq, NBk), np.uint64)
    _load().oracle_sample(_ptr(s), B, H, NBq, NBk, K, seed, cap, head_offset, batch_offset, _ptr(idx), _ptr(cnt),
                          _ptr(w), _ptr(theta))
    return idx, cnt, w, theta


def attend(q, k, v, n_valid: int, idx, cnt, w, items=None, scale: float | None = None, shift=None,
           blk: int = BLOCK, kblk: int | None = None):
    """HT-weighted softmax attention over each query block's kept list (SIP paragraph).

    List entries name key blocks of ``kblk`` tokens (default ``blk``; 4 for the
    kernel paragraph's fine-grained key blocks).  Returns out [n_items, blk, D]
    (fp64); with ``shift`` [n_items, blk] also (num, den)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N_pad, D = q.shape
    NB = n_blocks(n_valid, blk)
    kblk = blk if kblk is None else kblk
    scale = default_scale(D) if scale is None else scale
    idx = np.ascontiguousarray(idx, np.int32)
    cnt = np.ascontiguousarray(cnt, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    cap = idx.shape[-1]
    assert idx.shape == (B, H, NB, cap) and w.shape == idx.shape and cnt.shape == (B, H, NB)
    it = _items(items, B, H, NB)
    out = np.zeros((it.shape[0], blk, D), np.float64)
    num = den = None
    if shift is not None:
        shift = np.ascontiguousarray(shift, np.float64).reshape(it.shape[0], blk)
        num = np.zeros((it.shape[0], blk, D), np.float64)
        den = np.zeros((it.shape[0], blk), np.float64)
    _load().oracle_attend(_ptr(q), _ptr(k), _ptr(v), B, H, n_valid, N_pad, D, blk, kblk, scale, _ptr(idx), _ptr(cnt),
                          _ptr(w), cap, _ptr(it), it.shape[0], _ptr(shift), _ptr(out), _ptr(num), _ptr(den))
    return (out, num, den) if shift is not None else out


def attend_full(q, k, v, n_valid: int, items=None, scale: float | None = None, blk: int = BLOCK):
    """Dense softmax attention of the listed query blocks (full-attention reference)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N_pad, D = q.shape
    NB = n_blocks(n_valid, blk)
    scale = default_scale(D) if scale is None else scale
    it = _items(items, B, H, NB)
    out = np.zeros((it.shape[0], blk, D), np.float64)
    _load().oracle_attend_full(_ptr(q), _ptr(k), _ptr(v), B, H, n_valid, N_pad, D, blk, scale, _ptr(it),
                               it.shape[0], _ptr(out))
    return out


def block_mass(q, k, n_valid: int, items=None, scale: float | None = None, blk: int = BLOCK,
               kblk: int | None = None):
    """Dense attention mass per key block of ``kblk`` tokens (default ``blk``),
    averaged over the valid rows of each listed query block of ``blk`` tokens."""
    q, k = _f32(q), _f32(k)
    B, H, N_pad, D = q.shape
    NB = n_blocks(n_valid, blk)
    kblk = blk if kblk is None else kblk
    scale = default_scale(D) if scale is None else scale
    it = _items(items, B, H, NB)
    mass = np.zeros((it.shape[0], n_blocks(n_valid, kblk)), np.float64)
    _load().oracle_block_mass(_ptr(q), _ptr(k), B, H, n_valid, N_pad, D, blk, kblk, scale, _ptr(it), it.shape[0],
                              _ptr(mass))
    return mass


def topk_mass(mass_row, K: int) -> float:
    """Largest attention mass K key blocks can keep (ideal top-k)."""
    m = np.ascontiguousarray(np.asarray(mass_row, np.float64))
    return float(_load().oracle_topk_mass(_ptr(m), m.shape[0], K))


def layer_items(B: int, H: int, NB: int):
    return [(b, h, j) for b in range(B) for h in range(H) for j in range(NB)]
