"""Oracle for the gradient-aggregation hot path (test infrastructure only).

A plain CPU statement of the method in ``oracle.c`` (gcc, -O2
-ffp-contract=off, no fast-math), wrapped here with ctypes over numpy arrays.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use it;
the GPU library neither imports nor links it, and it shares no code with it.

Every function cites the passage of the pages it follows; see oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_P = ctypes.c_void_p


def build(force: bool = True) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-pthread", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.ora_f16_decode.restype = ctypes.c_float
        L.ora_f16_decode.argtypes = [ctypes.c_uint16]
        L.ora_tree_sum.restype = ctypes.c_int
        L.ora_tree_sum.argtypes = [ctypes.c_int32, ctypes.c_int64, _P, _P]
        L.ora_sgd.restype = None
        L.ora_sgd.argtypes = [ctypes.c_int64, _P, _P, _P, ctypes.c_float, ctypes.c_float]
        L.ora_dense_step.restype = ctypes.c_int
        L.ora_dense_step.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P,
                                     ctypes.c_float, ctypes.c_float, _P, _P, _P, ctypes.c_int32]
        L.ora_chunk_key.restype = ctypes.c_double
        L.ora_chunk_key.argtypes = [_P, ctypes.c_int64]
        L.ora_keep_count.restype = ctypes.c_int64
        L.ora_keep_count.argtypes = [ctypes.c_int64, ctypes.c_double]
        L.ora_topk.restype = ctypes.c_int
        L.ora_topk.argtypes = [ctypes.c_int64, _P, ctypes.c_int32, _P, _P]
        L.ora_sparse_step.restype = ctypes.c_int
        L.ora_sparse_step.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P,
                                      ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P, _P,
                                      ctypes.c_float, ctypes.c_float, _P, _P, _P, ctypes.c_int32]
        L.ora_round_f16.restype = ctypes.c_float
        L.ora_round_f16.argtypes = [ctypes.c_float]
        L.ora_ring_segment.restype = ctypes.c_int64
        L.ora_ring_segment.argtypes = [ctypes.c_int32, ctypes.c_int64]
        L.ora_reduce_variant.restype = ctypes.c_int
        L.ora_reduce_variant.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, _P, _P, _P,
                                         ctypes.c_int32]
        L.ora_pack.restype = ctypes.c_int
        L.ora_pack.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_int64, _P]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


def _threads(threads: Optional[int]) -> int:
    if threads:
        return int(threads)
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def f16_decode(bits) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, np.uint16).ravel()
    return np.array([L.ora_f16_decode(int(b)) for b in flat], np.float32).reshape(np.shape(bits))


def tree_sum(leaves: np.ndarray) -> np.ndarray:
    """Fixed binary-tree sum over axis 0 of a [W][n] float32 array."""
    leaves = np.ascontiguousarray(leaves, np.float32)
    W, n = leaves.shape
    out = np.empty(n, np.float32)
    if lib().ora_tree_sum(W, n, _ptr(leaves), _ptr(out)) != 0:
        raise RuntimeError("ora_tree_sum failed")
    return out


def sgd(gbar: np.ndarray, w: np.ndarray, v: np.ndarray, lr: float, mu: float) -> None:
    """In-place momentum SGD on float32 w, v."""
    gbar = np.ascontiguousarray(gbar, np.float32)
    lib().ora_sgd(gbar.size, _ptr(gbar), _ptr(w), _ptr(v), lr, mu)


def keep_count(n_chunks: int, rho: float) -> int:
    return int(lib().ora_keep_count(n_chunks, rho))


def chunk_key(a: np.ndarray) -> float:
    a = np.ascontiguousarray(a, np.float32)
    return float(lib().ora_chunk_key(_ptr(a), a.size))


def topk(keys: np.ndarray, k: int) -> Tuple[np.ndarray, float]:
    keys = np.ascontiguousarray(keys, np.float64)
    idx = np.empty(max(k, 1), np.int32)
    m = ctypes.c_double(0.0)
    if lib().ora_topk(keys.size, _ptr(keys), k, _ptr(idx), ctypes.byref(m)) != 0:
        raise RuntimeError("ora_topk failed")
    return idx[:k].copy(), m.value


def dense_step(bucket: np.ndarray, P: int, fp16: bool, lr: float, mu: float,
               w: Optional[np.ndarray], v: Optional[np.ndarray], want_gbar: bool = True,
               threads: Optional[int] = None) -> Optional[np.ndarray]:
    """One dense step over a [W][ld] bucket (float32, or uint16 binary16 bits).

    Updates w, v in place (when given) and returns the mean gradient."""
    W, ld = bucket.shape
    assert bucket.dtype == (np.uint16 if fp16 else np.float32)
    gbar = np.empty(P, np.float32) if want_gbar else None
    rc = lib().ora_dense_step(W, P, ld, int(fp16), _ptr(bucket), lr, mu, _ptr(w), _ptr(v), _ptr(gbar),
                              _threads(threads))
    if rc != 0:
        raise RuntimeError("ora_dense_step failed (%d)" % rc)
    return gbar


class SparseResult:
    def __init__(self, keys, sel_idx, sel_mask, margin, gbar):
        self.keys = keys
        self.sel_idx = sel_idx
        self.sel_mask = sel_mask
        self.margin = margin
        self.gbar = gbar


def sparse_step(bucket: np.ndarray, P: int, fp16: bool, chunk: int, k: int, resid: np.ndarray,
                lr: float, mu: float, w: Optional[np.ndarray], v: Optional[np.ndarray],
                want_keys: bool = True, want_gbar: bool = True,
                threads: Optional[int] = None) -> SparseResult:
    """One sparse step; resid ([W][ld] float32) is updated in place."""
    W, ld = bucket.shape
    assert resid.shape == (W, ld) and resid.dtype == np.float32
    n_c = (P + chunk - 1) // chunk
    mw = (n_c + 31) // 32
    keys = np.empty((W, n_c), np.float64) if want_keys else None
    sel_idx = np.empty((W, max(k, 1)), np.int32)
    sel_mask = np.empty((W, mw), np.uint32)
    margin = np.empty(W, np.float64)
    gbar = np.empty(P, np.float32) if want_gbar else None
    rc = lib().ora_sparse_step(W, P, ld, int(fp16), _ptr(bucket), chunk, k, _ptr(resid), _ptr(keys),
                               _ptr(sel_idx), _ptr(sel_mask), _ptr(margin), lr, mu, _ptr(w), _ptr(v),
                               _ptr(gbar), _threads(threads))
    if rc != 0:
        raise RuntimeError("ora_sparse_step failed (%d)" % rc)
    return SparseResult(keys, sel_idx[:, :k], sel_mask, margin, gbar)


ORDERS = {"tree": 0, "ps": 1, "server": 1, "ring": 2}


def round_f16(x) -> np.ndarray:
    """Nearest binary16 value of each binary32 value (ties to even), as binary32."""
    L = lib()
    flat = np.ascontiguousarray(x, np.float32).ravel()
    return np.array([L.ora_round_f16(float(v)) for v in flat], np.float32).reshape(np.shape(x))


def ring_segment(W: int, P: int) -> int:
    return int(lib().ora_ring_segment(W, P))


def reduce_variant(bucket: np.ndarray, P: int, fp16: bool, order: str, wire16: bool, lr: float = 0.0,
                   mu: float = 0.0, w: Optional[np.ndarray] = None, v: Optional[np.ndarray] = None,
                   threads: Optional[int] = None) -> np.ndarray:
    """Mean gradient under another summation order and/or a binary16 wire."""
    W, ld = bucket.shape
    gbar = np.empty(P, np.float32)
    rc = lib().ora_reduce_variant(W, P, ld, int(fp16), _ptr(bucket), ORDERS[order], int(wire16), lr, mu, _ptr(w),
                                  _ptr(v), _ptr(gbar), _threads(threads))
    if rc != 0:
        raise RuntimeError("ora_reduce_variant failed (%d)" % rc)
    return gbar


def pack(layers, ld: int) -> np.ndarray:
    """Fuse per-worker layer lists ``layers[w][l]`` (1-D arrays) into a [W][ld] bucket."""
    W, L = len(layers), len(layers[0])
    numel = np.array([layers[0][l].size for l in range(L)], np.int64)
    dt = layers[0][0].dtype
    ptrs = (ctypes.c_void_p * (W * L))()
    keep = []
    for w in range(W):
        for l in range(L):
            a = np.ascontiguousarray(layers[w][l])
            assert a.dtype == dt and a.size == numel[l]
            keep.append(a)
            ptrs[w * L + l] = a.ctypes.data
    out = np.zeros((W, ld), dt)
    if lib().ora_pack(W, L, _ptr(numel), ptrs, dt.itemsize, ld, _ptr(out)) != 0:
        raise RuntimeError("ora_pack failed")
    return out
