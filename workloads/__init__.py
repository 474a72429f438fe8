"""Workload presets and the seeded input generator.

The five presets are the layer lists, worker counts, gradient dtypes and value
distributions of the CNN workloads that the FireCaffe and GradientFlow pages
train (NiN, GoogLeNet, AlexNet on ImageNet-1k), taken as synthetic stand-ins:
no dataset or trained weights are involved.  This package only produces
inputs; it contains no step of the aggregation itself and is used by both the
CPU oracle side and the GPU side of the tests and the benchmark.

The generator is a small C library (``gen.c``) built with gcc.  Its definition
(SplitMix64 counters, Box-Muller normals, binary16 round-to-nearest-even) is
documented in that file.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgagen.so")

KIND_GRAD = 1
KIND_WEIGHT = 2
KIND_SCALE = 3

SEED_BASE = 20151031


def build(force: bool = True) -> str:
    """Compile gen.c into libgagen.so next to it (gcc, no fast-math)."""
    src = os.path.join(_HERE, "gen.c")
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
        L.gagen_key.restype = ctypes.c_uint64
        L.gagen_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.gagen_raw.restype = ctypes.c_uint64
        L.gagen_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.gagen_uniform.restype = ctypes.c_double
        L.gagen_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.gagen_normal.restype = ctypes.c_double
        L.gagen_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.gagen_f32_to_f16.restype = ctypes.c_uint16
        L.gagen_f32_to_f16.argtypes = [ctypes.c_float]
        L.gagen_fill.restype = ctypes.c_int
        L.gagen_fill.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_int32]
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


# ----------------------------------------------------------------------------
# Layer lists
# ----------------------------------------------------------------------------

def _conv(o: int, i: int, k: int) -> List[Tuple[int, ...]]:
    """A convolution's weight tensor followed by its bias."""
    return [(o, i, k, k), (o,)]


TINY_LAYERS: List[Tuple[int, ...]] = [
    (16, 3, 3, 3), (16,), (32, 16, 3, 3), (32,), (64, 32, 3, 3), (64,), (10, 576), (10,)]

# 12 mlpconv layers of a Network-in-Network for ImageNet (three 1x1 layers after
# each spatial conv, no fully connected layer), each with its bias.
NIN_LAYERS: List[Tuple[int, ...]] = (
    _conv(96, 3, 11) + _conv(96, 96, 1) + _conv(96, 96, 1)
    + _conv(256, 96, 5) + _conv(256, 256, 1) + _conv(256, 256, 1)
    + _conv(384, 256, 3) + _conv(384, 384, 1) + _conv(384, 384, 1)
    + _conv(1024, 384, 3) + _conv(1024, 1024, 1) + _conv(1000, 1024, 1))

# GoogLeNet-shaped: 3 stem convs, 9 inception modules of 6 convs each
# (1x1, 3x3-reduce, 3x3, 5x5-reduce, 5x5, pool-proj), then a 1000x1024 FC.
_INCEPTION = [  # (in, n1, n3r, n3, n5r, n5, pool_proj)
    (192, 64, 96, 128, 16, 32, 32), (256, 128, 128, 192, 32, 96, 64),
    (480, 192, 96, 208, 16, 48, 64), (512, 160, 112, 224, 24, 64, 64),
    (512, 128, 128, 256, 24, 64, 64), (512, 112, 144, 288, 32, 64, 64),
    (528, 256, 160, 320, 32, 128, 128), (832, 256, 160, 320, 32, 128, 128),
    (832, 384, 192, 384, 48, 128, 128)]


def _googlenet_layers() -> List[Tuple[int, ...]]:
    L = _conv(64, 3, 7) + _conv(64, 64, 1) + _conv(192, 64, 3)
    for c, n1, n3r, n3, n5r, n5, pp in _INCEPTION:
        L += (_conv(n1, c, 1) + _conv(n3r, c, 1) + _conv(n3, n3r, 3)
              + _conv(n5r, c, 1) + _conv(n5, n5r, 5) + _conv(pp, c, 1))
    L += [(1000, 1024), (1000,)]
    return L


GOOGLENET_LAYERS = _googlenet_layers()

ALEXNET_LAYERS: List[Tuple[int, ...]] = [
    (96, 3, 11, 11), (96,), (256, 48, 5, 5), (256,), (384, 256, 3, 3), (384,),
    (384, 192, 3, 3), (384,), (256, 192, 3, 3), (256,), (4096, 9216), (4096,),
    (4096, 4096), (4096,), (1000, 4096), (1000,)]


@dataclass
class Workload:
    name: str
    index: int
    W: int
    layers: List[Tuple[int, ...]]
    fp16: bool
    sigma: float
    mode: str                      # "dense" or "sparse"
    scale_mode: Optional[str]      # None, "layer" or "chunk"
    scale_log10: Tuple[float, float] = (-1.0, 1.0)
    chunk: int = 0
    rho: float = 0.0
    steps: int = 3
    lr: float = 0.01
    mu: float = 0.9
    w_sigma: float = 0.05

    @property
    def numels(self) -> List[int]:
        return [int(np.prod(s)) for s in self.layers]

    @property
    def P(self) -> int:
        return int(sum(self.numels))

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


WORKLOADS = {
    "tiny": Workload("tiny", 0, 4, TINY_LAYERS, False, 1e-2, "dense", "layer", (-1.0, 1.0)),
    "nin": Workload("nin", 1, 32, NIN_LAYERS, False, 1e-3, "dense", None),
    "googlenet": Workload("googlenet", 2, 128, GOOGLENET_LAYERS, True, 1e-3, "dense", None),
    "alexnet16": Workload("alexnet16", 3, 16, ALEXNET_LAYERS, True, 1e-3, "dense", "layer", (-1.0, 1.0)),
    "alexnet128_sparse": Workload("alexnet128_sparse", 4, 128, ALEXNET_LAYERS, True, 1e-3, "sparse",
                                  "chunk", (-4.0, 0.0), chunk=32768, rho=0.1),
}


def custom(W: int, numels: Sequence[int], fp16: bool, *, sigma: float = 1e-2, mode: str = "dense",
           scale_mode: Optional[str] = None, scale_log10=(-1.0, 1.0), chunk: int = 0,
           rho: float = 0.0, index: int = 99, name: str = "custom") -> Workload:
    """A workload with arbitrary sizes, for edge cases (layers given as flat numels)."""
    return Workload(name, index, W, [(int(n),) for n in numels], fp16, sigma, mode, scale_mode,
                    tuple(scale_log10), chunk=chunk, rho=rho)


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

def _log_uniform(u: float, lo: float, hi: float) -> float:
    return math.pow(10.0, lo + (hi - lo) * u)


def segments(wl: Workload, seed: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(seg_end int64, seg_scale float64) describing the per-element scale.

    "layer": one log-uniform scale per layer.  "chunk": one log-uniform scale
    per chunk of ``wl.chunk`` elements, shared by all workers and steps, all
    distinct (a colliding draw is replaced by the next one in the stream).
    """
    seed = wl.seed if seed is None else seed
    L = lib()
    key = L.gagen_key(seed, KIND_SCALE, 0, 0)
    lo, hi = wl.scale_log10
    if wl.scale_mode is None:
        return np.zeros(0, np.int64), np.zeros(0, np.float64)
    if wl.scale_mode == "layer":
        ends = np.cumsum(np.array(wl.numels, dtype=np.int64))
        sc = np.array([_log_uniform(L.gagen_uniform(key, i), lo, hi) for i in range(len(ends))])
        return ends, sc
    if wl.scale_mode == "chunk":
        C = wl.chunk
        nc = (wl.P + C - 1) // C
        ends = np.minimum(np.arange(1, nc + 1, dtype=np.int64) * C, wl.P)
        seen = set()
        sc = np.empty(nc, np.float64)
        n = 0
        for c in range(nc):
            while True:
                s = _log_uniform(L.gagen_uniform(key, n), lo, hi)
                n += 1
                if s not in seen:
                    break
            seen.add(s)
            sc[c] = s
        return ends, sc
    raise ValueError(wl.scale_mode)


def fill(out: np.ndarray, key: int, start: int, sigma: float, seg_end: np.ndarray,
         seg_scale: np.ndarray, threads: Optional[int] = None) -> np.ndarray:
    """Fill a contiguous float32 or uint16 (binary16 bits) array from a stream."""
    assert out.flags.c_contiguous
    fp16 = out.dtype == np.uint16
    assert fp16 or out.dtype == np.float32
    seg_end = np.ascontiguousarray(seg_end, dtype=np.int64)
    seg_scale = np.ascontiguousarray(seg_scale, dtype=np.float64)
    rc = lib().gagen_fill(key, start, out.size, sigma, len(seg_end),
                          seg_end.ctypes.data if len(seg_end) else None,
                          seg_scale.ctypes.data if len(seg_scale) else None,
                          int(fp16), out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise RuntimeError("gagen_fill failed")
    return out


def grad_row(wl: Workload, step: int, worker: int, seg=None, out: Optional[np.ndarray] = None,
             threads: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """Worker ``worker``'s flat gradient (length P) at step ``step`` (1-based)."""
    seed = wl.seed if seed is None else seed
    if seg is None:
        seg = segments(wl, seed)
    if out is None:
        out = np.empty(wl.P, np.uint16 if wl.fp16 else np.float32)
    key = lib().gagen_key(seed, KIND_GRAD, step, worker)
    return fill(out, key, 0, wl.sigma, seg[0], seg[1], threads)


def grad_bucket(wl: Workload, step: int, ld: int, seg=None, threads: Optional[int] = None,
                seed: Optional[int] = None, workers: Optional[Sequence[int]] = None) -> np.ndarray:
    """The [W][ld] bucket of all workers' gradients at ``step``; row padding is zero."""
    seed = wl.seed if seed is None else seed
    if seg is None:
        seg = segments(wl, seed)
    ws = list(range(wl.W)) if workers is None else list(workers)
    out = np.zeros((len(ws), ld), np.uint16 if wl.fp16 else np.float32)
    for r, w in enumerate(ws):
        grad_row(wl, step, w, seg, out[r, :wl.P], threads, seed)
    return out


def weights(wl: Workload, threads: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    """fp32 master weights N(0, w_sigma), length P."""
    seed = wl.seed if seed is None else seed
    key = lib().gagen_key(seed, KIND_WEIGHT, 0, 0)
    out = np.empty(wl.P, np.float32)
    return fill(out, key, 0, wl.w_sigma, np.zeros(0, np.int64), np.zeros(0), threads)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """binary16 bit patterns of float32 values via the generator's rounding."""
    L = lib()
    flat = np.ascontiguousarray(x, np.float32).ravel()
    return np.array([L.gagen_f32_to_f16(float(v)) for v in flat], np.uint16).reshape(np.shape(x))
