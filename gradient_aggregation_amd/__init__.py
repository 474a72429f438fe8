"""Python binding of libgradagg.so, the MI355X gradient-aggregation library.

Argument marshalling only: every step of the aggregation runs in the HIP
kernels behind the C ABI declared in include/gradagg.h.  PyTorch supplies the
device memory (tensors) and the stream (the current HIP stream).  There is no
fallback: if the library is not built, importing the binding's entry points
raises.

Terms follow the pages: W workers, a layer list, a chunk size and a keep ratio
(FireCaffe sec. 6 reduction tree; GradientFlow lazy allreduce, mixed precision
and coarse-grained sparse communication).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgradagg.so")

GA_OK, GA_ERR_INVALID, GA_ERR_ALIGN, GA_ERR_DEVICE, GA_ERR_UNSUPPORTED = range(5)
GA_FP32, GA_FP16 = 0, 1
ORDERS = {"tree": 0, "server": 1, "ring": 2}
MAX_WORKERS = 1024
MAX_CHUNKS = 65536
MAX_ELEMENTS = 1 << 33
STATIC_KEYS = 1 << 22


class GAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (status_name(status), msg))
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int64), ("ld", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("n_chunks", ctypes.c_int64), ("W", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("k", ctypes.c_int32), ("mask_words", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SGD(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("mu", ctypes.c_float)]


MAX_AGE = 2


class History(ctypes.Structure):
    """ga_history: what a deferred step holds of its residual (see gradagg.h)."""
    _fields_ = [("age", ctypes.c_int32), ("d_masks", ctypes.c_void_p * (MAX_AGE + 1)),
                ("d_layer_ptrs", ctypes.c_void_p * MAX_AGE)]


_VP = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgradagg.so is not built (run __graft_entry__.build() or "
                               "python gradient_aggregation_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        L.ga_abi_version.restype = ctypes.c_int32
        L.ga_status_str.restype = ctypes.c_char_p
        L.ga_status_str.argtypes = [st]
        L.ga_last_error.restype = ctypes.c_char_p
        L.ga_plan_compute_info.restype = st
        L.ga_plan_compute_info.argtypes = [ctypes.c_int32, ctypes.c_int32, _VP, st, ctypes.c_int64,
                                           ctypes.c_double, ctypes.POINTER(PlanInfo)]
        L.ga_plan_create.restype = st
        L.ga_plan_create.argtypes = [ctypes.c_int32, ctypes.c_int32, _VP, st, ctypes.c_int64, ctypes.c_double,
                                     ctypes.POINTER(_VP)]
        L.ga_plan_destroy.restype = None
        L.ga_plan_destroy.argtypes = [_VP]
        L.ga_plan_get_info.restype = st
        L.ga_plan_get_info.argtypes = [_VP, ctypes.POINTER(PlanInfo)]
        L.ga_bucket_pack.restype = st
        L.ga_bucket_pack.argtypes = [_VP, _VP, _VP, _VP]
        L.ga_tree_reduce.restype = st
        L.ga_tree_reduce.argtypes = [_VP, _VP, _VP, ctypes.POINTER(SGD), _VP, _VP, _VP]
        L.ga_tree_reduce_layers.restype = st
        L.ga_tree_reduce_layers.argtypes = [_VP, _VP, _VP, ctypes.POINTER(SGD), _VP, _VP, _VP]
        L.ga_chunk_norm_layers.restype = st
        L.ga_chunk_norm_layers.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP]
        L.ga_reduce_variant.restype = st
        L.ga_reduce_variant.argtypes = [_VP, _VP, st, ctypes.c_int32, _VP, ctypes.POINTER(SGD), _VP, _VP, _VP]
        L.ga_chunk_norm.restype = st
        L.ga_chunk_norm.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP]
        L.ga_chunk_topk.restype = st
        L.ga_chunk_topk.argtypes = [_VP, _VP, _VP, _VP, _VP]
        L.ga_chunk_norm_topk.restype = st
        L.ga_chunk_norm_topk.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.ga_chunk_norm_topk_static.restype = st
        L.ga_chunk_norm_topk_static.argtypes = [_VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.ga_sparse_gather_reduce.restype = st
        L.ga_sparse_gather_reduce.argtypes = [_VP, _VP, _VP, ctypes.c_int32, _VP, ctypes.POINTER(SGD), _VP, _VP,
                                              _VP]
        L.ga_tree_partial.restype = st
        L.ga_tree_partial.argtypes = [_VP, _VP, _VP, _VP]
        L.ga_tree_combine.restype = st
        L.ga_tree_combine.argtypes = [_VP, _VP, ctypes.c_int32, _VP, ctypes.POINTER(SGD), _VP, _VP, _VP]
        L.ga_sgd_momentum_apply.restype = st
        L.ga_sgd_momentum_apply.argtypes = [ctypes.c_int64, _VP, _VP, _VP, ctypes.POINTER(SGD), _VP]
        L.ga_chunk_norm_deferred.restype = st
        L.ga_chunk_norm_deferred.argtypes = [_VP, _VP, ctypes.POINTER(History), ctypes.c_int32, _VP, _VP, _VP]
        L.ga_sparse_gather_reduce_deferred.restype = st
        L.ga_sparse_gather_reduce_deferred.argtypes = [_VP, _VP, ctypes.POINTER(History), ctypes.c_int32, _VP, _VP,
                                                       _VP, ctypes.POINTER(SGD), _VP, _VP, _VP]
        L.ga_residual_flush.restype = st
        L.ga_residual_flush.argtypes = [_VP, _VP, ctypes.POINTER(History), ctypes.c_int32, _VP, _VP, _VP]
        L.ga_bucket_boundaries.restype = st
        L.ga_bucket_boundaries.argtypes = [ctypes.c_int32, _VP, ctypes.c_int32, ctypes.c_int64, _VP, _VP]
        L.ga_buckets_create.restype = st
        L.ga_buckets_create.argtypes = [_VP, ctypes.c_int64, _VP]
        L.ga_buckets_destroy.restype = None
        L.ga_buckets_destroy.argtypes = [_VP]
        L.ga_buckets_count.restype = ctypes.c_int32
        L.ga_buckets_count.argtypes = [_VP]
        L.ga_bucket_range.restype = st
        L.ga_bucket_range.argtypes = [_VP, ctypes.c_int32, _VP, _VP, _VP, _VP]
        L.ga_bucket_reduce_layers.restype = st
        L.ga_bucket_reduce_layers.argtypes = [_VP, ctypes.c_int32, _VP, _VP, _VP, ctypes.POINTER(SGD), _VP, _VP,
                                              ctypes.c_int32, _VP]
        _lib = L
    return _lib


def status_name(s: int) -> str:
    return lib().ga_status_str(s).decode()


def _check(s: int) -> None:
    if s != GA_OK:
        raise GAError(s, lib().ga_last_error().decode())


def compute_info(W: int, layer_numels: Sequence[int], fp16: bool, chunk: int = 0,
                 keep_ratio: float = 0.0) -> PlanInfo:
    """Plan sizes without touching a device."""
    arr = (ctypes.c_int64 * len(layer_numels))(*[int(n) for n in layer_numels])
    info = PlanInfo()
    _check(lib().ga_plan_compute_info(W, len(layer_numels), arr, GA_FP16 if fp16 else GA_FP32, chunk,
                                      keep_ratio, ctypes.byref(info)))
    return info


def bucket_boundaries(layer_numels: Sequence[int], fp16: bool, bucket_bytes: int):
    """First layer of every bucket, the bucket holding the last layer first
    (host only; the rule is ga_bucket_boundaries')."""
    n = len(layer_numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in layer_numels])
    first = (ctypes.c_int32 * max(n, 1))()
    nb = ctypes.c_int32(0)
    _check(lib().ga_bucket_boundaries(n, arr, 2 if fp16 else 4, int(bucket_bytes), first, ctypes.byref(nb)))
    return [int(first[b]) for b in range(nb.value)]


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _dev(t, dtype, min_numel: int, name: str):
    """Address of a contiguous CUDA tensor of `dtype` with at least min_numel elements."""
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < min_numel:
        raise ValueError("%s has %d elements, needs %d" % (name, t.numel(), min_numel))
    return t.data_ptr()


class Plan:
    """Sizes and the device layer table for W workers and a layer list.

    layer_numels: element count of every layer, in fusion order.
    fp16: gradients travel as binary16 (summed in binary32) instead of binary32.
    chunk: chunk size in elements for the sparse path (0: dense only).
    keep_ratio: fraction of chunks each worker sends.
    """

    def __init__(self, W: int, layer_numels: Sequence[int], fp16: bool, chunk: int = 0,
                 keep_ratio: float = 0.0):
        torch = _torch()
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU: the gradient-aggregation library runs on the GPU only")
        arr = (ctypes.c_int64 * len(layer_numels))(*[int(n) for n in layer_numels])
        h = _VP()
        _check(lib().ga_plan_create(W, len(layer_numels), arr, GA_FP16 if fp16 else GA_FP32, chunk,
                                    keep_ratio, ctypes.byref(h)))
        self._h = h
        info = PlanInfo()
        _check(lib().ga_plan_get_info(h, ctypes.byref(info)))
        self.info = info
        self.W, self.P, self.ld = info.W, info.P, info.ld
        self.chunk, self.n_chunks, self.k, self.mask_words = info.chunk, info.n_chunks, info.k, info.mask_words
        self.fp16 = fp16
        self.layer_numels = [int(n) for n in layer_numels]

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().ga_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- buffers ---------------------------------------------------------
    @property
    def grad_dtype(self):
        torch = _torch()
        return torch.float16 if self.fp16 else torch.float32

    def empty_bucket(self, device="cuda"):
        return _torch().zeros((self.W, self.ld), dtype=self.grad_dtype, device=device)

    def empty_residual(self, device="cuda"):
        return _torch().zeros((self.W, self.ld), dtype=_torch().float32, device=device)

    def empty_keys(self, device="cuda"):
        return _torch().empty((self.W, self.n_chunks), dtype=_torch().float64, device=device)

    def empty_sel(self, device="cuda"):
        torch = _torch()
        return (torch.empty((self.W, max(self.k, 1)), dtype=torch.int32, device=device),
                torch.zeros((self.W, self.mask_words), dtype=torch.int32, device=device))

    # ---- calls -------------------------------------------------------------
    def bucket_pack(self, layer_ptrs, bucket) -> None:
        """layer_ptrs: int64 tensor of W*L device addresses, worker-major."""
        torch = _torch()
        L = len(self.layer_numels)
        _check(lib().ga_bucket_pack(self._h, _dev(layer_ptrs, torch.int64, self.W * L, "layer_ptrs"),
                                    _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"), _stream_ptr()))

    def tree_reduce(self, bucket, grad=None, w=None, v=None, lr: Optional[float] = None,
                    mu: Optional[float] = None) -> None:
        torch = _torch()
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        _check(lib().ga_tree_reduce(self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
                                    _dev(grad, torch.float32, self.P, "grad"), sgd,
                                    _dev(w, torch.float32, self.P, "w"), _dev(v, torch.float32, self.P, "v"),
                                    _stream_ptr()))

    def tree_partial(self, bucket, out) -> None:
        """Unscaled tree sum S of the W rows of bucket into out ([P] float32):
        one GPU's part of the dense step split across GPUs."""
        torch = _torch()
        _check(lib().ga_tree_partial(self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
                                     _dev(out, torch.float32, self.P, "out"), _stream_ptr()))

    def tree_combine(self, partials, w_total: int, grad=None, w=None, v=None, lr: Optional[float] = None,
                     mu: Optional[float] = None) -> None:
        """The owner's step of the split dense step: the tree over the W rows of
        partials ([W][ld] float32, this plan binary32), mean over w_total
        workers, SGD on this slice."""
        torch = _torch()
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        _check(lib().ga_tree_combine(self._h, _dev(partials, torch.float32, self.W * self.ld, "partials"),
                                     int(w_total), _dev(grad, torch.float32, self.P, "grad"), sgd,
                                     _dev(w, torch.float32, self.P, "w"), _dev(v, torch.float32, self.P, "v"),
                                     _stream_ptr()))

    def tree_reduce_layers(self, layer_ptrs, grad=None, w=None, v=None, lr: Optional[float] = None,
                           mu: Optional[float] = None) -> None:
        """tree_reduce reading the leaves straight from the per-layer tensors
        (layer_ptrs: int64 tensor of W*L device addresses, worker-major)."""
        torch = _torch()
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        L = len(self.layer_numels)
        _check(lib().ga_tree_reduce_layers(self._h, _dev(layer_ptrs, torch.int64, self.W * L, "layer_ptrs"),
                                           _dev(grad, torch.float32, self.P, "grad"), sgd,
                                           _dev(w, torch.float32, self.P, "w"), _dev(v, torch.float32, self.P, "v"),
                                           _stream_ptr()))

    def reduce_variant(self, bucket, order: str = "tree", wire16: bool = False, grad=None, w=None, v=None,
                       lr: Optional[float] = None, mu: Optional[float] = None) -> None:
        """Dense aggregation in another summation order ("tree", "server" or
        "ring"), optionally with a binary16 wire."""
        torch = _torch()
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        _check(lib().ga_reduce_variant(self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
                                       ORDERS[order], int(bool(wire16)), _dev(grad, torch.float32, self.P, "grad"),
                                       sgd, _dev(w, torch.float32, self.P, "w"), _dev(v, torch.float32, self.P, "v"),
                                       _stream_ptr()))

    def chunk_norm_layers(self, layer_ptrs, resid, keys, prev_mask=None) -> None:
        """chunk_norm reading the gradient straight from the per-layer tensors."""
        torch = _torch()
        L = len(self.layer_numels)
        _check(lib().ga_chunk_norm_layers(self._h, _dev(layer_ptrs, torch.int64, self.W * L, "layer_ptrs"),
                                          _dev(resid, torch.float32, self.W * self.ld, "resid"),
                                          _dev(prev_mask, torch.int32, self.W * self.mask_words, "prev_mask"),
                                          _dev(keys, torch.float64, self.W * self.n_chunks, "keys"), _stream_ptr()))

    def history(self, masks, layer_tables=()):
        """A ga_history: masks[j] = selection of step t-1-j (int32 [W][mw]
        tensor or None), j = 0..age; layer_tables[j] = layer table of step
        t-1-j, j = 0..age-1.  age = len(masks) - 1."""
        torch = _torch()
        age = len(masks) - 1
        if age < 0 or age > MAX_AGE:
            raise ValueError("history needs 1..%d masks" % (MAX_AGE + 1))
        if len(layer_tables) != age:
            raise ValueError("age %d needs %d earlier layer tables, got %d" % (age, age, len(layer_tables)))
        h = History()
        h.age = age
        n = self.W * len(self.layer_numels)
        for j, m in enumerate(masks):
            h.d_masks[j] = _dev(m, torch.int32, self.W * self.mask_words, "mask %d" % j)
        for j, t in enumerate(layer_tables):
            h.d_layer_ptrs[j] = _dev(t, torch.int64, n, "layer table %d" % j)
        return h

    def chunk_norm_deferred(self, layer_ptrs, hist, store: bool, resid, keys) -> None:
        """Deferred-residual norm pass of one step (hist from history())."""
        torch = _torch()
        n = self.W * len(self.layer_numels)
        _check(lib().ga_chunk_norm_deferred(self._h, _dev(layer_ptrs, torch.int64, n, "layer_ptrs"),
                                            ctypes.byref(hist), int(bool(store)),
                                            _dev(resid, torch.float32, self.W * self.ld, "resid"),
                                            _dev(keys, torch.float64, self.W * self.n_chunks, "keys"),
                                            _stream_ptr()))

    def sparse_gather_reduce_deferred(self, layer_ptrs, hist, stored: bool, resid, sel_mask, grad=None, w=None,
                                      v=None, lr: Optional[float] = None, mu: Optional[float] = None) -> None:
        """Deferred-residual gather-reduce of one step (hist and stored as given
        to its norm pass)."""
        torch = _torch()
        n = self.W * len(self.layer_numels)
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        _check(lib().ga_sparse_gather_reduce_deferred(
            self._h, _dev(layer_ptrs, torch.int64, n, "layer_ptrs"), ctypes.byref(hist), int(bool(stored)),
            _dev(resid, torch.float32, self.W * self.ld, "resid"),
            _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"),
            _dev(grad, torch.float32, self.P, "grad"), sgd, _dev(w, torch.float32, self.P, "w"),
            _dev(v, torch.float32, self.P, "v"), _stream_ptr()))

    def residual_flush(self, layer_ptrs, hist, stored: bool, resid, sel_mask) -> None:
        """Write the residual after a deferred step (zero on the sent chunks)."""
        torch = _torch()
        n = self.W * len(self.layer_numels)
        _check(lib().ga_residual_flush(self._h, _dev(layer_ptrs, torch.int64, n, "layer_ptrs"), ctypes.byref(hist),
                                       int(bool(stored)), _dev(resid, torch.float32, self.W * self.ld, "resid"),
                                       _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"),
                                       _stream_ptr()))

    def chunk_norm(self, bucket, resid, keys, prev_mask=None) -> None:
        torch = _torch()
        _check(lib().ga_chunk_norm(self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
                                   _dev(resid, torch.float32, self.W * self.ld, "resid"),
                                   _dev(prev_mask, torch.int32, self.W * self.mask_words, "prev_mask"),
                                   _dev(keys, torch.float64, self.W * self.n_chunks, "keys"), _stream_ptr()))

    def chunk_topk(self, keys, sel_idx, sel_mask) -> None:
        torch = _torch()
        _check(lib().ga_chunk_topk(self._h, _dev(keys, torch.float64, self.W * self.n_chunks, "keys"),
                                   _dev(sel_idx, torch.int32, self.W * self.k, "sel_idx"),
                                   _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"),
                                   _stream_ptr()))

    def chunk_norm_topk(self, bucket, resid, keys, sel_idx, sel_mask, prev_mask=None) -> None:
        torch = _torch()
        _check(lib().ga_chunk_norm_topk(
            self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
            _dev(resid, torch.float32, self.W * self.ld, "resid"),
            _dev(prev_mask, torch.int32, self.W * self.mask_words, "prev_mask"),
            _dev(keys, torch.float64, self.W * self.n_chunks, "keys"),
            _dev(sel_idx, torch.int32, self.W * self.k, "sel_idx"),
            _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"), _stream_ptr()))

    def chunk_norm_topk_static(self, bucket, resid, sel_idx, sel_mask, prev_mask=None) -> None:
        """chunk_norm_topk with the keys (and the partial sums of chunks longer
        than 2048 elements) in the library's fixed array (no allocation;
        concurrent calls on one device race)."""
        torch = _torch()
        _check(lib().ga_chunk_norm_topk_static(
            self._h, _dev(bucket, self.grad_dtype, self.W * self.ld, "bucket"),
            _dev(resid, torch.float32, self.W * self.ld, "resid"),
            _dev(prev_mask, torch.int32, self.W * self.mask_words, "prev_mask"),
            _dev(sel_idx, torch.int32, self.W * self.k, "sel_idx"),
            _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"), _stream_ptr()))

    def sparse_gather_reduce(self, resid, sel_mask, zero_selected: bool = True, grad=None, w=None, v=None,
                             lr: Optional[float] = None, mu: Optional[float] = None) -> None:
        torch = _torch()
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        _check(lib().ga_sparse_gather_reduce(
            self._h, _dev(resid, torch.float32, self.W * self.ld, "resid"),
            _dev(sel_mask, torch.int32, self.W * self.mask_words, "sel_mask"), int(bool(zero_selected)),
            _dev(grad, torch.float32, self.P, "grad"), sgd, _dev(w, torch.float32, self.P, "w"),
            _dev(v, torch.float32, self.P, "v"), _stream_ptr()))


class DeferredResidual:
    """Buffer rotation of the deferred-residual step (host bookkeeping only).

    Keeps `depth` earlier gradient batches: the norm pass stores a every
    depth+1 steps, the other steps re-form the residual from the held layer
    tables and masks.  The caller passes each step's layer table and keeps its
    tensors unchanged while they are in the history (the next `depth` steps).
    Without `resid` the residual starts at zero, described by an all-ones mask
    (every chunk "sent" before the first step), so the buffer is not read
    until written; a given `resid` (a flushed residual, say from a checkpoint)
    is the starting residual itself, read at age 0.  depth = 0 is the
    lazy-zero form."""

    def __init__(self, plan: Plan, depth: int, resid=None):
        torch = _torch()
        if depth < 0 or depth > MAX_AGE:
            raise ValueError("depth must be in [0, %d]" % MAX_AGE)
        self.plan, self.depth = plan, depth
        W, mw = plan.W, plan.mask_words
        self.resid = plan.empty_residual() if resid is None else resid
        self.keys = plan.empty_keys()
        self.sel_idx = torch.empty((W, max(plan.k, 1)), dtype=torch.int32, device="cuda")
        self.masks = [torch.zeros((W, mw), dtype=torch.int32, device="cuda") for _ in range(depth + 2)]
        words = []
        for q in range(mw):
            word = (1 << min(32, plan.n_chunks - 32 * q)) - 1
            words.append(word - (1 << 32) if word >= (1 << 31) else word)
        self.all_sent = torch.tensor(words, dtype=torch.int32).repeat(W, 1).cuda()
        # masks[j]: step t-1-j; None at age 0: the buffer holds the residual
        self.hist_masks = [self.all_sent] if resid is None else [None]
        self.hist_tables = []               # layer tables of steps t-1, t-2, ...
        self.next = 0                       # mask buffer the next top-k writes
        # (hist, stored, layer_ptrs, sel) of the last step; None while the
        # residual is the starting one or was flushed in place since
        self.last = None

    @property
    def age(self) -> int:
        return len(self.hist_masks) - 1

    def step(self, layer_ptrs, grad=None, w=None, v=None, lr=None, mu=None, events=None) -> bool:
        """One step on the current stream; returns whether it stored.  events:
        optional list of 3 torch.cuda.Event recorded after each call."""
        p = self.plan
        hist = p.history(self.hist_masks, self.hist_tables)
        store = self.age >= self.depth
        p.chunk_norm_deferred(layer_ptrs, hist, store, self.resid, self.keys)
        if events:
            events[0].record()
        sel = self.masks[self.next]
        p.chunk_topk(self.keys, self.sel_idx, sel)
        if events:
            events[1].record()
        p.sparse_gather_reduce_deferred(layer_ptrs, hist, store, self.resid, sel, grad, w, v, lr, mu)
        if events:
            events[2].record()
        self.last = (hist, store, layer_ptrs, sel)
        if store:
            self.hist_masks, self.hist_tables = [sel], []
        else:
            self.hist_masks = [sel] + self.hist_masks
            self.hist_tables = [layer_ptrs] + self.hist_tables
        self.next = (self.next + 1) % len(self.masks)
        return store

    def flush(self, out=None):
        """Write the residual after the last step into `out` (default: the live
        buffer, after which the history restarts at age 0 with no mask, so a
        second flush changes nothing).  Before any step it is the starting
        residual: zero, or the given one."""
        if self.last is None:
            zero_start = self.hist_masks[0] is not None
            target = self.resid if out is None else out
            if zero_start:
                target.zero_()
            elif target.data_ptr() != self.resid.data_ptr():
                target.copy_(self.resid)
            if out is None:
                self.hist_masks, self.hist_tables = [None], []
            return target
        hist, stored, layer_ptrs, sel = self.last
        if out is None:
            self.plan.residual_flush(layer_ptrs, hist, stored, self.resid, sel)
            self.hist_masks, self.hist_tables = [None], []
            self.last = None
            return self.resid
        if out.data_ptr() != self.resid.data_ptr():
            out.copy_(self.resid)
        self.plan.residual_flush(layer_ptrs, hist, stored, out, sel)
        return out


class Buckets:
    """Multi-bucket schedule of a plan: layers grouped from the last one down
    into buckets of at least bucket_bytes per worker, each reduced on its own
    once its layers are ready."""

    def __init__(self, plan: Plan, bucket_bytes: int):
        h = _VP()
        _check(lib().ga_buckets_create(plan._h, int(bucket_bytes), ctypes.byref(h)))
        self._h = h
        self.plan = plan
        self.count = int(lib().ga_buckets_count(h))
        self.ranges = []
        for b in range(self.count):
            f, n, e0, e1 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
            _check(lib().ga_bucket_range(h, b, ctypes.byref(f), ctypes.byref(n), ctypes.byref(e0),
                                         ctypes.byref(e1)))
            self.ranges.append((f.value, n.value, e0.value, e1.value))

    def __len__(self) -> int:
        return self.count

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().ga_buckets_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reduce_layers(self, b: int, layer_ptrs, ready=None, grad=None, w=None, v=None,
                      lr: Optional[float] = None, mu: Optional[float] = None, max_workgroups: int = 0) -> None:
        """Reduce bucket b on the current stream, after `ready` (a
        torch.cuda.Event, or None) has completed; max_workgroups > 0 caps the
        grid."""
        torch = _torch()
        p = self.plan
        sgd = None if lr is None else ctypes.byref(SGD(lr, mu))
        ev = None if ready is None else ready.cuda_event
        _check(lib().ga_bucket_reduce_layers(self._h, int(b),
                                             _dev(layer_ptrs, torch.int64, p.W * len(p.layer_numels), "layer_ptrs"),
                                             ev, _dev(grad, torch.float32, p.P, "grad"), sgd,
                                             _dev(w, torch.float32, p.P, "w"), _dev(v, torch.float32, p.P, "v"),
                                             int(max_workgroups), _stream_ptr()))


def sgd_momentum_apply(grad, w, v, lr: float, mu: float) -> None:
    torch = _torch()
    P = w.numel()
    _check(lib().ga_sgd_momentum_apply(P, _dev(grad, torch.float32, P, "grad"), _dev(w, torch.float32, P, "w"),
                                       _dev(v, torch.float32, P, "v"), ctypes.byref(SGD(lr, mu)), _stream_ptr()))
