"""The seeded input generator: determinism, rounding and distributions."""
import math

import numpy as np

import workloads


def test_f32_to_f16_matches_numpy_rne():
    """The generator's binary16 rounding equals numpy's (IEEE round-to-nearest-even),
    including every exact midpoint between neighbouring binary16 values."""
    L = workloads.lib()
    rng = np.random.default_rng(1)
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[1:] + h[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e-3),
        (rng.standard_normal(20000) * 1e-6).astype(np.float32),
        (rng.standard_normal(5000) * 3e4).astype(np.float32),
        mids, -mids,
        np.array([65504, 65519, 65520, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
                  2.0 ** -14 - 2.0 ** -25, 1e-40, -0.0, 0.0, np.inf, -np.inf], np.float32)])
    mine = np.array([L.gagen_f32_to_f16(float(v)) for v in vals], np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_streams_deterministic_and_thread_invariant():
    wl = workloads.WORKLOADS["tiny"]
    a = workloads.grad_row(wl, 1, 2, threads=1)
    b = workloads.grad_row(wl, 1, 2, threads=7)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = workloads.grad_row(wl, 2, 2)
    d = workloads.grad_row(wl, 1, 3)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_fill_offset_consistency():
    """Filling from an odd start gives the same elements as a fill from 0."""
    key = workloads.lib().gagen_key(5, 1, 1, 0)
    full = workloads.fill(np.empty(1001, np.float32), key, 0, 1.0, np.zeros(0, np.int64), np.zeros(0))
    part = workloads.fill(np.empty(400, np.float32), key, 301, 1.0, np.zeros(0, np.int64), np.zeros(0))
    assert np.array_equal(full[301:701], part)
    L = workloads.lib()
    for e in (0, 1, 2, 301, 1000):
        assert np.float32(L.gagen_normal(key, e)) == full[e]


def test_normal_moments():
    key = workloads.lib().gagen_key(7, 1, 1, 0)
    x = workloads.fill(np.empty(400000, np.float32), key, 0, 1.0, np.zeros(0, np.int64), np.zeros(0))
    assert abs(float(x.mean())) < 0.01
    assert abs(float(x.std()) - 1.0) < 0.01
    assert abs(float((np.abs(x) < 1.0).mean()) - math.erf(1 / math.sqrt(2))) < 0.005


def test_layer_scales_loguniform_range():
    wl = workloads.WORKLOADS["alexnet16"]
    ends, sc = workloads.segments(wl)
    assert list(ends) == list(np.cumsum(wl.numels))
    assert np.all(sc >= 0.1) and np.all(sc <= 10.0)


def test_chunk_scales_distinct_shared():
    wl = workloads.WORKLOADS["alexnet128_sparse"]
    ends, sc = workloads.segments(wl)
    assert len(sc) == 1861 and ends[-1] == wl.P and ends[0] == 32768
    assert len(set(sc.tolist())) == len(sc)
    assert sc.min() >= 1e-4 and sc.max() <= 1.0
    # log-uniform: log10 roughly uniform on [-4, 0]
    lg = np.log10(sc)
    assert abs(float(lg.mean()) + 2.0) < 0.15


def test_weights_sigma():
    wl = workloads.WORKLOADS["nin"]
    w = workloads.weights(wl)
    assert w.dtype == np.float32 and w.size == wl.P
    assert abs(float(w.std()) - 0.05) < 1e-3
