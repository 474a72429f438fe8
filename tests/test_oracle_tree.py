"""Pins of the oracle's reduction tree and dense step against facts that do not
come from the oracle itself: hand-derived fixtures, exact integer sums, a
level-by-level formulation of the tree, error bounds and exhaustive decoding.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_tree_fixture():
    rows = []
    with open(os.path.join(GOLDEN, "tree_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            W, leaves, s, m = [p.strip() for p in line.split(";")]
            rows.append((int(W), [float.fromhex(x) for x in leaves.split()], float.fromhex(s),
                         None if m == "-" else float.fromhex(m)))
    return rows


def level_pairing(leaves: np.ndarray) -> np.ndarray:
    """The tree as a level-by-level pairing of adjacent nodes (binary32 adds),
    an odd last node carried up: a second formulation of the same tree."""
    level = [np.asarray(r, np.float32) for r in leaves]
    while len(level) > 1:
        nxt = [level[i] + level[i + 1] for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def test_fp16_decode_exhaustive():
    """All 65536 binary16 patterns decode like numpy's float16 -> float32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # subnormals survive (smallest is 2^-24) and signed zero keeps its sign
    assert oracle.f16_decode(np.array([1], np.uint16))[0] == np.float32(2.0 ** -24)
    assert np.signbit(oracle.f16_decode(np.array([0x8000], np.uint16))[0])


@pytest.mark.parametrize("row", _read_tree_fixture(), ids=lambda r: "W%d" % r[0])
def test_tree_golden(row):
    W, leaves, s, m = row
    x = np.array(leaves, np.float32).reshape(W, 1)
    assert oracle.tree_sum(x)[0] == np.float32(s)
    if m is not None:
        g = oracle.dense_step(x.copy(), 1, False, 0.0, 0.0, None, None)
        assert g[0] == np.float32(m)


def _spread(rng, W, n):
    """Values whose binary32 sums depend on the summation order."""
    e = rng.integers(-30, 30, size=(W, n))
    return (rng.choice([-1.0, 1.0], size=(W, n)) * rng.random((W, n)) * np.exp2(e)).astype(np.float32)


def test_tree_equals_level_pairing_w1_to_300():
    rng = np.random.default_rng(0)
    for W in range(1, 301):
        x = _spread(rng, W, 64)
        a = oracle.tree_sum(x)
        b = level_pairing(x)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), W


def test_tree_is_not_sequential_order():
    """Sanity of the pin above: the data does distinguish summation orders."""
    rng = np.random.default_rng(1)
    x = _spread(rng, 16, 4096)
    seq = x[0].copy()
    for w in range(1, 16):
        seq = seq + x[w]
    assert not np.array_equal(oracle.tree_sum(x), seq)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 7, 8, 16, 33, 128])
def test_tree_integer_inputs_exact(W):
    rng = np.random.default_rng(W)
    x = rng.integers(-1024, 1025, size=(W, 257)).astype(np.float32)
    exact = x.astype(np.int64).sum(axis=0)
    assert np.array_equal(oracle.tree_sum(x), exact.astype(np.float32))


def test_tree_error_bound():
    """|S - sum| <= gamma_d * sum|x|, d = ceil(log2 W): pairwise summation."""
    rng = np.random.default_rng(3)
    u = 2.0 ** -24
    for W in (3, 16, 100, 128):
        x = rng.standard_normal((W, 200)).astype(np.float32)
        s = oracle.tree_sum(x)
        d = math.ceil(math.log2(W))
        gamma = d * u / (1 - d * u)
        for i in range(0, 200, 7):
            exact = sum(Fraction(float(v)) for v in x[:, i])
            absum = sum(abs(Fraction(float(v))) for v in x[:, i])
            assert abs(Fraction(float(s[i])) - exact) <= Fraction(gamma) * absum


@pytest.mark.parametrize("W", [1, 2, 4, 8, 32, 128])
@pytest.mark.parametrize("fp16", [False, True])
def test_identical_power_of_two_buffers_average_to_themselves(W, fp16):
    rng = np.random.default_rng(W)
    row = rng.standard_normal(1000).astype(np.float32) * np.float32(1e-3)
    if fp16:
        row16 = row.astype(np.float16)
        bucket = np.tile(row16.view(np.uint16), (W, 1))
        expect = row16.astype(np.float32)
    else:
        bucket = np.tile(row, (W, 1))
        expect = row
    g = oracle.dense_step(bucket, 1000, fp16, 0.0, 0.0, None, None)
    assert np.array_equal(g.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("W", [2, 3, 8, 128])
def test_dense_fp16_integers_exact(W):
    """binary16 leaves holding integers |x| <= 2048 sum exactly in binary32."""
    rng = np.random.default_rng(10 + W)
    x = rng.integers(-2048, 2049, size=(W, 300)).astype(np.float16)
    exact = x.astype(np.int64).sum(axis=0)
    g = oracle.dense_step(x.view(np.uint16).copy(), 300, True, 0.0, 0.0, None, None)
    if W & (W - 1) == 0:
        assert np.array_equal(g, (exact / W).astype(np.float32))
    assert np.array_equal(g, exact.astype(np.float32) * np.float32(1.0 / W))


def test_dense_ignores_row_padding_and_thread_count():
    rng = np.random.default_rng(5)
    W, P, ld = 6, 1000, 1024
    b = rng.standard_normal((W, ld)).astype(np.float32)
    b2 = b.copy()
    b2[:, P:] = np.nan
    w = rng.standard_normal(P).astype(np.float32)
    v = rng.standard_normal(P).astype(np.float32)
    w1, v1, w2, v2 = w.copy(), v.copy(), w.copy(), v.copy()
    g1 = oracle.dense_step(b, P, False, 0.01, 0.9, w1, v1, threads=1)
    g2 = oracle.dense_step(b2, P, False, 0.01, 0.9, w2, v2, threads=7)
    assert np.array_equal(g1, g2) and np.array_equal(w1, w2) and np.array_equal(v1, v2)


def test_dense_nonfinite_propagates():
    b = np.zeros((4, 8), np.float32)
    b[1, 0] = np.inf
    b[2, 1] = np.nan
    b[0, 2], b[3, 2] = np.inf, -np.inf
    g = oracle.dense_step(b, 8, False, 0.0, 0.0, None, None)
    assert g[0] == np.inf and np.isnan(g[1]) and np.isnan(g[2])
