"""Pins of the oracle's other summation orders (parameter server, ring) and of
the binary16 wire: hand-derived fixtures, numpy's binary16 rounding, exact
integer sums, the ring-as-rotated-server identity, and error growth."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixtures():
    rows = []
    with open(os.path.join(GOLDEN, "variant_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            W, P, e, vals, order, wire, s = [p.strip() for p in line.split(";")]
            rows.append((int(W), int(P), int(e), [float.fromhex(x) for x in vals.split()], order, wire,
                         float.fromhex(s)))
    return rows


@pytest.mark.parametrize("row", _fixtures(), ids=lambda r: "W%d-%s-%s-e%d" % (r[0], r[4], r[5], r[2]))
def test_variant_fixtures(row):
    W, P, e, vals, order, wire, s = row
    b = np.repeat(np.array(vals, np.float32)[:, None], P, axis=1)
    g = oracle.reduce_variant(b, P, False, order, wire == "f16")
    assert g[e] == np.float32(s) * np.float32(1.0 / W)


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(0)
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[1:] + h[:-1]) / 2).astype(np.float32)
    x = np.concatenate([mids, -mids[::7], rng.standard_normal(20000).astype(np.float32) * 1e-3,
                        (rng.standard_normal(20000) * 1e-6).astype(np.float32),
                        (rng.standard_normal(5000) * 3e4).astype(np.float32),
                        np.array([65504, 65519, 65520, 1e9, -0.0, 0.0, 1e-45, np.inf, -np.inf], np.float32)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float32)
    got = oracle.round_f16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(oracle.round_f16(np.array([np.nan], np.float32))[0])


@pytest.mark.parametrize("order", ["tree", "ps", "ring"])
@pytest.mark.parametrize("wire", [False, True])
@pytest.mark.parametrize("W", [1, 2, 3, 5, 8, 32])
def test_variants_exact_on_small_integers(order, wire, W):
    """Partial sums of integers |x| <= 64 over W <= 32 workers stay within 2048,
    exact in binary16 and binary32: every order and wire gives the exact sum."""
    rng = np.random.default_rng(W)
    P = 700
    b = rng.integers(-64, 65, size=(W, P)).astype(np.float32)
    g = oracle.reduce_variant(b, P, False, order, wire)
    exact = b.astype(np.int64).sum(axis=0)
    assert np.array_equal(g, exact.astype(np.float32) * np.float32(1.0 / W))


def test_tree_without_wire_is_the_dense_step():
    rng = np.random.default_rng(1)
    for W in (1, 3, 16, 100):
        b = (rng.standard_normal((W, 1000)) * np.exp2(rng.integers(-20, 20, (W, 1000)))).astype(np.float32)
        assert np.array_equal(oracle.reduce_variant(b, 1000, False, "tree", False),
                              oracle.dense_step(b, 1000, False, 0.0, 0.0, None, None))


def test_ring_is_the_server_order_rotated_per_segment():
    rng = np.random.default_rng(2)
    W, P = 7, 1000
    b = (rng.standard_normal((W, P)) * np.exp2(rng.integers(-20, 20, (W, P)))).astype(np.float32)
    Q = oracle.ring_segment(W, P)
    assert Q == 192
    ring = oracle.reduce_variant(b, P, False, "ring", False)
    for s in range((P + Q - 1) // Q):
        rows = [(s + 1 + j) % W for j in range(W)]
        ps = oracle.reduce_variant(np.ascontiguousarray(b[rows]), P, False, "ps", False)
        lo, hi = s * Q, min((s + 1) * Q, P)
        assert np.array_equal(ring[lo:hi], ps[lo:hi])


def test_server_order_is_sequential():
    """The server's order shows in rounding: its error grows with W, the
    tree's with log2 W (checked in aggregate on random data)."""
    rng = np.random.default_rng(3)
    W, P = 128, 20000
    b = rng.standard_normal((W, P)).astype(np.float32)
    exact = b.astype(np.float64).sum(axis=0) / W
    err = {o: np.sqrt(np.mean((oracle.reduce_variant(b, P, False, o, False) - exact) ** 2)) for o in ("tree", "ps")}
    assert err["ps"] > 2 * err["tree"]
    seq = b[0].copy()
    for w in range(1, W):
        seq = seq + b[w]
    assert np.array_equal(oracle.reduce_variant(b, P, False, "ps", False), seq * np.float32(1.0 / W))


@pytest.mark.parametrize("order,wire", [("tree", True), ("tree", False), ("ps", True), ("ps", False),
                                        ("ring", False)])
def test_identical_power_of_two_buffers(order, wire):
    """W identical binary16 rows, W a power of two: the tree's partial sums are
    2^j x and the server's k x (k <= 64) are exact in binary32, and only the
    tree's 2^j x are sent over the wire, so each mean is x exactly.  (The ring
    with a binary16 wire sends k x, which binary16 may round.)"""
    rng = np.random.default_rng(4)
    row = rng.standard_normal(500).astype(np.float16)
    for W in (2, 8, 64):
        b = np.tile(row.view(np.uint16), (W, 1))
        g = oracle.reduce_variant(b, 500, True, order, wire)
        assert np.array_equal(g, row.astype(np.float32))
