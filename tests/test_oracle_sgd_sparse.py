"""Pins of the oracle's momentum SGD, chunk keys, top-k selection, residual
split and fusion against closed forms, exact rational arithmetic, library sorts
and the invariants of the method (keep ratio 1 is the dense path, keep ratio 0
sends nothing, residual plus transmitted equals the input)."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


# ----------------------------------------------------------------------------
# momentum SGD
# ----------------------------------------------------------------------------

def test_sgd_caffe_form_exact_dyadic():
    """With dyadic values every operation is exact, so the oracle must equal the
    Caffe-form update in rational arithmetic: v <- mu v + lr g; w <- w - v."""
    rng = np.random.default_rng(0)
    g = (rng.integers(-64, 64, 500) / 64.0).astype(np.float32)
    w = (rng.integers(-64, 64, 500) / 8.0).astype(np.float32)
    v = (rng.integers(-64, 64, 500) / 16.0).astype(np.float32)
    lr, mu = 0.25, 0.5
    w_ex = [Fraction(float(x)) for x in w]
    v_ex = [Fraction(float(x)) for x in v]
    oracle.sgd(g, w, v, lr, mu)
    for i in range(500):
        vn = Fraction(mu) * v_ex[i] + Fraction(lr) * Fraction(float(g[i]))
        assert Fraction(float(v[i])) == vn
        assert Fraction(float(w[i])) == w_ex[i] - vn


def test_sgd_first_step_from_zero_velocity():
    rng = np.random.default_rng(1)
    g = rng.standard_normal(1000).astype(np.float32)
    w = rng.standard_normal(1000).astype(np.float32)
    w0 = w.copy()
    v = np.zeros(1000, np.float32)
    oracle.sgd(g, w, v, 0.01, 0.9)
    assert np.array_equal(v, np.float32(0.01) * g)          # one rounding of lr*g
    assert np.array_equal(w, w0 - v)


def test_sgd_constant_gradient_geometric_series():
    """v_n -> lr g (1 - mu^n) / (1 - mu) within a few ulps per step."""
    g = np.full(4, 0.37, np.float32)
    w = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    lr, mu = np.float32(0.01), np.float32(0.9)
    for n in range(1, 40):
        oracle.sgd(g, w, v, lr, mu)
        ref = float(lr) * float(g[0]) * (1 - float(mu) ** n) / (1 - float(mu))
        assert abs(float(v[0]) - ref) <= n * 4 * 2.0 ** -24 * abs(ref) * 10


def test_sgd_mu_zero_is_plain_sgd():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(100).astype(np.float32)
    w = rng.standard_normal(100).astype(np.float32)
    w0 = w.copy()
    v = rng.standard_normal(100).astype(np.float32)
    oracle.sgd(g, w, v, 0.5, 0.0)
    assert np.array_equal(w, w0 - np.float32(0.5) * g)


# ----------------------------------------------------------------------------
# chunk keys (squared L2 norms)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("e", [-60, -20, -1, 0, 7, 60])
@pytest.mark.parametrize("n", [1, 3, 32768])
def test_key_of_constant_power_of_two_chunk(e, n):
    a = np.full(n, 2.0 ** e, np.float32)
    assert oracle.chunk_key(a) == n * 2.0 ** (2 * e)


def test_key_is_rounded_exact_sum_of_squares():
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(1, 60))
        a = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
        exact = sum(Fraction(float(x)) ** 2 for x in a)
        k = oracle.chunk_key(a)
        assert abs(Fraction(k) - exact) <= Fraction(np.spacing(float(exact)))


def test_key_nonfinite():
    a = np.ones(10, np.float32)
    a[3] = np.inf
    assert oracle.chunk_key(a) == np.inf
    a[4] = np.nan
    assert np.isnan(oracle.chunk_key(a))
    assert oracle.chunk_key(np.zeros(5, np.float32)) == 0.0


# ----------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------

def _lib_topk(keys, k):
    order = sorted(range(len(keys)), key=lambda c: (0 if np.isnan(keys[c]) else 1,
                                                    -keys[c] if not np.isnan(keys[c]) else 0, c))
    return sorted(order[:k])


def test_keep_count():
    assert oracle.keep_count(1861, 0.1) == 187
    assert oracle.keep_count(10, 1.0) == 10
    assert oracle.keep_count(10, 0.0) == 0
    assert oracle.keep_count(4, 0.25) == 1
    assert oracle.keep_count(3, 0.5) == 2
    assert oracle.keep_count(10, 0.3) == 3       # 0.3*10 is 3.0000000000000004 in binary64
    assert oracle.keep_count(459, 0.25) == 115
    assert oracle.keep_count(0, 0.5) == 0


def test_topk_matches_library_sort():
    rng = np.random.default_rng(5)
    for trial in range(50):
        n = int(rng.integers(1, 3000))
        keys = rng.random(n) * np.exp2(rng.integers(-30, 30, n))
        if trial % 3 == 0:
            keys = np.round(keys * 4) / 4          # plenty of exact ties
        k = int(rng.integers(0, n + 1))
        idx, m = oracle.topk(keys, k)
        assert list(idx) == _lib_topk(keys, k)


def test_topk_special_cases():
    keys = np.array([3.0, 9.0, 9.0, 1.0, 0.0])
    assert list(oracle.topk(keys, 1)[0]) == [int(np.argmax(keys))]
    assert list(oracle.topk(keys, 2)[0]) == [1, 2]
    assert list(oracle.topk(np.zeros(10), 4)[0]) == [0, 1, 2, 3]
    assert list(oracle.topk(keys, 5)[0]) == [0, 1, 2, 3, 4]
    assert list(oracle.topk(np.array([1.0, np.nan, np.inf, 2.0]), 2)[0]) == [1, 2]
    idx, m = oracle.topk(np.array([4.0, 1.0, 3.0]), 2)
    assert m == (3.0 - 1.0) / 3.0
    assert oracle.topk(np.array([2.0, 2.0, 1.0]), 1)[1] == 0.0


# ----------------------------------------------------------------------------
# sparse step
# ----------------------------------------------------------------------------

def _level_pairing(leaves):
    level = [np.asarray(r, np.float32) for r in leaves]
    while len(level) > 1:
        nxt = [level[i] + level[i + 1] for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def _mask_to_chunks(mask_row, n_c):
    return [c for c in range(n_c) if (int(mask_row[c >> 5]) >> (c & 31)) & 1]


def _tiny_sparse(fp16=False, W=4, seed=None):
    wl = workloads.WORKLOADS["tiny"]
    P = wl.P
    ld = (P + 63) // 64 * 64
    if fp16:
        wl = workloads.custom(W, wl.numels, True, sigma=1e-2, scale_mode="layer")
    else:
        wl = workloads.custom(W, wl.numels, False, sigma=1e-2, scale_mode="layer")
    return wl, P, ld


@pytest.mark.parametrize("fp16", [False, True])
def test_sparse_step_independent_recomputation(fp16):
    """Every output of a sparse step recomputed with numpy from its definition:
    a = leaf + r, keys (binary64 sums of squares), selection (library sort),
    transmitted sum by the level-pairing tree, residual split."""
    wl, P, ld = _tiny_sparse(fp16, W=5)
    C = 64
    n_c = (P + C - 1) // C
    k = oracle.keep_count(n_c, 0.25)
    rng = np.random.default_rng(6)
    r = np.zeros((wl.W, ld), np.float32)
    r[:, :P] = rng.standard_normal((wl.W, P)).astype(np.float32) * np.float32(3e-3)
    w = workloads.weights(wl)
    v = np.zeros(P, np.float32)
    for step in (1, 2):
        b = workloads.grad_bucket(wl, step, ld)
        leaf = b.view(np.float16).astype(np.float32) if fp16 else b
        a = (leaf[:, :P] + r[:, :P]).astype(np.float32)
        r_in = r.copy()
        w0, v0 = w.copy(), v.copy()
        res = oracle.sparse_step(b, P, fp16, C, k, r, 0.01, 0.9, w, v)
        t = np.zeros_like(a)
        for wk in range(wl.W):
            keys_np = np.array([np.sum(a[wk, c * C:(c + 1) * C].astype(np.float64) ** 2) for c in range(n_c)])
            assert np.allclose(res.keys[wk], keys_np, rtol=1e-12, atol=0)
            assert res.margin[wk] > 1e-12
            sel = _lib_topk(keys_np, k)
            assert list(res.sel_idx[wk]) == sel
            assert _mask_to_chunks(res.sel_mask[wk], n_c) == sel
            on = np.zeros(P, bool)
            for c in sel:
                on[c * C:(c + 1) * C] = True
            t[wk, on] = a[wk, on]
            # residual split: r + t == a bitwise, disjoint supports
            assert np.all(r[wk, :P][on] == 0)
            assert np.array_equal(r[wk, :P][~on].view(np.uint32), a[wk, ~on].view(np.uint32))
            assert np.array_equal((r[wk, :P] + t[wk]).view(np.uint32), a[wk].view(np.uint32)) or \
                np.array_equal(r[wk, :P] + t[wk], a[wk])
        g = _level_pairing(t) * np.float32(1.0 / wl.W)
        assert np.array_equal(res.gbar, g)
        vn = np.float32(0.9) * v0 + np.float32(0.01) * g
        assert np.array_equal(v, vn) and np.array_equal(w, w0 - vn)
        assert np.all(r[:, P:] == r_in[:, P:])


@pytest.mark.parametrize("fp16", [False, True])
def test_keep_ratio_one_equals_dense(fp16):
    wl, P, ld = _tiny_sparse(fp16, W=4)
    b = workloads.grad_bucket(wl, 1, ld)
    r = np.zeros((wl.W, ld), np.float32)
    w1 = workloads.weights(wl)
    v1 = np.zeros(P, np.float32)
    w2, v2 = w1.copy(), v1.copy()
    n_c = (P + 63) // 64
    res = oracle.sparse_step(b, P, fp16, 64, oracle.keep_count(n_c, 1.0), r, 0.01, 0.9, w1, v1)
    g = oracle.dense_step(b, P, fp16, 0.01, 0.9, w2, v2)
    assert np.array_equal(w1, w2) and np.array_equal(v1, v2)
    assert np.array_equal(res.gbar, g)              # equal as numbers (+0 == -0)
    assert np.all(r == 0)


def test_keep_ratio_zero_sends_nothing_and_accumulates():
    wl, P, ld = _tiny_sparse(False, W=3)
    r = np.zeros((wl.W, ld), np.float32)
    run = np.zeros((wl.W, P), np.float32)
    w = workloads.weights(wl)
    v = np.full(P, 0.5, np.float32)
    for step in (1, 2, 3):
        b = workloads.grad_bucket(wl, step, ld)
        run = run + b[:, :P]
        w0, v0 = w.copy(), v.copy()
        res = oracle.sparse_step(b, P, False, 64, 0, r, 0.01, 0.9, w, v)
        assert np.all(res.gbar == 0) and np.all(res.sel_mask == 0)
        assert np.array_equal(r[:, :P], run)
        assert np.array_equal(v, np.float32(0.9) * v0) and np.array_equal(w, w0 - v)


def test_multi_step_checkpoint_resume_and_threads():
    wl, P, ld = _tiny_sparse(True, W=4)
    k = oracle.keep_count((P + 63) // 64, 0.1)
    seq = []
    for threads in (1, 5):
        r = np.zeros((wl.W, ld), np.float32)
        w = workloads.weights(wl)
        v = np.zeros(P, np.float32)
        for step in (1, 2):
            oracle.sparse_step(workloads.grad_bucket(wl, step, ld), P, True, 64, k, r, 0.01, 0.9, w, v,
                               threads=threads)
        ck = (r.copy(), w.copy(), v.copy())
        res = oracle.sparse_step(workloads.grad_bucket(wl, 3, ld), P, True, 64, k, r, 0.01, 0.9, w, v,
                                 threads=threads)
        r2, w2, v2 = ck
        res2 = oracle.sparse_step(workloads.grad_bucket(wl, 3, ld), P, True, 64, k, r2, 0.01, 0.9, w2, v2,
                                  threads=threads)
        assert np.array_equal(r, r2) and np.array_equal(w, w2) and np.array_equal(v, v2)
        assert np.array_equal(res.sel_idx, res2.sel_idx)
        seq.append((r, w, v))
    assert all(np.array_equal(x, y) for x, y in zip(seq[0], seq[1]))


def test_partial_last_chunk_and_chunks_cross_layers():
    """Chunks run over the fused vector, across layer boundaries; the last chunk
    is shorter.  Keys of the last chunk cover only the elements that exist."""
    W, P, C = 2, 1000, 96          # n_c = 11, last chunk has 40 elements
    rng = np.random.default_rng(8)
    b = np.zeros((W, 1024), np.float32)
    b[:, :P] = rng.standard_normal((W, P)).astype(np.float32)
    b[:, P:] = 100.0               # padding must never count
    r = np.zeros((W, 1024), np.float32)
    res = oracle.sparse_step(b, P, False, C, 3, r, 0.01, 0.9, None, None)
    last = np.sum(b[:, 960:P].astype(np.float64) ** 2, axis=1)
    assert np.allclose(res.keys[:, 10], last, rtol=1e-12)
    assert res.keys.shape == (W, 11)


# ----------------------------------------------------------------------------
# fusion (pack)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [np.float32, np.uint16])
def test_pack_is_concatenation(dt):
    rng = np.random.default_rng(9)
    numels = [432, 16, 4608, 32, 10, 7]
    W = 3
    layers = [[rng.integers(0, 60000, n).astype(dt) for n in numels] for _ in range(W)]
    ld = 5120
    out = oracle.pack(layers, ld)
    for w in range(W):
        cat = np.concatenate(layers[w])
        assert np.array_equal(out[w, :cat.size], cat)
        assert np.all(out[w, cat.size:] == 0)
