"""The pending forms of the deferred residual, as a bookkeeping rule, checked
on the CPU against the oracle.

The GPU kernels of the pending forms compute the residual recurrence of
coarse-grained sparse communication (GradientFlow, arXiv abstract: only the
important chunks are sent, the rest stay in the worker's residual) without
storing every value of it: a chunk sent at step t-1 stores nothing at step t,
and at depth 2 neither does a chunk sent at t-2 and not at t-1.  Whoever needs
such a value later recomputes it from the gradients still held, in the order
of the recurrence itself.  This test states that rule in numpy (binary32
arithmetic, round to nearest even) and runs it beside the oracle's plain
recurrence for several steps: every a the rule forms, the keys they give, and
the whole residual after a flush must equal the oracle's, bit for bit.  No
kernel runs here; the GPU tests check the kernels against the oracle."""
import numpy as np
import pytest

import oracle
import workloads

F0 = np.float32(0.0)


def widen(b, fp16):
    return b.view(np.float16).astype(np.float32) if fp16 else b.astype(np.float32)


def run_model(wl, depth, steps, hook=None, mutate=None):
    W, P, C = wl.W, wl.P, wl.chunk
    ld = (P + 63) // 64 * 64
    n_c = (P + C - 1) // C
    k = oracle.keep_count(n_c, wl.rho)
    w_ref, v_ref = workloads.weights(wl), np.zeros(P, np.float32)
    r_ref = np.zeros((W, ld), np.float32)
    R = np.zeros((W, P), np.float32)                  # what the rule stores
    G = {}                                            # widened gradients by step
    M = {s: np.zeros((W, n_c), bool) for s in (-2, -1, 0)}   # selections by step
    kinds_seen = set()

    def elems(m):
        return np.repeat(m, C, axis=1)[:, :P]

    for t in range(1, steps + 1):
        b = workloads.grad_bucket(wl, t, ld)
        if hook is not None:
            hook(b, t)
        res = oracle.sparse_step(b, P, wl.fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        G[t] = widen(b[:, :P], wl.fp16)
        g = G[t]
        A = elems(M[t - 1])                               # sent at t-1: residual +0
        B = elems(M[t - 2]) & ~A                          # pending one step
        Cc = elems(M[t - 3]) & ~elems(M[t - 2]) & ~A if depth == 2 else np.zeros_like(A)
        D = ~(A | B | Cc)
        a = np.empty_like(g)
        a[A] = g[A] + F0
        if B.any():
            # mutate == "B": the pending residual without its + 0 (a planted mistake)
            a[B] = g[B] + (G[t - 1][B] if mutate == "B" else G[t - 1][B] + F0)
        if Cc.any():
            a[Cc] = g[Cc] + (G[t - 1][Cc] + (G[t - 2][Cc] + F0))
        a[D] = g[D] + R[D]
        kinds_seen.update(nm for nm, m in (("A", A), ("B", B), ("C", Cc)) if m.any())
        # keys from the rule's a: the oracle's within its binary64 reduction order
        key = np.zeros((W, n_c))
        for c in range(n_c):
            seg = a[:, c * C:min((c + 1) * C, P)].astype(np.float64)
            key[:, c] = (seg * seg).sum(axis=1)
        np.testing.assert_allclose(key, res.keys, rtol=1e-12, atol=0)
        ch = np.arange(n_c)
        M[t] = ((res.sel_mask[:, ch >> 5] >> (ch & 31)) & 1).astype(bool)
        sent = elems(M[t])
        # what the norm pass stores: everything but A, and at depth 2 but B
        store = ~A & ~(B if depth == 2 else np.zeros_like(B))
        R[store] = a[store]
        # the flush: the values still held as gradients, then the sent chunks read as zero
        L = R.copy()
        fl = A & ~sent
        L[fl] = g[fl] + F0
        fl2 = B & ~sent
        if depth == 2 and fl2.any():
            L[fl2] = g[fl2] + (G[t - 1][fl2] + F0)
        L[sent] = 0.0
        assert np.array_equal(L.view(np.uint32), r_ref[:, :P].view(np.uint32)), "residual after step %d" % t
        # the unsent values the rule formed are the oracle's residual itself
        assert np.array_equal(a[~sent].view(np.uint32), r_ref[:, :P][~sent].view(np.uint32))
        G.pop(t - 2, None)
    return kinds_seen


@pytest.mark.parametrize("depth", [1, 2])
@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", [(3, [3000, 7, 2000], 256), (16, [8, 1, 5000, 7, 4096, 333, 64], 256),
                                        (40, [20000, 37, 4003], 512)])
def test_pending_rule_matches_oracle(depth, fp16, W, numels, C):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    kinds = run_model(wl, depth, steps=7)
    # the rule's special cases all occurred
    assert kinds >= ({"A", "B", "C"} if depth == 2 else {"A", "B"}), kinds


@pytest.mark.parametrize("depth", [1, 2])
def test_pending_rule_negative_zero(depth):
    """-0 gradients: every recomputed residual is formed with + 0 first, as the
    stored one was, so the bits agree."""
    def hook(b, t):
        b[:, 100:300] = 0x8000
        b[1:, 600:900] = 0x8000
    wl = workloads.custom(4, [3000], True, sigma=1e-2, chunk=256, rho=0.5)
    run_model(wl, depth, steps=6, hook=hook)


@pytest.mark.parametrize("depth", [1, 2])
def test_pending_rule_catches_a_dropped_zero(depth):
    """The check is sharp: the same rule with the pending residual formed as
    g1 instead of g1 + 0 disagrees with the oracle once -0 gradients meet it."""
    def hook(b, t):
        b[:, :] = np.where(np.arange(b.shape[1]) % 3 == 0, np.uint16(0x8000), b)
    wl = workloads.custom(8, [8192], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=256,
                          rho=0.2)
    run_model(wl, depth, steps=7, hook=hook)
    with pytest.raises(AssertionError):
        run_model(wl, depth, steps=7, hook=hook, mutate="B")
