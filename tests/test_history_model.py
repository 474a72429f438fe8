"""The deferred residual as a bookkeeping rule, checked on the CPU against the
oracle.

Coarse-grained sparse communication (GradientFlow, arXiv abstract: only the
important gradient chunks are sent) carries every unsent chunk in a per-worker
residual: a_t = g_t + r_{t-1}, and r_t = 0 on the chunks sent at t, a_t
elsewhere.  The GPU kernels of the deferred form do not store a_t at every
step.  The buffer is written only on the steps the caller marks as storing
(and by a flush); between two such writes the residual is re-formed from what
the caller still holds: the buffer (the value of the step it was written at,
its "age"), the selection masks of the steps since then and their gradient
tensors.  For each (worker, chunk), if the chunk was sent j steps back (the
most recent such step, j <= age), r_{t-1} is the last j gradients added onto
+0; otherwise it is the last `age` gradients added onto the buffer, always
newest outermost: g_{t-1} + (g_{t-2} + (... + base)).

This test states that rule in numpy (binary32, round to nearest even) and runs
it beside the oracle's plain recurrence for several steps, over store
schedules of period 1 (store every step: the lazy-zero form), 2 and 3 and
random ones: every a the rule forms must give the oracle's keys, its sent
values the oracle's mean gradient and its unsent values the oracle's residual,
bit for bit, and the flush (buffer or re-formed a, zero on the sent chunks)
must reproduce the oracle's residual exactly.  Planted mistakes in the rule
must fail.  No kernel runs here; the GPU tests check the kernels against the
oracle."""
import numpy as np
import pytest

import oracle
import workloads

F0 = np.float32(0.0)
MAX_AGE = 2


def widen(b, fp16):
    return b.view(np.float16).astype(np.float32) if fp16 else b.astype(np.float32)


def reform(g, R, masks, grads, age, elems, mutate=None):
    """a = g + r_{t-1} under the rule, and the (n, zero-base) case of each element."""
    W, P = g.shape
    n = np.full((W, P), age, np.int64)
    zero = np.zeros((W, P), bool)
    found = np.zeros((W, P), bool)
    for j in range(age + 1):
        m = masks[j]
        if m is None:
            continue
        hit = elems(m) & ~found
        if mutate == "last_mask" and j == age:
            hit[:] = False                   # planted: the oldest mask ignored
        n[hit] = j
        zero[hit] = True
        found |= hit
    acc = np.where(zero, F0, R)
    if mutate == "zero_as_buffer":
        acc = R.copy()                       # planted: a sent chunk's residual read from the buffer
    for j in reversed(range(age)):
        add = n > j
        if mutate == "drop_plus_zero":
            # planted: a residual of one gradient onto +0 taken as that gradient
            first = add & zero & (n == j + 1)
            acc = np.where(first, grads[j], np.where(add, grads[j] + acc, acc))
        else:
            acc = np.where(add, grads[j] + acc, acc)
    if mutate == "order" and age >= 1:
        # planted: the newest gradients added first, (g_t + g_{t-1}) + (g_{t-2} + ... + base)
        rest = np.where(zero, F0, R)
        for j in reversed(range(1, age)):
            rest = np.where(n > j, grads[j] + rest, rest)
        return np.where(n >= 1, (g + grads[0]) + rest, g + acc), n, zero
    return g + acc, n, zero


def run_model(wl, schedule, steps, hook=None, mutate=None, flush_every=False, check_flush=True):
    """schedule(t, age) -> store this step?  Returns the set of (n, zero) cases seen."""
    W, P, C = wl.W, wl.P, wl.chunk
    ld = (P + 63) // 64 * 64
    n_c = (P + C - 1) // C
    k = oracle.keep_count(n_c, wl.rho)
    w_ref, v_ref = workloads.weights(wl), np.zeros(P, np.float32)
    r_ref = np.zeros((W, ld), np.float32)
    R = np.zeros((W, P), np.float32)           # the buffer: zero = r_0
    age = 0
    masks = [None]                             # masks[j]: selection of step t-1-j (None: nothing sent)
    grads = []                                 # grads[j]: widened gradient of step t-1-j
    cases = set()

    def elems(m):
        return np.repeat(m, C, axis=1)[:, :P]

    for t in range(1, steps + 1):
        b = workloads.grad_bucket(wl, t, ld)
        if hook is not None:
            hook(b, t)
        res = oracle.sparse_step(b, P, wl.fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        g = widen(b[:, :P], wl.fp16)
        a, n, zero = reform(g, R, masks, grads, age, elems, mutate)
        cases.update(zip(n.ravel().tolist()[::97], zero.ravel().tolist()[::97]))
        key = np.zeros((W, n_c))
        for c in range(n_c):
            seg = a[:, c * C:min((c + 1) * C, P)].astype(np.float64)
            key[:, c] = (seg * seg).sum(axis=1)
        np.testing.assert_allclose(key, res.keys, rtol=1e-12, atol=0)
        ch = np.arange(n_c)
        sel = ((res.sel_mask[:, ch >> 5] >> (ch & 31)) & 1).astype(bool)
        sent = elems(sel)
        # the sent values are the oracle's transmitted leaves: their tree is its mean gradient
        t_leaves = np.where(sent, a, F0)
        gbar = oracle.tree_sum(t_leaves) * np.float32(1.0 / W)
        assert np.array_equal(gbar.view(np.uint32), res.gbar.view(np.uint32)), "mean gradient step %d" % t
        # the unsent values are the oracle's residual
        assert np.array_equal(a[~sent].view(np.uint32), r_ref[:, :P][~sent].view(np.uint32)), "a step %d" % t
        store = bool(schedule(t, age))
        assert store or age < MAX_AGE, "schedule exceeds the largest age"
        if store:
            R = a.copy()
        if check_flush:
            flushed = (R if store else a).copy()
            flushed[sent] = 0.0
            assert np.array_equal(flushed.view(np.uint32), r_ref[:, :P].view(np.uint32)), "flush step %d" % t
        if flush_every:
            R = (R if store else a).copy()
            R[sent] = 0.0
            age, masks, grads = 0, [None], []
        elif store:
            age, masks, grads = 0, [sel], []
        else:
            age, masks, grads = age + 1, [sel] + masks, [g] + grads
    return cases


def every(period):
    return lambda t, age: age == period - 1


def random_schedule(seed):
    rng = np.random.default_rng(seed)
    return lambda t, age: age == MAX_AGE or rng.random() < 0.4


@pytest.mark.parametrize("period", [1, 2, 3])
@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", [(3, [3000, 7, 2000], 256), (16, [8, 1, 5000, 7, 4096, 333, 64], 256),
                                        (40, [20000, 37, 4003], 512)])
def test_history_rule_matches_oracle(period, fp16, W, numels, C):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    cases = run_model(wl, every(period), steps=7)
    want = {(j, True) for j in range(period)} | {(period - 1, False)}
    assert cases >= want, cases


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_history_rule_random_schedule(seed):
    wl = workloads.custom(24, [5000, 3, 9000, 250], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=256, rho=0.15)
    cases = run_model(wl, random_schedule(seed), steps=9)
    assert cases >= {(0, True), (1, True), (0, False), (1, False)}, cases


@pytest.mark.parametrize("period", [2, 3])
def test_history_rule_flushed_every_step(period):
    """A flush leaves the oracle's residual in the buffer; the next step then
    starts at age 0 with no mask and no earlier gradient."""
    wl = workloads.custom(8, [6000, 5, 3000], False, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=256, rho=0.2)
    run_model(wl, every(period), steps=6, flush_every=True)


def test_history_rule_all_sent_start():
    """A zero residual can be described without reading the buffer: every chunk
    sent one step before the first (a mask of all ones)."""
    wl = workloads.custom(6, [4000, 300], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=256, rho=0.25)
    W, P, C = wl.W, wl.P, wl.chunk
    n_c = (P + C - 1) // C
    ld = (P + 63) // 64 * 64
    b = workloads.grad_bucket(wl, 1, ld)
    g = widen(b[:, :P], True)
    garbage = np.full((W, P), 7.0, np.float32)
    a, n, zero = reform(g, garbage, [np.ones((W, n_c), bool)], [], 0,
                        lambda m: np.repeat(m, C, axis=1)[:, :P])
    assert zero.all() and (n == 0).all()
    assert np.array_equal(a.view(np.uint32), (g + F0).view(np.uint32))


@pytest.mark.parametrize("period", [2, 3])
def test_history_rule_negative_zero(period):
    """-0 gradients: a residual re-formed onto +0 adds +0 first, as the stored
    one was formed, so the bits agree."""
    def hook(b, t):
        b[:, 100:300] = 0x8000
        b[1:, 600:900] = 0x8000
    wl = workloads.custom(4, [3000], True, sigma=1e-2, chunk=256, rho=0.5)
    run_model(wl, every(period), steps=6, hook=hook)


@pytest.mark.parametrize("mutate,period,fp16", [("drop_plus_zero", 2, True), ("drop_plus_zero", 3, True),
                                                ("last_mask", 2, True), ("last_mask", 3, True),
                                                ("zero_as_buffer", 2, True), ("order", 2, False),
                                                ("order", 3, False)])
def test_history_rule_catches_planted_mistakes(mutate, period, fp16):
    """The checks are sharp: each planted mistake in the rule disagrees with the
    oracle (a dropped + 0 once -0 gradients meet it; the order of the adds once
    binary32 gradients make the rounding visible)."""
    def hook(b, t):
        if fp16:
            b[:, :] = np.where(np.arange(b.shape[1]) % 3 == 0, np.uint16(0x8000), b)
    wl = workloads.custom(8, [8192], fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=256,
                          rho=0.2)
    run_model(wl, every(period), steps=7, hook=hook)
    with pytest.raises(AssertionError):
        run_model(wl, every(period), steps=7, hook=hook, mutate=mutate)
