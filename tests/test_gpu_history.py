"""GPU parity of the deferred-residual sparse step (the residual buffer written
only on storing steps and re-formed from the held gradients and masks in
between) against the oracle's plain recurrence, step by step: keys, selected
chunks, mean gradient, w and v every step, and the residual through a flush
(into a copy, so the steps themselves never see it, and in place in a
separate run).  Store schedules of period 1 (the lazy-zero form), 2 and 3 and
random ones; binary16 and binary32 gradients; layer tensors whose alignment
changes from step to step."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, assert_close, assert_same_bits, device_layers, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# misalignment of worker w's layer l at step t, in elements past a 16-byte boundary
MIS = {"aligned": lambda w, l, t: 0, "mixed": lambda w, l, t: (3 * w + l + t) % 4}


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def every(period):
    return lambda t, age: age == period - 1


def random_schedule(seed):
    rng = np.random.default_rng(seed)
    return lambda t, age: age == 2 or rng.random() < 0.4


def strict_same(got, ref, name):
    assert np.array_equal(np.asarray(got).view(np.uint32), np.asarray(ref).view(np.uint32)), name


def run_history(ga, wl, schedule, mis="aligned", steps=6, hook=None, strict=False, flush_every=False,
                start="ones"):
    """Drive the three deferred entry points directly for `steps` steps and
    compare every output with the oracle.  start: "ones" describes the zero
    residual by an all-ones mask (the buffer is not read), "zero" reads the
    zero-filled buffer at age 0."""
    C, P, W = wl.chunk, wl.P, wl.W
    plan = ga.Plan(W, wl.numels, wl.fp16, chunk=C, keep_ratio=wl.rho)
    ld, k, n_c, mw = plan.ld, plan.k, plan.n_chunks, plan.mask_words
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd, keys = plan.empty_residual(), plan.empty_keys()
    if start == "ones":
        rd.fill_(float("nan"))          # never read before it is written
        ones = np.zeros((W, mw), np.uint32)
        for c in range(n_c):
            ones[:, c >> 5] |= np.uint32(1 << (c & 31))
        masks = [to_dev(ones.view(np.int32))]
    else:
        masks = [None]
    tables, kept = [], []
    idx = torch.full((W, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    print("[history] W=%d P=%d fp16=%s C=%d rho=%g %s start=%s" % (W, P, wl.fp16, C, wl.rho, mis, start),
          flush=True)
    stores = []
    same = strict_same if strict else assert_same_bits
    for t in range(1, steps + 1):
        b = workloads.grad_bucket(wl, t, ld)
        if hook is not None:
            hook(b, t)
        res = oracle.sparse_step(b, P, wl.fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        buf, ptrs = device_layers(b[:, :P], wl.numels, lambda w, l: MIS[mis](w, l, t))
        age = len(masks) - 1
        store = bool(schedule(t, age))
        hist = plan.history(masks, tables)
        sel = torch.zeros((W, mw), dtype=torch.int32, device="cuda")
        plan.chunk_norm_deferred(ptrs, hist, store, rd, keys)
        plan.chunk_topk(keys, idx, sel)
        plan.sparse_gather_reduce_deferred(ptrs, hist, store, rd, sel, gd, wd, vd, wl.lr, wl.mu)
        if flush_every:
            plan.residual_flush(ptrs, hist, store, rd, sel)
            r_view = rd
        else:
            r_view = rd.clone()
            plan.residual_flush(ptrs, hist, store, r_view, sel)
        torch.cuda.synchronize()
        stores.append(store)
        if wl.rho not in (0.0, 1.0):
            assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        assert_close(host(keys), res.keys, KEY_RTOL, "keys step %d" % t)
        if k > 0:
            assert np.array_equal(host(idx)[:, :k], res.sel_idx), "selected chunk indices differ step %d" % t
        assert np.array_equal(host(sel).view(np.uint32), res.sel_mask), "mask step %d" % t
        same(host(r_view)[:, :P], r_ref[:, :P], "residual step %d" % t)
        same(host(gd), res.gbar, "gbar step %d" % t)
        same(host(wd), w_ref, "w step %d" % t)
        same(host(vd), v_ref, "v step %d" % t)
        if flush_every:
            masks, tables, kept = [None], [], []
        elif store:
            masks, tables, kept = [sel], [], []
        else:
            masks, tables, kept = [sel] + masks, [ptrs] + tables, [buf] + kept
    plan.close()
    return stores


CONFIGS = [(1, [3000, 7, 2000], 256), (3, workloads.WORKLOADS["tiny"].numels, 512),
           (16, [8, 1, 5000, 7, 4096, 333, 64], 256), (33, [20000, 37, 4003], 1024),
           (128, [2048, 16, 4099, 520], 256), (300, [3000, 17, 1000], 512),
           # chunks longer than one 2048-element norm part: three parts (the
           # last of 256), the last chunk 1197 long (two parts empty); four
           (7, [5000, 3, 9000, 250], 4352), (40, [20000, 37, 4003], 8192)]


@pytest.mark.parametrize("period", [1, 2, 3])
@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", CONFIGS)
@pytest.mark.parametrize("mis", list(MIS))
def test_history_matches_oracle(ga, period, fp16, W, numels, C, mis):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    stores = run_history(ga, wl, every(period), mis, steps=6)
    assert stores == [(t % period) == 0 for t in range(1, 7)]


@pytest.mark.parametrize("fp16,mis", [(True, "mixed"), (False, "aligned")])
def test_history_maximum_worker_count(ga, fp16, mis):
    """W at the library's limit (1024 workers: eleven tree levels, and the
    groups' bitmaps reloaded per group rather than kept), stored every third
    step so that every age (0, 1, 2) runs."""
    wl = workloads.custom(ga.MAX_WORKERS, [3000, 77, 1100], fp16, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.25)
    stores = run_history(ga, wl, every(3), mis, steps=5)
    assert stores == [False, False, True, False, False]


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
@pytest.mark.parametrize("fp16", [False, True])
def test_history_random_schedule(ga, seed, fp16):
    wl = workloads.custom(40, [5000, 3, 9000, 250, 1024], fp16, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.15)
    run_history(ga, wl, random_schedule(seed), "mixed", steps=9)


@pytest.mark.parametrize("period", [1, 2, 3])
def test_history_zero_buffer_start(ga, period):
    """The other description of the zero start: age 0, no mask, the buffer read."""
    wl = workloads.custom(16, [8, 1, 5000, 7, 4096, 333, 64], True, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.2)
    run_history(ga, wl, every(period), "mixed", steps=5, start="zero")


@pytest.mark.parametrize("period", [2, 3])
@pytest.mark.parametrize("fp16", [False, True])
def test_history_flushed_every_step(ga, period, fp16):
    """A flush in place leaves the residual itself; the next step resumes at
    age 0 with no mask and no earlier tensor."""
    wl = workloads.custom(16, [8, 1, 5000, 7, 4096, 333, 64], fp16, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.2)
    run_history(ga, wl, every(period), "mixed", steps=6, flush_every=True)


@pytest.mark.parametrize("period", [1, 2, 3])
@pytest.mark.parametrize("rho", [0.0, 1.0])
def test_history_keep_ratio_extremes(ga, rho, period):
    wl = workloads.custom(6, [9000, 11, 300], True, sigma=1e-2, chunk=256, rho=rho)
    run_history(ga, wl, every(period), "mixed", steps=4)


@pytest.mark.parametrize("period", [1, 2, 3])
def test_history_negative_zero_leaves(ga, period):
    """-0 gradients: a residual re-formed onto +0 adds the +0 as the recurrence
    does, so the residual, sums and state match bit for bit (strictly)."""
    def hook(b, t):
        b[:, 100:300] = 0x8000          # binary16 -0 in every worker
        b[1:, 600:700] = 0x8000
    for rho, steps in ((1.0, 3), (0.5, 6)):
        wl = workloads.custom(4, [3000], True, sigma=1e-2, chunk=256, rho=rho)
        run_history(ga, wl, every(period), "aligned", steps=steps, hook=hook, strict=True)


@pytest.mark.parametrize("depth", [0, 1, 2])
def test_deferred_residual_helper(ga, depth):
    """The binding's buffer rotation gives the same results as the oracle, and
    its flush the oracle's residual."""
    wl = workloads.custom(24, [4096, 5, 3000], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=512, rho=0.2)
    P, W = wl.P, wl.W
    plan = ga.Plan(W, wl.numels, True, chunk=wl.chunk, keep_ratio=wl.rho)
    dr = ga.DeferredResidual(plan, depth)
    w_ref, v_ref = workloads.weights(wl), np.zeros(P, np.float32)
    r_ref = np.zeros((W, plan.ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    kept = []
    for t in range(1, 8):
        b = workloads.grad_bucket(wl, t, plan.ld)
        res = oracle.sparse_step(b, P, True, wl.chunk, plan.k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        buf, ptrs = device_layers(b[:, :P], wl.numels, lambda w, l: (w + l + t) % 4)
        kept = (kept + [buf])[-(depth + 1):]
        stored = dr.step(ptrs, gd, wd, vd, wl.lr, wl.mu)
        assert stored == (t % (depth + 1) == 0)
        r = dr.flush(torch.empty_like(dr.resid))
        torch.cuda.synchronize()
        assert_same_bits(host(r)[:, :P], r_ref[:, :P], "residual step %d" % t)
        assert_same_bits(host(gd), res.gbar, "gbar step %d" % t)
        assert_same_bits(host(wd), w_ref, "w step %d" % t)
        assert_same_bits(host(vd), v_ref, "v step %d" % t)
    plan.close()


@pytest.mark.parametrize("depth", [1, 2])
def test_deferred_residual_helper_resume_and_flush(ga, depth):
    """The helper's checkpoint path: a flush before any step is the starting
    residual (zero, or the one given); a second flush in place changes
    nothing; a helper built on a flushed residual (resid=) continues exactly
    as the oracle does, with no earlier gradient tensor."""
    wl = workloads.custom(20, [4096, 5, 3000], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=256, rho=0.25)
    P, W = wl.P, wl.W
    plan = ga.Plan(W, wl.numels, True, chunk=wl.chunk, keep_ratio=wl.rho)
    dr = ga.DeferredResidual(plan, depth)
    dr.resid.fill_(float("nan"))
    assert torch.count_nonzero(dr.flush(torch.empty_like(dr.resid))).item() == 0
    w_ref, v_ref = workloads.weights(wl), np.zeros(P, np.float32)
    r_ref = np.zeros((W, plan.ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    kept = []
    for t in range(1, 7):
        b = workloads.grad_bucket(wl, t, plan.ld)
        res = oracle.sparse_step(b, P, True, wl.chunk, plan.k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        buf, ptrs = device_layers(b[:, :P], wl.numels, lambda w, l: (w + 2 * l + t) % 4)
        kept = (kept + [buf])[-(depth + 1):]
        dr.step(ptrs, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        assert_same_bits(host(gd), res.gbar, "gbar step %d" % t)
        assert_same_bits(host(wd), w_ref, "w step %d" % t)
        if t == depth:                               # a step that did not store
            assert dr.age > 0
            saved = dr.flush().clone()
            again = dr.flush().clone()               # nothing left to add
            torch.cuda.synchronize()
            assert_same_bits(host(saved)[:, :P], r_ref[:, :P], "flushed residual")
            assert torch.equal(saved.view(torch.int32), again.view(torch.int32))
            # resume: a new helper on the saved residual alone
            dr = ga.DeferredResidual(plan, depth, resid=saved)
            assert torch.equal(dr.flush(torch.empty_like(saved)).view(torch.int32), saved.view(torch.int32))
            kept = []
    torch.cuda.synchronize()
    assert_same_bits(host(dr.flush(torch.empty_like(dr.resid)))[:, :P], r_ref[:, :P], "residual at the end")
    plan.close()


def test_history_errors(ga):
    plan = ga.Plan(4, [1000], True, chunk=256, keep_ratio=0.5)
    W, mw = 4, plan.mask_words
    p0 = torch.zeros(4, dtype=torch.int64, device="cuda")
    p1 = torch.zeros(4, dtype=torch.int64, device="cuda")
    rd, keys = plan.empty_residual(), plan.empty_keys()
    m0 = torch.zeros((W, mw), dtype=torch.int32, device="cuda")
    m1 = torch.zeros((W, mw), dtype=torch.int32, device="cuda")
    g = torch.zeros(plan.P, device="cuda")

    def status(fn, *a):
        with pytest.raises(ga.GAError) as e:
            fn(*a)
        return e.value.status

    h = plan.history([m0, m1], [p1])
    h.age = 3                                       # beyond the largest age
    assert status(plan.chunk_norm_deferred, p0, h, False, rd, keys) == ga.GA_ERR_INVALID
    h = plan.history([m0, m1], [p1])
    h.d_layer_ptrs[0] = None                        # a missing earlier table
    assert status(plan.chunk_norm_deferred, p0, h, False, rd, keys) == ga.GA_ERR_INVALID
    h = plan.history([m0, m1], [p0])                # an earlier table that is this step's
    assert status(plan.chunk_norm_deferred, p0, h, False, rd, keys) == ga.GA_ERR_INVALID
    assert status(plan.sparse_gather_reduce_deferred, p0, h, False, rd, m1, g) == ga.GA_ERR_INVALID
    assert status(plan.residual_flush, p0, h, False, rd, m1) == ga.GA_ERR_INVALID
    h = plan.history([m0, m1, m0], [p1, p1])        # two steps sharing a table
    assert status(plan.chunk_norm_deferred, p0, h, False, rd, keys) == ga.GA_ERR_INVALID
    h = plan.history([m0, m1], [p1])                # the selection written over a history mask
    assert status(plan.sparse_gather_reduce_deferred, p0, h, False, rd, m1, g) == ga.GA_ERR_INVALID
    assert status(plan.residual_flush, p0, h, False, rd, m0) == ga.GA_ERR_INVALID
    plan64 = ga.Plan(4, [1000], True, chunk=64, keep_ratio=0.5)
    rd64 = plan64.empty_residual()
    m64 = torch.zeros((W, plan64.mask_words), dtype=torch.int32, device="cuda")
    s64 = torch.zeros((W, plan64.mask_words), dtype=torch.int32, device="cuda")
    h = plan64.history([m64])
    assert status(plan64.sparse_gather_reduce_deferred, p0, h, True, rd64, s64, g) == ga.GA_ERR_UNSUPPORTED
    dense = ga.Plan(4, [1000], True)
    assert status(dense.chunk_norm_deferred, p0, dense.history([None]), True, rd, keys) == ga.GA_ERR_INVALID
    torch.cuda.synchronize()
