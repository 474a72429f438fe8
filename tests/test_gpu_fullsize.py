"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, against the oracle run on the host cores.

NiN-, GoogLeNet- and AlexNet-shaped dense aggregation are compared on every
element, from a packed bucket and from the per-layer tensors.  The
AlexNet-shaped W=128 sparse workload (2048 per-layer tensors read with zero
copy) is run in the lazy-zero sequence of the boundary's calls and in the
benchmarked deferred form, over consecutive steps, and compared on every
selected index, every key and every element of the mean gradient, the
weights, the velocity and the residual of all 128 workers.  The deferred form
is also checkpointed (flushed, saved to the host) and resumed from the saved
state alone, and one of its steps is repeated from the same state to show it
bitwise deterministic."""
import os
import time

import numpy as np
import pytest

import oracle
import workloads
from helpers import (KEY_RTOL, TOL_FP16_PATH, TOL_FP32, assert_close, assert_same_bits, device_layers, host,
                     to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


_capman = None


@pytest.fixture(autouse=True)
def _progress(request):
    """Progress lines of these minutes-long tests go to the terminal even while
    pytest captures output, so that a long test is seen to be running."""
    global _capman
    _capman = request.config.pluginmanager.getplugin("capturemanager")
    yield
    _capman = None


def log(msg):
    line = "[fullsize] %s" % msg
    if _capman is not None:
        with _capman.global_and_fixture_disabled():
            print(line, flush=True)
    else:
        print(line, flush=True)


@pytest.mark.parametrize("source", ["bucket", "layers"])
@pytest.mark.parametrize("name", ["nin", "googlenet", "alexnet16"])
def test_dense_full_size(ga, name, source):
    wl = workloads.WORKLOADS[name]
    plan = ga.Plan(wl.W, wl.numels, wl.fp16)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    for step in (1, 2):
        t0 = time.time()
        b = workloads.grad_bucket(wl, step, plan.ld)
        if source == "layers":
            src, ptrs = device_layers(b[:, :wl.P], wl.numels)
        else:
            src = to_dev(b, wl.fp16)
        g_ref = oracle.dense_step(b, wl.P, wl.fp16, wl.lr, wl.mu, w_ref, v_ref)
        del b
        if source == "layers":
            plan.tree_reduce_layers(ptrs, gd, wd, vd, wl.lr, wl.mu)
        else:
            plan.tree_reduce(src, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        del src
        assert_close(host(gd), g_ref, TOL_FP16_PATH if wl.fp16 else TOL_FP32, "gbar")
        assert_same_bits(host(gd), g_ref, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
        log("%s (%s) step %d ok in %.1fs" % (name, source, step, time.time() - t0))


def sent_elements(mask, C, P):
    """[W][P] bool: the elements of the chunks set in a [W][mw] mask."""
    m = np.asarray(mask).view(np.uint32).astype(np.int64)
    n_c = (P + C - 1) // C
    ch = np.arange(n_c)
    return np.repeat(((m[:, ch >> 5] >> (ch & 31)) & 1).astype(bool), C, axis=1)[:, :P]


def sent_elements_dev(mask, C, P):
    """[W][P] bool on the device: the elements of the chunks set in a [W][mw]
    int32 mask."""
    n_c = (P + C - 1) // C
    ch = torch.arange(n_c, device=mask.device)
    bits = ((mask[:, ch >> 5] >> (ch & 31)) & 1).bool()
    return bits.repeat_interleave(C, dim=1)[:, :P]


def assert_residual(got, ref_dev, P, name, lazy_mask=None, C=0):
    """Every element of every worker's residual against the oracle's (already
    on the device), compared on the device 16 workers at a time: bitwise, +0
    and -0 taken as equal, NaN by position; with lazy_mask, the chunks it sets
    are read as zero (the lazy-zero buffer)."""
    W = got.shape[0]
    for w0 in range(0, W, 16):
        a = got[w0:w0 + 16, :P]
        b = ref_dev[w0:w0 + 16, :P]
        if lazy_mask is not None:
            a = torch.where(sent_elements_dev(lazy_mask[w0:w0 + 16], C, P), torch.zeros_like(a), a)
        same = (a.view(torch.int32) == b.view(torch.int32)) | (a == b) | (torch.isnan(a) & torch.isnan(b))
        if not bool(same.all()):
            bad = (~same).nonzero()[0].tolist()
            raise AssertionError("%s: %d mismatches, first at worker %d element %d: %r vs %r" % (
                name, int((~same).sum()), w0 + bad[0], bad[1], float(a[bad[0], bad[1]]), float(b[bad[0], bad[1]])))


def test_sparse_alexnet128_full_size(ga):
    """The lazy-zero sequence of the boundary's calls: chunk_norm_layers ->
    chunk_topk -> sparse_gather_reduce without zeroing, one mask buffer."""
    wl = workloads.WORKLOADS["alexnet128_sparse"]
    C = wl.chunk
    plan = ga.Plan(wl.W, wl.numels, True, chunk=C, keep_ratio=wl.rho)
    P, ld, k, n_c = wl.P, plan.ld, plan.k, plan.n_chunks
    assert (n_c, k) == (1861, 187)
    seg = workloads.segments(wl)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((wl.W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd = plan.empty_residual()
    keys = plan.empty_keys()
    idx = torch.empty((wl.W, k), dtype=torch.int32, device="cuda")
    mask = torch.zeros((wl.W, plan.mask_words), dtype=torch.int32, device="cuda")
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    for step in (1, 2, 3):
        t0 = time.time()
        b = workloads.grad_bucket(wl, step, ld, seg=seg)
        buf, ptrs = device_layers(b[:, :P], wl.numels)
        log("step %d generated+uploaded as %d layer tensors in %.1fs" % (step, wl.W * len(wl.numels),
                                                                       time.time() - t0))
        t1 = time.time()
        res = oracle.sparse_step(b, P, True, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        del b
        log("step %d oracle in %.1fs" % (step, time.time() - t1))
        plan.chunk_norm_layers(ptrs, rd, keys, mask if step > 1 else None)
        plan.chunk_topk(keys, idx, mask)
        plan.sparse_gather_reduce(rd, mask, False, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        del buf
        assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        assert np.array_equal(host(idx), res.sel_idx), "selected chunk indices differ"
        assert np.array_equal(host(mask).view(np.uint32), res.sel_mask)
        assert_close(host(keys), res.keys, KEY_RTOL, "keys")
        assert_same_bits(host(gd), res.gbar, "gbar")
        assert_close(host(gd), res.gbar, TOL_FP32, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
        ref_dev = torch.from_numpy(r_ref).cuda()
        assert_residual(rd, ref_dev, P, "lazy residual step %d" % step, lazy_mask=mask, C=C)
        del ref_dev
        log("step %d compared in %.1fs (total %.1fs)" % (step, time.time() - t1, time.time() - t0))


@pytest.mark.parametrize("cap", [0, 512])
def test_buckets_alexnet16_full_size(ga, cap):
    """Multi-bucket lazy allreduce at full size, as `bench.py --overlap` runs it
    (4 MiB buckets, layers last-first, each bucket after its event)."""
    wl = workloads.WORKLOADS["alexnet16"]
    plan = ga.Plan(wl.W, wl.numels, wl.fp16)
    bk = ga.Buckets(plan, 4 << 20)
    assert bk.count == 5
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    side = torch.cuda.Stream()
    for step in (1, 2):
        t0 = time.time()
        b = workloads.grad_bucket(wl, step, plan.ld)
        src, ptrs = device_layers(b[:, :wl.P], wl.numels)
        g_ref = oracle.dense_step(b, wl.P, wl.fp16, wl.lr, wl.mu, w_ref, v_ref)
        del b
        ready = torch.cuda.Event()
        ready.record()
        with torch.cuda.stream(side):
            for i in range(bk.count):
                bk.reduce_layers(i, ptrs, ready, None, wd, vd, wl.lr, wl.mu, max_workgroups=cap)
        torch.cuda.synchronize()
        del src
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
        log("alexnet16 buckets (cap %d) step %d ok in %.1fs" % (cap, step, time.time() - t0))


class DeviceRun:
    """One GPU instance of the deferred step: its residual, state and history."""

    def __init__(self, plan, w_init, v_init=None):
        self.plan = plan
        self.rd = plan.empty_residual()
        self.keys = plan.empty_keys()
        self.idx = torch.empty((plan.W, plan.k), dtype=torch.int32, device="cuda")
        self.wd = to_dev(w_init.copy())
        self.vd = torch.zeros(plan.P, dtype=torch.float32, device="cuda") if v_init is None else to_dev(v_init)
        self.gd = torch.empty(plan.P, dtype=torch.float32, device="cuda")
        self.masks, self.tables = [None], []
        self.last = None

    def step(self, ptrs, depth, lr, mu):
        p = self.plan
        store = len(self.masks) - 1 >= depth
        hist = p.history(self.masks, self.tables)
        sel = torch.zeros((p.W, p.mask_words), dtype=torch.int32, device="cuda")
        p.chunk_norm_deferred(ptrs, hist, store, self.rd, self.keys)
        p.chunk_topk(self.keys, self.idx, sel)
        p.sparse_gather_reduce_deferred(ptrs, hist, store, self.rd, sel, self.gd, self.wd, self.vd, lr, mu)
        self.last = (ptrs, hist, store, sel)
        if store:
            self.masks, self.tables = [sel], []
        else:
            self.masks, self.tables = [sel] + self.masks, [ptrs] + self.tables

    def flush(self, out):
        ptrs, hist, store, sel = self.last
        if out.data_ptr() != self.rd.data_ptr():
            out.copy_(self.rd)
        self.plan.residual_flush(ptrs, hist, store, out, sel)
        return out

    def check(self, res, w_ref, v_ref, ref_dev, scratch, name):
        assert np.array_equal(host(self.idx), res.sel_idx), name + ": selected chunk indices differ"
        assert np.array_equal(host(self.masks[0]).view(np.uint32), res.sel_mask), name + ": mask"
        assert_close(host(self.keys), res.keys, KEY_RTOL, name + ": keys")
        assert_same_bits(host(self.gd), res.gbar, name + ": gbar")
        assert_same_bits(host(self.wd), w_ref, name + ": w")
        assert_same_bits(host(self.vd), v_ref, name + ": v")
        assert_residual(self.flush(scratch), ref_dev, self.plan.P, name + ": flushed residual")


def _sparse_setup(ga):
    wl = workloads.WORKLOADS["alexnet128_sparse"]
    plan = ga.Plan(wl.W, wl.numels, True, chunk=wl.chunk, keep_ratio=wl.rho)
    return wl, plan, workloads.segments(wl)


@pytest.mark.parametrize("depth,steps,resume_after", [(2, 4, 2), (1, 3, 1)])
def test_sparse_alexnet128_full_size_deferred(ga, depth, steps, resume_after):
    """The deferred form at full size (depth 2 as benchmarked, and depth 1),
    every output against the oracle at every step (the residual of all 128
    workers through a flush into a copy).  A second run beside the straight
    one is checkpointed after step `resume_after`, a step that did not store
    the residual: flushed in place, its residual, weights and velocity copied
    to the host, its device buffers and history dropped, and resumed from the
    host copies alone (age 0, no mask, no earlier gradient tensor); it must
    match the oracle, and so the straight run, at every later step.  The
    straight run at depth 2 passes every age (0, 1, 2, then 0 again)."""
    wl, plan, seg = _sparse_setup(ga)
    C, P, ld, k = wl.chunk, wl.P, plan.ld, plan.k
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((wl.W, ld), np.float32)
    runs = {"straight": DeviceRun(plan, w_ref)}
    if resume_after:
        runs["resumed"] = DeviceRun(plan, w_ref)
    scratch = plan.empty_residual()
    kept = []
    for step in range(1, steps + 1):
        t0 = time.time()
        b = workloads.grad_bucket(wl, step, ld, seg=seg)
        buf, ptrs = device_layers(b[:, :P], wl.numels)
        kept = (kept + [buf])[-(depth + 1):]
        res = oracle.sparse_step(b, P, True, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        del b
        assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        ref_dev = torch.from_numpy(r_ref).cuda()
        log("depth %d step %d: inputs and oracle in %.1fs" % (depth, step, time.time() - t0))
        for name, run in runs.items():
            run.step(ptrs, depth, wl.lr, wl.mu)
            torch.cuda.synchronize()
            run.check(res, w_ref, v_ref, ref_dev, scratch, "depth %d %s step %d" % (depth, name, step))
        del ref_dev
        if resume_after and step == resume_after:
            old = runs.pop("resumed")
            old.flush(old.rd)
            torch.cuda.synchronize()
            saved = (host(old.rd), host(old.wd), host(old.vd))
            del old
            torch.cuda.empty_cache()
            new = DeviceRun(plan, saved[1], saved[2])
            new.rd.copy_(torch.from_numpy(saved[0]))
            del saved
            runs["resumed"] = new          # age 0, no mask, no earlier tensor
            log("depth %d: checkpoint after step %d, resumed from the host copy" % (depth, step))
        log("depth %d step %d compared in %.1fs" % (depth, step, time.time() - t0))


def test_sparse_alexnet128_deferred_deterministic(ga):
    """The benchmarked step at full size (depth 2, so that every earlier-step
    table and mask is in play) repeated ten times from one saved state: keys,
    masks, mean gradient, weights, velocity and the flushed residual are
    bitwise identical every time."""
    wl, plan, seg = _sparse_setup(ga)
    P, ld, depth = wl.P, plan.ld, 2
    run = DeviceRun(plan, workloads.weights(wl))
    scratch = plan.empty_residual()
    kept, ptrs = [], None
    for step in range(1, 4):
        b = workloads.grad_bucket(wl, step, ld, seg=seg)
        buf, ptrs = device_layers(b[:, :P], wl.numels)
        del b
        kept = (kept + [buf])[-(depth + 1):]
        if step < 3:
            run.step(ptrs, depth, wl.lr, wl.mu)
        log("deterministic: step %d ready" % step)
    state = (run.rd.clone(), run.wd.clone(), run.vd.clone(), list(run.masks), list(run.tables))
    first = None
    for rep in range(10):
        run.rd.copy_(state[0])
        run.wd.copy_(state[1])
        run.vd.copy_(state[2])
        run.masks, run.tables = list(state[3]), list(state[4])
        run.step(ptrs, depth, wl.lr, wl.mu)
        out = [run.keys.view(torch.int64).clone(), run.masks[0].clone(), run.gd.view(torch.int32).clone(),
               run.wd.view(torch.int32).clone(), run.vd.view(torch.int32).clone()]
        run.flush(scratch)
        torch.cuda.synchronize()
        if first is None:
            first, first_r = out, scratch.clone()
        else:
            for name, a, b in zip(("keys", "mask", "gbar", "w", "v"), first, out):
                assert torch.equal(a, b), "repetition %d: %s differs" % (rep, name)
            assert torch.equal(scratch.view(torch.int32), first_r.view(torch.int32)), "repetition %d: residual" % rep
        log("deterministic: repetition %d done" % rep)
