"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, against the oracle run on the host cores.

NiN-, GoogLeNet- and AlexNet-shaped dense aggregation are compared on every
element, from a packed bucket and from the per-layer tensors.  The
AlexNet-shaped W=128 sparse workload is run as benchmarked (2048 per-layer
tensors read with zero copy, 3 consecutive steps, lazy-zero residual with one
reused mask buffer) and compared on every selected index, every key, every
mean-gradient/weight/velocity element and the residual of a sample of
workers."""
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


def log(msg):
    print("[fullsize] %s" % msg, flush=True)


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


def test_sparse_alexnet128_full_size(ga):
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
    sample = [0, 1, 63, 127]
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
        # lazy-zero mode, one mask buffer reused across steps, as benchmarked
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
        m = host(mask).view(np.uint32)
        for w in sample:
            r = host(rd[w, :P]).copy()
            for c in range(n_c):
                if (int(m[w, c >> 5]) >> (c & 31)) & 1:
                    r[c * C:min((c + 1) * C, P)] = 0.0
            assert_same_bits(r, r_ref[w, :P], "residual of worker %d" % w)
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


@pytest.mark.parametrize("mode,steps", [("defer", 3), ("pending", 4), ("pending2", 5)])
def test_sparse_alexnet128_full_size_deferred(ga, mode, steps):
    """The AlexNet-shaped W=128 sparse workload as benchmarked: 2048 per-layer
    tensors, consecutive steps in deferred lazy-zero mode (two mask buffers)
    or its pending forms (the previous steps' tensors kept; the residual is
    compared through a flushed copy), every output compared with the oracle."""
    wl = workloads.WORKLOADS["alexnet128_sparse"]
    C = wl.chunk
    plan = ga.Plan(wl.W, wl.numels, True, chunk=C, keep_ratio=wl.rho)
    P, ld, k, n_c = wl.P, plan.ld, plan.k, plan.n_chunks
    seg = workloads.segments(wl)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((wl.W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd = plan.empty_residual()
    keys = plan.empty_keys()
    idx = torch.empty((wl.W, k), dtype=torch.int32, device="cuda")
    masks = [torch.zeros((wl.W, plan.mask_words), dtype=torch.int32, device="cuda") for _ in range(3)]
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    sample = [0, 1, 63, 127]
    prev_layers = []
    for step in range(1, steps + 1):
        t0 = time.time()
        b = workloads.grad_bucket(wl, step, ld, seg=seg)
        buf, ptrs = device_layers(b[:, :P], wl.numels)
        res = oracle.sparse_step(b, P, True, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        del b
        prev, cur = masks[(step + 1) % 2], masks[step % 2]
        if mode == "pending2":
            cur, prev, prev2 = masks[step % 3], masks[(step + 2) % 3], masks[(step + 1) % 3]
        r_view = rd
        if mode == "defer":
            plan.chunk_norm_layers_defer(ptrs, rd, keys, prev)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_defer(ptrs, rd, prev, cur, gd, wd, vd, wl.lr, wl.mu)
        elif mode == "pending2":
            pptrs = prev_layers[-1][1] if prev_layers else ptrs
            ppptrs = prev_layers[-2][1] if len(prev_layers) > 1 else ptrs
            plan.chunk_norm_layers_pending2(ptrs, pptrs, ppptrs, rd, keys, prev, prev2, cur)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_pending2(ptrs, pptrs, rd, prev, cur, prev2, gd, wd, vd, wl.lr, wl.mu)
            r_view = rd.clone()
            plan.residual_flush_layers2(ptrs, pptrs, r_view, prev, cur, prev2)
            prev_layers = (prev_layers + [(buf, ptrs)])[-2:]
        else:
            pptrs = prev_layers[-1][1] if prev_layers else ptrs
            plan.chunk_norm_layers_pending(ptrs, pptrs, rd, keys, prev, cur)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_pending(ptrs, rd, prev, cur, gd, wd, vd, wl.lr, wl.mu)
            r_view = rd.clone()
            plan.residual_flush_layers(ptrs, r_view, prev, cur)
            prev_layers = [(buf, ptrs)]
        torch.cuda.synchronize()
        del buf
        assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        assert np.array_equal(host(idx), res.sel_idx), "selected chunk indices differ"
        assert np.array_equal(host(cur).view(np.uint32), res.sel_mask)
        assert_close(host(keys), res.keys, KEY_RTOL, "keys")
        assert_same_bits(host(gd), res.gbar, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
        m = host(cur).view(np.uint32)
        for w in sample:
            r = host(r_view[w, :P]).copy()
            for c in range(n_c):
                if (int(m[w, c >> 5]) >> (c & 31)) & 1:
                    r[c * C:min((c + 1) * C, P)] = 0.0
            assert_same_bits(r, r_ref[w, :P], "residual of worker %d" % w)
        del r_view
        log("%s step %d compared in %.1fs" % (mode, step, time.time() - t0))
