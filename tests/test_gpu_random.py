"""Seeded random configurations, each run through every entry point of the
path that applies to it and compared with the oracle element by element:
random worker counts, layer lists (aligned and ragged sizes, small and large
layers), binary16 or binary32 gradients, chunk sizes and keep ratios, both
residual modes, zero-copy tensors at random misalignments, and multi-bucket
schedules at random thresholds, and the deferred residual form where it
applies (a random depth and store schedule, layer tensors whose alignment
changes from step to step, the residual checked through a flushed copy).
The case is printed before it runs."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, assert_close, assert_same_bits, device_layers, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 150


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 17, 31, 64, 65, 100, 128, 200]))
    L = int(rng.integers(1, 13))
    numels = []
    for _ in range(L):
        r = rng.random()
        n = int(rng.integers(1, 40)) if r < 0.3 else int(rng.integers(40, 3000)) if r < 0.8 else \
            int(rng.integers(3000, 40000))
        if rng.random() < 0.4:
            n = 8 * ((n + 7) // 8)
        numels.append(n)
    fp16 = bool(rng.random() < 0.6)
    sparse = bool(rng.random() < 0.5)
    u = rng.random()
    # a multiple of 256 (the deferred form applies), one longer than a 2048-element
    # norm part (the storing pass splits it), or any multiple of 8
    chunk = ((256 * int(rng.integers(1, 4)) if u < 0.4 else 256 * int(rng.integers(9, 33)) if u < 0.55
              else 8 * int(rng.integers(1, 65))) if sparse else 0)
    rho = float(rng.choice([0.0, 0.05, 0.1, 0.25, 0.5, 1.0, rng.random()])) if sparse else 0.0
    lazy = bool(rng.random() < 0.5)
    # deferred residual where it applies (C a multiple of 256)
    deferred = bool(sparse and chunk % 256 == 0 and rng.random() < 0.7)
    mis = int(rng.integers(0, 4))
    thr = int(rng.choice([1, 64, 1024, 16384, 1 << 30]))
    depth = int(rng.integers(0, 3)) if deferred else None
    return dict(W=W, numels=numels, fp16=fp16, sparse=sparse, chunk=chunk, rho=rho, lazy=lazy or deferred,
                deferred=deferred, mis=mis, thr=thr, depth=depth)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(ga, seed):
    c = draw(seed)
    print("[random] seed %d: %s" % (seed, c), flush=True)
    W, numels, fp16 = c["W"], c["numels"], c["fp16"]
    misalign = (lambda w, l: 0) if c["mis"] == 0 else (lambda w, l: (c["mis"] * w + l) % 4)
    if not c["sparse"]:
        wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer", index=200 + seed)
        plan = ga.Plan(W, numels, fp16)
        bk = ga.Buckets(plan, c["thr"])
        w_ref = workloads.weights(wl)
        v_ref = np.zeros(wl.P, np.float32)
        dev = {k: (to_dev(w_ref.copy()), to_dev(v_ref.copy())) for k in ("bucket", "layers", "buckets")}
        gd = {k: torch.empty(wl.P, dtype=torch.float32, device="cuda") for k in dev}
        for step in (1, 2):
            b = workloads.grad_bucket(wl, step, plan.ld)
            g_ref = oracle.dense_step(b, wl.P, fp16, wl.lr, wl.mu, w_ref, v_ref)
            buf, ptrs = device_layers(b[:, :wl.P], numels, misalign)
            plan.tree_reduce(to_dev(b, fp16), gd["bucket"], *dev["bucket"], wl.lr, wl.mu)
            plan.tree_reduce_layers(ptrs, gd["layers"], *dev["layers"], wl.lr, wl.mu)
            for i in range(bk.count):
                bk.reduce_layers(i, ptrs, None, gd["buckets"], *dev["buckets"], wl.lr, wl.mu,
                                 max_workgroups=(0 if seed % 2 else 5))
            torch.cuda.synchronize()
            for k in dev:
                assert_same_bits(host(gd[k]), g_ref, "%s gbar" % k)
                assert_same_bits(host(dev[k][0]), w_ref, "%s w" % k)
                assert_same_bits(host(dev[k][1]), v_ref, "%s v" % k)
        return
    C, rho = c["chunk"], c["rho"]
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=rho, index=200 + seed)
    plan = ga.Plan(W, numels, fp16, chunk=C, keep_ratio=rho)
    P, ld, k, n_c = wl.P, plan.ld, plan.k, plan.n_chunks
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd, keys = plan.empty_residual(), plan.empty_keys()
    idx = torch.full((W, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    mask = torch.zeros((W, plan.mask_words), dtype=torch.int32, device="cuda")
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    depth = c["depth"]
    rng = np.random.default_rng(5000 + seed)
    hist_masks, hist_tables, kept = [None], [], []
    for step in range(1, 6 if depth is not None else 4):
        b = workloads.grad_bucket(wl, step, ld)
        res = oracle.sparse_step(b, P, fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        mis_t = (lambda w, l: 0) if c["mis"] == 0 else (lambda w, l: (c["mis"] * w + l + step) % 4)
        buf, ptrs = device_layers(b[:, :P], numels, mis_t)
        r_view = rd
        cur = mask
        if depth is not None:
            # a random store schedule that never holds more than `depth` earlier steps
            age = len(hist_masks) - 1
            store = age >= depth or bool(rng.random() < 0.3)
            hist = plan.history(hist_masks, hist_tables)
            cur = torch.zeros((W, plan.mask_words), dtype=torch.int32, device="cuda")
            plan.chunk_norm_deferred(ptrs, hist, store, rd, keys)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_deferred(ptrs, hist, store, rd, cur, gd, wd, vd, wl.lr, wl.mu)
            r_view = rd.clone()
            plan.residual_flush(ptrs, hist, store, r_view, cur)
            if store:
                hist_masks, hist_tables, kept = [cur], [], []
            else:
                hist_masks, hist_tables, kept = [cur] + hist_masks, [ptrs] + hist_tables, [buf] + kept
        else:
            plan.chunk_norm_layers(ptrs, rd, keys, mask if (c["lazy"] and step > 1) else None)
            plan.chunk_topk(keys, idx, mask)
            plan.sparse_gather_reduce(rd, mask, not c["lazy"], gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        if not np.all(res.margin > 1e-12):
            pytest.skip("selection boundary too close to certify at seed %d" % seed)
        assert_close(host(keys), res.keys, KEY_RTOL, "keys")
        if k > 0:
            assert np.array_equal(host(idx)[:, :k], res.sel_idx), "selected chunk indices differ"
        assert np.array_equal(host(cur).view(np.uint32), res.sel_mask)
        r_got = host(r_view)
        if c["lazy"]:
            m = host(cur).view(np.uint32).astype(np.int64)
            ch = np.arange(n_c)
            sent = ((m[:, ch >> 5] >> (ch & 31)) & 1).astype(bool)          # [W][n_c]
            r_got[:, :P][np.repeat(sent, C, axis=1)[:, :P]] = 0.0
        assert_same_bits(r_got[:, :P], r_ref[:, :P], "residual")
        assert_same_bits(host(gd), res.gbar, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
