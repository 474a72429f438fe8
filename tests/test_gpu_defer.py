"""GPU parity of the deferred-residual sparse step (norms that do not store a
for chunks sent in the previous step; a gather that reads the gradient tensors
for chunks sent twice in a row and writes the residual of chunks sent before
but not now) against the oracle over consecutive steps, and bit for bit
against the plain lazy-zero sequence on the GPU.  The pending form (that
residual left as the step's gradient, read by the next step's norm pass, and
written on demand by the flush) is checked the same way: its residual through
a flushed copy, so the steps themselves never see a flush, and once more with
the live buffer flushed after every step."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, assert_close, assert_same_bits, device_layers, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MIS = {"aligned": lambda w, l: 0, "mixed": lambda w, l: (3 * w + l) % 4}


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def sent_elements(mask, C, P, n_c):
    m = np.asarray(mask).view(np.uint32).astype(np.int64)
    ch = np.arange(n_c)
    sent = ((m[:, ch >> 5] >> (ch & 31)) & 1).astype(bool)
    return np.repeat(sent, C, axis=1)[:, :P]


def run_defer(ga, wl, mis="aligned", steps=4, hook=None, strict=False, mode="defer"):
    C, P = wl.chunk, wl.P
    plan = ga.Plan(wl.W, wl.numels, wl.fp16, chunk=C, keep_ratio=wl.rho)
    ld, k, n_c = plan.ld, plan.k, plan.n_chunks
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((wl.W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd, keys = plan.empty_residual(), plan.empty_keys()
    idx = torch.full((wl.W, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    masks = [torch.zeros((wl.W, plan.mask_words), dtype=torch.int32, device="cuda") for _ in range(3)]
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    print("[%s] W=%d P=%d fp16=%s C=%d rho=%g %s" % (mode, wl.W, P, wl.fp16, C, wl.rho, mis), flush=True)
    prev_layers = []        # the previous steps' tensors, kept alive for the pending forms
    for step in range(1, steps + 1):
        b = workloads.grad_bucket(wl, step, ld)
        if hook is not None:
            hook(b, step)
        res = oracle.sparse_step(b, P, wl.fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        if mode.startswith("pending2"):
            # three buffers in turn: cur holds the mask of three steps back
            cur, prev, prev2 = masks[step % 3], masks[(step + 2) % 3], masks[(step + 1) % 3]
        else:
            cur, prev = masks[step % 2], masks[(step + 1) % 2]
        buf, ptrs = device_layers(b[:, :P], wl.numels, MIS[mis])
        r_view = rd
        if mode == "defer":
            plan.chunk_norm_layers_defer(ptrs, rd, keys, prev)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_defer(ptrs, rd, prev, cur, gd, wd, vd, wl.lr, wl.mu)
        elif mode.startswith("pending2"):
            pptrs = prev_layers[-1][1] if prev_layers else ptrs
            ppptrs = prev_layers[-2][1] if len(prev_layers) > 1 else ptrs
            plan.chunk_norm_layers_pending2(ptrs, pptrs, ppptrs, rd, keys, prev, prev2, cur)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_pending2(ptrs, pptrs, rd, prev, cur, prev2, gd, wd, vd, wl.lr, wl.mu)
            if mode == "pending2_flush":
                plan.residual_flush_layers2(ptrs, pptrs, rd, prev, cur, prev2)
            else:
                r_view = rd.clone()
                plan.residual_flush_layers2(ptrs, pptrs, r_view, prev, cur, prev2)
            prev_layers = (prev_layers + [(buf, ptrs)])[-2:]
        else:
            # cur still holds the mask of two steps back (all zero at first)
            pptrs = prev_layers[-1][1] if prev_layers else ptrs
            plan.chunk_norm_layers_pending(ptrs, pptrs, rd, keys, prev, cur)
            plan.chunk_topk(keys, idx, cur)
            plan.sparse_gather_reduce_layers_pending(ptrs, rd, prev, cur, gd, wd, vd, wl.lr, wl.mu)
            if mode == "pending_flush":
                plan.residual_flush_layers(ptrs, rd, prev, cur)
            else:
                r_view = rd.clone()
                plan.residual_flush_layers(ptrs, r_view, prev, cur)
            prev_layers = [(buf, ptrs)]
        torch.cuda.synchronize()
        if wl.rho not in (0.0, 1.0):
            assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        assert_close(host(keys), res.keys, KEY_RTOL, "keys")
        if k > 0:
            assert np.array_equal(host(idx)[:, :k], res.sel_idx), "selected chunk indices differ"
        assert np.array_equal(host(cur).view(np.uint32), res.sel_mask)
        r_got = host(r_view)[:, :P].copy()
        r_got[sent_elements(host(cur), C, P, n_c)] = 0.0
        same = assert_same_bits
        if strict:
            def same(got, ref, name):
                assert np.array_equal(np.asarray(got).view(np.uint32), np.asarray(ref).view(np.uint32)), name
        same(r_got, r_ref[:, :P], "residual step %d" % step)
        same(host(gd), res.gbar, "gbar step %d" % step)
        same(host(wd), w_ref, "w step %d" % step)
        same(host(vd), v_ref, "v step %d" % step)
    plan.close()


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", [(1, [3000, 7, 2000], 256), (3, workloads.WORKLOADS["tiny"].numels, 512),
                                        (16, [8, 1, 5000, 7, 4096, 333, 64], 256), (33, [20000, 37, 4003], 1024),
                                        (128, [2048, 16, 4099, 520], 256), (300, [3000, 17, 1000], 512)])
@pytest.mark.parametrize("mis", list(MIS))
def test_defer_matches_oracle(ga, fp16, W, numels, C, mis):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    run_defer(ga, wl, mis)


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", [(1, [3000, 7, 2000], 256), (3, workloads.WORKLOADS["tiny"].numels, 512),
                                        (16, [8, 1, 5000, 7, 4096, 333, 64], 256), (33, [20000, 37, 4003], 1024),
                                        (128, [2048, 16, 4099, 520], 256), (300, [3000, 17, 1000], 512)])
@pytest.mark.parametrize("mis", list(MIS))
def test_pending_matches_oracle(ga, fp16, W, numels, C, mis):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    run_defer(ga, wl, mis, steps=5, mode="pending")


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,C", [(1, [3000, 7, 2000], 256), (3, workloads.WORKLOADS["tiny"].numels, 512),
                                        (16, [8, 1, 5000, 7, 4096, 333, 64], 256), (33, [20000, 37, 4003], 1024),
                                        (128, [2048, 16, 4099, 520], 256), (300, [3000, 17, 1000], 512)])
@pytest.mark.parametrize("mis", list(MIS))
def test_pending2_matches_oracle(ga, fp16, W, numels, C, mis):
    wl = workloads.custom(W, numels, fp16, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0), chunk=C,
                          rho=0.2)
    run_defer(ga, wl, mis, steps=6, mode="pending2")


@pytest.mark.parametrize("fp16", [False, True])
def test_pending2_flushed_every_step(ga, fp16):
    wl = workloads.custom(16, [8, 1, 5000, 7, 4096, 333, 64], fp16, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.2)
    run_defer(ga, wl, "mixed", steps=6, mode="pending2_flush")


@pytest.mark.parametrize("fp16", [False, True])
def test_pending_flushed_every_step(ga, fp16):
    """Flushing the live residual after every step changes nothing: the next
    norm pass computes the same pending values itself."""
    wl = workloads.custom(16, [8, 1, 5000, 7, 4096, 333, 64], fp16, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.2)
    run_defer(ga, wl, "mixed", steps=5, mode="pending_flush")


@pytest.mark.parametrize("mode", ["defer", "pending", "pending2"])
@pytest.mark.parametrize("rho", [0.0, 1.0])
def test_defer_keep_ratio_extremes(ga, rho, mode):
    wl = workloads.custom(6, [9000, 11, 300], True, sigma=1e-2, chunk=256, rho=rho)
    run_defer(ga, wl, "mixed", steps=3, mode=mode)


def test_defer_negative_zero_leaves(ga):
    """A chunk sent twice in a row has a = g + 0: a -0 gradient becomes +0, as
    in the non-deferred pass, so the sums and the residual match bit for bit."""
    def hook(b, step):
        b[:, 100:300] = 0x8000          # binary16 -0 in every worker
        b[1:, 600:700] = 0x8000
    for mode in ("defer", "pending", "pending2"):
        wl = workloads.custom(4, [3000], True, sigma=1e-2, chunk=256, rho=1.0)
        run_defer(ga, wl, "aligned", steps=3, hook=hook, strict=True, mode=mode)
        wl = workloads.custom(4, [3000], True, sigma=1e-2, chunk=256, rho=0.5)
        run_defer(ga, wl, "aligned", steps=5, hook=hook, strict=True, mode=mode)


def test_defer_errors(ga):
    plan = ga.Plan(4, [1000], True, chunk=64, keep_ratio=0.5)
    ptrs = torch.zeros(4, dtype=torch.int64, device="cuda")
    rd = plan.empty_residual()
    m0 = torch.zeros((4, plan.mask_words), dtype=torch.int32, device="cuda")
    m1 = torch.zeros((4, plan.mask_words), dtype=torch.int32, device="cuda")
    g = torch.zeros(plan.P, device="cuda")
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_defer(ptrs, rd, m0, m1, g)
    assert e.value.status == ga.GA_ERR_UNSUPPORTED
    plan = ga.Plan(4, [1000], True, chunk=256, keep_ratio=0.5)
    rd = plan.empty_residual()
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_defer(ptrs, rd, m0, m0, g)
    assert e.value.status == ga.GA_ERR_INVALID
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_pending(ptrs, rd, m0, m0, g)
    assert e.value.status == ga.GA_ERR_INVALID
    m2 = torch.zeros((4, plan.mask_words), dtype=torch.int32, device="cuda")
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_pending2(ptrs, ptrs, rd, m0, m1, m1, g)
    assert e.value.status == ga.GA_ERR_INVALID
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_pending2(ptrs, ptrs, rd, m1, m1, m2, g)
    assert e.value.status == ga.GA_ERR_INVALID
    plan = ga.Plan(4, [1000], True, chunk=64, keep_ratio=0.5)
    rd = plan.empty_residual()
    with pytest.raises(ga.GAError) as e:
        plan.sparse_gather_reduce_layers_pending(ptrs, rd, m0, m1, g)
    assert e.value.status == ga.GA_ERR_UNSUPPORTED

