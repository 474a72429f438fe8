"""GPU parity of the dense path (tree reduce + mean + fused SGD, standalone SGD)
against the oracle, element by element, at sizes that span many workgroups and
end in a ragged tail, and on the edge cases of the method."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import TOL_FP16_PATH, TOL_FP32, assert_close, assert_same_bits, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def run_dense(ga, wl, steps=2, pad_value=None, bucket_hook=None, want_grad=True, want_sgd=True):
    plan = ga.Plan(wl.W, wl.numels, wl.fp16)
    P = wl.P
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    for step in range(1, steps + 1):
        b = workloads.grad_bucket(wl, step, plan.ld)
        if bucket_hook is not None:
            bucket_hook(b)
        if pad_value is not None and plan.ld > P:
            b[:, P:] = pad_value
        g_ref = oracle.dense_step(b, P, wl.fp16, wl.lr, wl.mu, w_ref if want_sgd else None,
                                  v_ref if want_sgd else None)
        if want_sgd:
            plan.tree_reduce(to_dev(b, wl.fp16), gd if want_grad else None, wd, vd, wl.lr, wl.mu)
        else:
            plan.tree_reduce(to_dev(b, wl.fp16), gd)
        torch.cuda.synchronize()
        tol = TOL_FP16_PATH if wl.fp16 else TOL_FP32
        if want_grad:
            assert_close(host(gd), g_ref, tol, "gbar")
            assert_same_bits(host(gd), g_ref, "gbar")
        if want_sgd:
            assert_close(host(wd), w_ref, TOL_FP32, "w")
            assert_same_bits(host(wd), w_ref, "w")
            assert_same_bits(host(vd), v_ref, "v")
    plan.close()


@pytest.mark.parametrize("W", [1, 2, 3, 5, 7, 8, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 300, 1024])
@pytest.mark.parametrize("fp16", [False, True])
def test_dense_worker_counts(ga, W, fp16):
    P_layers = [1000, 3, 517] if W > 300 else [4096 * 7 + 5, 10, 999]
    wl = workloads.custom(W, P_layers, fp16, sigma=1e-2, scale_mode="layer")
    run_dense(ga, wl, steps=2)


@pytest.mark.parametrize("numels", [[1], [7], [9], [8], [4099], [64, 1], [300001, 17, 64 * 1024]])
@pytest.mark.parametrize("fp16", [False, True])
def test_dense_ragged_sizes(ga, numels, fp16):
    wl = workloads.custom(6, numels, fp16, sigma=1e-3)
    run_dense(ga, wl, steps=1, pad_value=np.nan if not fp16 else 0x7E00)


def test_dense_tiny_workload_three_steps(ga):
    run_dense(ga, workloads.WORKLOADS["tiny"], steps=3)


@pytest.mark.parametrize("fp16", [False, True])
def test_dense_grad_only_and_sgd_only(ga, fp16):
    wl = workloads.custom(12, [5000, 333], fp16)
    run_dense(ga, wl, steps=1, want_grad=True, want_sgd=False)
    run_dense(ga, wl, steps=1, want_grad=False, want_sgd=True)


def test_dense_fp16_special_values(ga):
    """Subnormals, signed zeros, the largest finite value, infinities and NaN
    travel through the binary16 leaves exactly as the oracle decodes them."""
    specials = np.array([0x0001, 0x03FF, 0x8001, 0x0000, 0x8000, 0x7BFF, 0xFBFF, 0x0400, 0x3C00,
                         0x7C00, 0xFC00, 0x7E00, 0x3555, 0x0200], np.uint16)

    def hook(b):
        rng = np.random.default_rng(3)
        W = b.shape[0]
        for r in range(W):
            b[r, :4096] = rng.choice(specials, 4096)
        b[:, 4096:8192] = 0x0001       # all workers subnormal: exact sums of 2^-24
        b[:, 8192:8200] = 0x8000       # all -0: the sum keeps the sign
    wl = workloads.custom(8, [10000], True)
    run_dense(ga, wl, steps=1, bucket_hook=hook)


@pytest.mark.parametrize("W", [2, 4, 64, 128])
def test_identical_power_of_two_buffers_average_to_themselves(ga, W):
    plan = ga.Plan(W, [12345], True)
    row = (np.random.default_rng(W).standard_normal(plan.ld) * 1e-3).astype(np.float16)
    b = np.tile(row, (W, 1))
    gd = torch.empty(plan.P, dtype=torch.float32, device="cuda")
    plan.tree_reduce(to_dev(b.view(np.uint16), True), gd)
    torch.cuda.synchronize()
    assert np.array_equal(host(gd), row[:plan.P].astype(np.float32))


def test_standalone_sgd(ga):
    rng = np.random.default_rng(7)
    for P in (1, 3, 4, 1001, 1 << 20):
        g = rng.standard_normal(P).astype(np.float32)
        w = rng.standard_normal(P).astype(np.float32)
        v = rng.standard_normal(P).astype(np.float32)
        wd, vd = to_dev(w.copy()), to_dev(v.copy())
        ga.sgd_momentum_apply(to_dev(g), wd, vd, 0.01, 0.9)
        oracle.sgd(g, w, v, 0.01, 0.9)
        torch.cuda.synchronize()
        assert_same_bits(host(wd), w, "w")
        assert_same_bits(host(vd), v, "v")


def test_dense_deterministic(ga):
    wl = workloads.custom(128, [1 << 18, 77], True)
    plan = ga.Plan(wl.W, wl.numels, True)
    bd = to_dev(workloads.grad_bucket(wl, 1, plan.ld), True)
    outs = []
    for _ in range(3):
        gd = torch.empty(plan.P, dtype=torch.float32, device="cuda")
        plan.tree_reduce(bd, gd)
        outs.append(host(gd))
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


def test_device_argument_errors(ga):
    plan = ga.Plan(4, [1000], False)
    b = torch.zeros(4 * plan.ld + 1, dtype=torch.float32, device="cuda")
    g = torch.zeros(plan.P + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(ga.GAError) as e:
        plan.tree_reduce(b[1:], g[:plan.P])
    assert e.value.status == ga.GA_ERR_ALIGN
    with pytest.raises(ga.GAError) as e:
        plan.tree_reduce(b[:4 * plan.ld], g[1:])
    assert e.value.status == ga.GA_ERR_ALIGN
    with pytest.raises(ga.GAError) as e:
        plan.chunk_norm(b, torch.zeros(4 * plan.ld, device="cuda"), torch.zeros(4, dtype=torch.float64,
                                                                                 device="cuda"))
    assert e.value.status == ga.GA_ERR_INVALID
    # every entry point that writes g, w, v with 128-bit stores rejects a misaligned one before launching
    wv = torch.zeros(plan.P + 1, dtype=torch.float32, device="cuda")
    for call in (lambda: plan.reduce_variant(b[:4 * plan.ld], "ring", False, g[1:]),
                 lambda: plan.reduce_variant(b[:4 * plan.ld], "server", True, None, wv[1:], wv[:plan.P], 0.1, 0.9),
                 lambda: plan.tree_reduce(b[:4 * plan.ld], None, wv[:plan.P], wv[1:], 0.1, 0.9)):
        with pytest.raises(ga.GAError) as e:
            call()
        assert e.value.status == ga.GA_ERR_ALIGN
    with pytest.raises(ValueError):
        plan.tree_reduce(b[:4 * plan.ld].cpu(), g)
    with pytest.raises(ValueError):
        plan.tree_reduce(torch.zeros(10, device="cuda"), g)
