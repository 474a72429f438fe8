"""bench.py's full-size parity verdict, on small workloads: the timed path
run for as many steps as the cpu_baseline leg ran the oracle, from the same
state, must report bitwise agreement of w, v and the residual, and must
report a difference planted in the oracle's state."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bench():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench as b
    return b


def _setup(bench, wl):
    import gradient_aggregation_amd as ga
    plan = ga.Plan(wl.W, wl.numels, wl.fp16, chunk=wl.chunk, keep_ratio=wl.rho)
    sources, keep, host_first = bench.load_batches(wl, plan, 1, True, 4, True)
    w_init = workloads.weights(wl)
    return plan, sources, keep, host_first, w_init


def _planted(ostate, where):
    """A copy of the oracle's state with one value moved by one ulp."""
    steps, w, v, r = ostate
    w, v = w.copy(), v.copy()
    r = None if r is None else r.copy()
    arr, idx = {"w": (w, 17), "v": (v, 3), "r": (r, (1, 5))}[where]
    arr[idx] = np.nextafter(arr[idx], np.float32(np.inf))
    return steps, w, v, r


@pytest.mark.parametrize("mode,depth", [("deferred", 2), ("deferred", 1), ("lazy", 0)])
def test_sparse_parity_verdict(bench, mode, depth):
    wl = workloads.custom(5, [3000, 17, 1000, 2500], True, sigma=1e-3, mode="sparse", scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.25)
    plan, sources, keep, host_first, w_init = _setup(bench, wl)
    print("[bench-parity] %s depth %d: W=%d P=%d n_c=%d k=%d" % (mode, depth, wl.W, wl.P, plan.n_chunks, plan.k),
          flush=True)
    _, ostate = bench.cpu_baseline(wl, plan, host_first, w_init, 2, min_s=1e9, max_steps=3)
    assert ostate[0] == 3
    got = bench.full_size_parity(plan, wl, sources[0], w_init, mode, depth, True, ostate)
    assert (got["w"], got["v"]) == ("bitwise", "bitwise"), got
    assert got["residual"] == "bitwise, all 5 workers", got
    for where in ("w", "v", "r"):
        bad = bench.full_size_parity(plan, wl, sources[0], w_init, mode, depth, True, _planted(ostate, where))
        if where == "r":
            assert bad["residual"] == "1 elements differ" and bad["w"] == "bitwise", bad
        else:
            assert bad[where] == "differs", bad


def test_dense_parity_verdict(bench):
    wl = workloads.custom(6, [1000, 37, 4099], True, sigma=1e-2, scale_mode="layer")
    plan, sources, keep, host_first, w_init = _setup(bench, wl)
    _, ostate = bench.cpu_baseline(wl, plan, host_first, w_init, 2, min_s=1e9, max_steps=4)
    got = bench.full_size_parity(plan, wl, sources[0], w_init, "lazy", 0, True, ostate)
    assert (got["w"], got["v"], got["form"]) == ("bitwise", "bitwise", "dense tree"), got
    assert bench.full_size_parity(plan, wl, sources[0], w_init, "lazy", 0, True, _planted(ostate, "v"))["v"] \
        == "differs"
