"""GPU parity of the sparse path (chunk norms with the residual, top-k chunk
selection, gather-reduce with the residual split, fused SGD) against the
oracle over several consecutive steps, in both residual modes."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, TOL_FP16_PATH, TOL_FP32, assert_close, assert_same_bits, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def mask_chunks(mask_row, n_c):
    m = np.asarray(mask_row).view(np.uint32)
    return [c for c in range(n_c) if (int(m[c >> 5]) >> (c & 31)) & 1]


def materialize(r, mask, C, P):
    """Residual of lazy-zero mode: chunks set in `mask` read as zero."""
    r = r.copy()
    m = np.asarray(mask).view(np.uint32)
    n_c = (P + C - 1) // C
    for w in range(r.shape[0]):
        for c in mask_chunks(m[w], n_c):
            r[w, c * C:min((c + 1) * C, P)] = 0.0
    return r


def run_sparse(ga, wl, steps=3, lazy=False, bucket_hook=None, require_margin=True, check_keys=True):
    C = wl.chunk
    plan = ga.Plan(wl.W, wl.numels, wl.fp16, chunk=C, keep_ratio=wl.rho)
    P, ld, k, n_c = wl.P, plan.ld, plan.k, plan.n_chunks
    assert k == oracle.keep_count(n_c, wl.rho)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(P, np.float32)
    r_ref = np.zeros((wl.W, ld), np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd = plan.empty_residual()
    keys = plan.empty_keys()
    idx = torch.full((wl.W, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    masks = [torch.zeros((wl.W, plan.mask_words), dtype=torch.int32, device="cuda") for _ in range(2)]
    gd = torch.empty(P, dtype=torch.float32, device="cuda")
    tol = TOL_FP16_PATH if wl.fp16 else TOL_FP32
    for step in range(1, steps + 1):
        b = workloads.grad_bucket(wl, step, ld)
        if bucket_hook is not None:
            bucket_hook(b, step)
        res = oracle.sparse_step(b, P, wl.fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        cur, prev = masks[step % 2], masks[(step + 1) % 2]
        plan.chunk_norm_topk(to_dev(b, wl.fp16), rd, keys, idx, cur, prev if (lazy and step > 1) else None)
        plan.sparse_gather_reduce(rd, cur, not lazy, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        if require_margin:
            assert np.all(res.margin > 1e-12), "selection boundary too close to certify"
        if check_keys:
            kh = host(keys)
            assert_close(kh, res.keys, KEY_RTOL, "keys")
        if k > 0:
            assert np.array_equal(host(idx)[:, :k], res.sel_idx), "selected chunk indices differ"
        assert np.array_equal(host(cur).view(np.uint32), res.sel_mask), "selection masks differ"
        r_got = host(rd)
        if lazy:
            r_got = materialize(r_got, host(cur), C, P)
        assert_same_bits(r_got[:, :P], r_ref[:, :P], "residual")
        assert_close(host(gd), res.gbar, tol, "gbar")
        assert_same_bits(host(gd), res.gbar, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
    plan.close()
    return res


TINY = workloads.TINY_LAYERS


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("C,rho", [(64, 0.25), (256, 0.1), (1024, 0.5), (8, 0.05),
                                   # chunks split into 2048-element norm parts (ragged, empty parts)
                                   (4352, 0.3), (8192, 0.5)])
@pytest.mark.parametrize("lazy", [False, True])
def test_sparse_tiny(ga, fp16, C, rho, lazy):
    numels = [int(np.prod(s)) for s in TINY]
    wl = workloads.custom(4, numels, fp16, sigma=1e-2, scale_mode="layer", chunk=C, rho=rho)
    run_sparse(ga, wl, steps=3, lazy=lazy)


@pytest.mark.parametrize("W", [1, 2, 3, 5, 33, 128, 300])
def test_sparse_worker_counts(ga, W):
    wl = workloads.custom(W, [20000, 37, 4003], True, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=512, rho=0.1)
    run_sparse(ga, wl, steps=3, lazy=(W % 2 == 1))


@pytest.mark.parametrize("rho", [0.0, 1.0])
def test_sparse_keep_ratio_extremes(ga, rho):
    wl = workloads.custom(6, [9000, 11], True, sigma=1e-2, chunk=256, rho=rho)
    run_sparse(ga, wl, steps=2)


def test_sparse_keep_ratio_one_equals_dense_on_gpu(ga):
    wl = workloads.custom(8, [30000, 5], True, sigma=1e-2, chunk=1024, rho=1.0)
    sp = ga.Plan(wl.W, wl.numels, True, chunk=1024, keep_ratio=1.0)
    dp = ga.Plan(wl.W, wl.numels, True)
    b = to_dev(workloads.grad_bucket(wl, 1, sp.ld), True)
    w0 = workloads.weights(wl)
    w1, v1 = to_dev(w0.copy()), torch.zeros(wl.P, device="cuda")
    w2, v2 = to_dev(w0.copy()), torch.zeros(wl.P, device="cuda")
    rd, keys = sp.empty_residual(), sp.empty_keys()
    idx, mask = sp.empty_sel()
    sp.chunk_norm_topk(b, rd, keys, idx, mask)
    sp.sparse_gather_reduce(rd, mask, True, None, w1, v1, wl.lr, wl.mu)
    dp.tree_reduce(b, None, w2, v2, wl.lr, wl.mu)
    torch.cuda.synchronize()
    assert np.array_equal(host(w1), host(w2)) and np.array_equal(host(v1), host(v2))
    assert not host(rd).any()


def test_sparse_partial_chunks_and_ragged(ga):
    # P = 10013: last chunk of 1000-element chunks has 13 elements; P % 8 != 0.
    wl = workloads.custom(7, [10000, 13], False, sigma=1e-2, chunk=1000, rho=0.3)
    run_sparse(ga, wl, steps=3, lazy=True)
    wl = workloads.custom(3, [50], True, sigma=1e-2, chunk=4096, rho=0.5)   # one chunk, shorter than C
    run_sparse(ga, wl, steps=2)


def test_sparse_many_chunks_multi_tile_topk(ga):
    """More chunks than the top-k kernel stages in LDS at once (4096)."""
    wl = workloads.custom(3, [8 * 9000 + 5], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=8, rho=0.1)
    run_sparse(ga, wl, steps=2)


def test_sparse_exact_ties_break_by_index(ga):
    """Chunks of equal constant power-of-two values have bitwise equal keys on
    both sides, so the index order alone decides: lower index first."""
    def hook(b, step):
        b[:] = 0
        vals = np.array([0x3C00, 0x4000, 0x3800], np.uint16)    # 1, 2, 0.5
        n_c = 40
        for c in range(n_c):
            b[:, c * 64:(c + 1) * 64] = vals[c % 3]
        b[1, 64:128] = 0x7E00                                   # a NaN chunk ranks first
    wl = workloads.custom(3, [40 * 64], True, chunk=64, rho=0.3)
    run_sparse(ga, wl, steps=1, bucket_hook=hook, require_margin=False)


def test_sparse_all_zero_gradients(ga):
    def hook(b, step):
        b[:] = 0
    wl = workloads.custom(4, [5000], False, chunk=64, rho=0.2)
    run_sparse(ga, wl, steps=2, bucket_hook=hook, require_margin=False)


def test_sparse_deterministic(ga):
    wl = workloads.custom(16, [1 << 17], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=4096, rho=0.1)
    plan = ga.Plan(wl.W, wl.numels, True, chunk=4096, keep_ratio=0.1)
    b = to_dev(workloads.grad_bucket(wl, 1, plan.ld), True)
    outs = []
    for _ in range(3):
        rd, keys = plan.empty_residual(), plan.empty_keys()
        idx, mask = plan.empty_sel()
        gd = torch.empty(plan.P, device="cuda")
        plan.chunk_norm_topk(b, rd, keys, idx, mask)
        plan.sparse_gather_reduce(rd, mask, True, gd)
        outs.append([host(t).copy() for t in (rd, keys, idx, mask, gd)])
    for o in outs[1:]:
        for a, b2 in zip(outs[0], o):
            assert np.array_equal(a.view(np.uint8), b2.view(np.uint8))


def test_checkpoint_resume_matches_straight_run(ga):
    wl = workloads.custom(8, [30000], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=512, rho=0.1)
    plan = ga.Plan(wl.W, wl.numels, True, chunk=512, keep_ratio=0.1)
    buckets = [to_dev(workloads.grad_bucket(wl, s, plan.ld), True) for s in (1, 2, 3)]

    def steps(state, which):
        rd, wd, vd = state
        for s in which:
            keys = plan.empty_keys()
            idx, mask = plan.empty_sel()
            plan.chunk_norm_topk(buckets[s - 1], rd, keys, idx, mask)
            plan.sparse_gather_reduce(rd, mask, True, None, wd, vd, wl.lr, wl.mu)
        return state

    init = (plan.empty_residual(), to_dev(workloads.weights(wl)), torch.zeros(wl.P, device="cuda"))
    straight = steps(tuple(t.clone() for t in init), (1, 2, 3))
    ck = steps(tuple(t.clone() for t in init), (1, 2))
    saved = tuple(host(t).copy() for t in ck)                  # checkpoint to host memory
    resumed = steps(tuple(to_dev(a) for a in saved), (3,))
    torch.cuda.synchronize()
    for a, b2 in zip(straight, resumed):
        assert np.array_equal(host(a), host(b2))


def test_sparse_maximum_chunk_count(ga):
    """n_c at the library's limit (65536 chunks of 8 elements, the last one
    ragged), with the top-k selecting 6554 of them per worker."""
    n_c = ga.MAX_CHUNKS
    wl = workloads.custom(2, [8 * (n_c - 1) + 5], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=8, rho=0.1)
    res = run_sparse(ga, wl, steps=2, lazy=True)
    assert res.keys.shape == (2, n_c)


def test_sparse_maximum_worker_count(ga):
    """W at the library's limit (1024 workers): eleven tree levels."""
    wl = workloads.custom(ga.MAX_WORKERS, [3000, 77], True, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=256, rho=0.25)
    run_sparse(ga, wl, steps=2, lazy=True)


def test_sparse_both_limits(ga):
    """W and n_c both at the library's limits (1024 workers x 65536 chunks of
    8 elements, the last one ragged): 2^26 (worker, chunk) pairs, more
    workgroups than a 1-D grid of 256-thread groups can address.  One step
    (the oracle takes about half a minute for it)."""
    n_c = ga.MAX_CHUNKS
    wl = workloads.custom(ga.MAX_WORKERS, [8 * (n_c - 1) + 5], True, sigma=1e-3, scale_mode="chunk",
                          scale_log10=(-4.0, 0.0), chunk=8, rho=0.1)
    print("W=%d n_c=%d P=%d" % (wl.W, n_c, wl.P), flush=True)
    res = run_sparse(ga, wl, steps=1, lazy=False)
    assert res.keys.shape == (ga.MAX_WORKERS, n_c)
