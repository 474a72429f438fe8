"""ga_chunk_norm_topk_static, the entry point that allocates nothing (its
binary64 keys, and the partial sums of chunks longer than 2048 elements, live
in a fixed array inside the library), called through the C ABI and checked
against ga_chunk_norm_topk with a caller key buffer, bit for bit: on two calls
in a row, the second with a smaller plan (so the array holds
the first call's keys when it starts), in plain and lazy-zero mode, and
against the oracle.  Oversized plans are refused before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_same_bits, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_both(ga, wl, steps):
    """`steps` lazy-zero steps of chunk norms + top-k through both entry points
    on two copies of the same residual, plus the oracle on the host."""
    L = ga.lib()
    plan = ga.Plan(wl.W, wl.numels, wl.fp16, chunk=wl.chunk, keep_ratio=wl.rho)
    W, P, ld, k, mw = wl.W, wl.P, plan.ld, plan.k, plan.mask_words
    r_a, r_b = plan.empty_residual(), plan.empty_residual()
    keys = plan.empty_keys()
    idx_a = torch.full((W, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    idx_b = idx_a.clone()
    m_a = [torch.zeros((W, mw), dtype=torch.int32, device="cuda") for _ in range(2)]
    m_b = [torch.zeros((W, mw), dtype=torch.int32, device="cuda") for _ in range(2)]
    r_ref = np.zeros((W, ld), np.float32)
    w_ref, v_ref = workloads.weights(wl), np.zeros(P, np.float32)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for t in range(1, steps + 1):
        b = workloads.grad_bucket(wl, t, ld)
        res = oracle.sparse_step(b, P, wl.fp16, wl.chunk, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        bd = to_dev(b, wl.fp16)
        cur, prev = t % 2, (t + 1) % 2
        pa = m_a[prev] if t > 1 else None
        pb = m_b[prev] if t > 1 else None
        st = L.ga_chunk_norm_topk(plan._h, _ptr(bd), _ptr(r_a), _ptr(pa), _ptr(keys), _ptr(idx_a), _ptr(m_a[cur]),
                                  stream)
        assert st == ga.GA_OK, ga.lib().ga_last_error()
        st = L.ga_chunk_norm_topk_static(plan._h, _ptr(bd), _ptr(r_b), _ptr(pb), _ptr(idx_b), _ptr(m_b[cur]),
                                         stream)
        assert st == ga.GA_OK, ga.lib().ga_last_error()
        # the gather of the lazy-zero step leaves the residual as is: only the
        # masks carry the zeroing to the next norm pass
        torch.cuda.synchronize()
        assert np.array_equal(host(idx_b), host(idx_a)), "step %d: selected indices differ" % t
        assert np.array_equal(host(m_b[cur]), host(m_a[cur])), "step %d: masks differ" % t
        assert np.array_equal(host(r_b).view(np.uint32), host(r_a).view(np.uint32)), "step %d: residual" % t
        if wl.rho not in (0.0, 1.0):
            assert np.all(res.margin > 1e-12)
        if k > 0:
            assert np.array_equal(host(idx_b)[:, :k], res.sel_idx), "step %d: selection vs oracle" % t
        assert np.array_equal(host(m_b[cur]).view(np.uint32), res.sel_mask)
        # the oracle zeroes what was sent; the lazy buffer reads those chunks as zero
        m = host(m_b[cur]).view(np.uint32).astype(np.int64)
        ch = np.arange(plan.n_chunks)
        sent = np.repeat(((m[:, ch >> 5] >> (ch & 31)) & 1).astype(bool), wl.chunk, axis=1)[:, :P]
        r_got = host(r_b)[:, :P].copy()
        r_got[sent] = 0.0
        assert_same_bits(r_got, r_ref[:, :P], "step %d: residual vs oracle" % t)
    plan.close()


def test_static_keys_two_calls_second_smaller(ga):
    big = workloads.custom(48, [20000, 37, 4003, 9000], True, sigma=1e-3, scale_mode="chunk",
                           scale_log10=(-4.0, 0.0), chunk=256, rho=0.15)
    small = workloads.custom(5, [3000, 11], False, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                             chunk=64, rho=0.3)
    run_both(ga, big, steps=3)
    run_both(ga, small, steps=3)


def test_static_keys_long_chunks(ga):
    """Chunks longer than 2048 elements: the norm pass sums 2048-element parts
    into the fixed array (after the keys), then adds them into the keys; the
    caller-buffer call does the same in the plan's workspace."""
    wl = workloads.custom(9, [20000, 37, 4003], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=4352, rho=0.3)
    run_both(ga, wl, steps=3)


def _limit_case(ga, W, chunk, n_c, status):
    L = ga.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    plan = ga.Plan(W, [chunk * n_c], True, chunk=chunk, keep_ratio=0.01)
    assert plan.n_chunks == n_c
    print("[no-alloc limit] W=%d C=%d n_c=%d expect %d" % (W, chunk, n_c, status), flush=True)
    if status == ga.GA_OK:
        bd = torch.zeros((W, plan.ld), dtype=torch.float16, device="cuda")
        rd = plan.empty_residual()
    else:
        # refused before any launch: nothing is read through these pointers
        bd = torch.zeros(8, dtype=torch.float16, device="cuda")
        rd = torch.zeros(8, dtype=torch.float32, device="cuda")
    idx = torch.zeros((W, plan.k), dtype=torch.int32, device="cuda")
    mask = torch.zeros((W, plan.mask_words), dtype=torch.int32, device="cuda")
    st = L.ga_chunk_norm_topk_static(plan._h, _ptr(bd), _ptr(rd), None, _ptr(idx), _ptr(mask), stream)
    assert st == status, (W, chunk, n_c, L.ga_last_error())
    torch.cuda.synchronize()
    if status == ga.GA_OK:
        # all-zero keys: the k lowest chunk indices in every row
        assert np.array_equal(host(idx), np.tile(np.arange(plan.k, dtype=np.int32), (W, 1)))
    del bd, rd
    plan.close()


def test_static_keys_limit(ga):
    """A workspace beyond the fixed array is refused before any launch; at the
    limit it runs: W * n_c keys for chunks of at most 2048 elements,
    W * n_c * (1 + parts) values for longer ones (here 2 parts of a
    2056-element chunk: the partial sums end 1024 values short of the array's
    end)."""
    W = 1024
    n_c = ga.STATIC_KEYS // W
    _limit_case(ga, W, 8, n_c + 1, ga.GA_ERR_UNSUPPORTED)
    _limit_case(ga, W, 8, n_c, ga.GA_OK)
    n_c = ga.STATIC_KEYS // (W * 3)
    _limit_case(ga, W, 2056, n_c + 1, ga.GA_ERR_UNSUPPORTED)
    _limit_case(ga, W, 2056, n_c, ga.GA_OK)
