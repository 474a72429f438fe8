"""The dense step split across G groups of W/G consecutive workers, as G GPUs
would run it: every group's unscaled tree sum (ga_tree_partial), a
reduce-scatter emulated by copying each owner's slice of the G partials into
a [G][ld] buffer, and the owner's tree over the partials with the mean over
all W workers and SGD (ga_tree_combine).  Bit for bit against the one-launch
tree over all W workers and against the oracle's dense step."""
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


def split_step(ga, bd, W, G, numels, fp16, P, w0, lr, mu):
    """ḡ, w, v of the split step; bd: the [W][ld] bucket on the device."""
    m = W // G
    grp = ga.Plan(m, numels, fp16)
    sums = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(G)]
    for j in range(G):
        print("group %d of %d: workers %d..%d" % (j, G, j * m, (j + 1) * m - 1), flush=True)
        grp.tree_partial(bd[j * m:(j + 1) * m], sums[j])
    # ownership: G slices of Q elements (a multiple of 64, so every slice of
    # g, w and v starts 16-byte aligned); the last one ragged or empty
    Q = ((P + G - 1) // G + 63) // 64 * 64
    g = torch.full((P,), float("nan"), dtype=torch.float32, device="cuda")
    w = to_dev(w0.copy())
    v = torch.zeros(P, dtype=torch.float32, device="cuda")
    for k in range(G):
        lo, hi = k * Q, min(P, (k + 1) * Q)
        if lo >= hi:
            continue
        own = ga.Plan(G, [hi - lo], False)
        part = torch.zeros((G, own.ld), dtype=torch.float32, device="cuda")
        for j in range(G):
            part[j, :hi - lo] = sums[j][lo:hi]
        own.tree_combine(part, W, g[lo:hi], w[lo:hi], v[lo:hi], lr, mu)
        own.close()
    grp.close()
    torch.cuda.synchronize()
    return host(g), host(w), host(v)


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,G", [(2, 2), (8, 2), (8, 8), (16, 4), (6, 3), (12, 3), (128, 8), (256, 2), (320, 5)])
def test_split_step_equals_one_gpu(ga, fp16, W, G):
    m = W // G
    assert m * G == W and m & (m - 1) == 0
    numels = [5000, 3, 12345]
    wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer")
    P = wl.P
    full = ga.Plan(W, numels, fp16)
    b = workloads.grad_bucket(wl, 1, full.ld)
    w0 = workloads.weights(wl)
    bd = to_dev(b, fp16)
    # one launch over all W workers
    g1 = torch.empty(P, dtype=torch.float32, device="cuda")
    w1, v1 = to_dev(w0.copy()), torch.zeros(P, dtype=torch.float32, device="cuda")
    full.tree_reduce(bd, g1, w1, v1, wl.lr, wl.mu)
    torch.cuda.synchronize()
    # the oracle
    w_ref, v_ref = w0.copy(), np.zeros(P, np.float32)
    g_ref = oracle.dense_step(b, P, fp16, wl.lr, wl.mu, w_ref, v_ref)
    g2, w2, v2 = split_step(ga, bd, W, G, numels, fp16, P, w0, wl.lr, wl.mu)
    assert_same_bits(g2, host(g1), "gbar (split vs one launch)")
    assert_same_bits(w2, host(w1), "w (split vs one launch)")
    assert_same_bits(v2, host(v1), "v (split vs one launch)")
    assert_same_bits(g2, g_ref, "gbar (split vs oracle)")
    assert_same_bits(w2, w_ref, "w (split vs oracle)")
    assert_same_bits(v2, v_ref, "v (split vs oracle)")
    full.close()


def test_partial_is_the_unscaled_tree_sum(ga):
    """ga_tree_partial = the oracle's tree sum (W=5, a non-power-of-two tree),
    binary16 leaves, -0 and subnormal leaves kept bit for bit."""
    W, numels = 5, [777, 64]
    wl = workloads.custom(W, numels, True, sigma=1e-2)
    plan = ga.Plan(W, numels, True)
    b = workloads.grad_bucket(wl, 1, plan.ld)
    b[:, 0] = 0x8000            # every leaf -0: the sum is -0
    b[:, 1] = 0x0001            # smallest subnormal
    b[0, 2] = 0x8000
    out = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    plan.tree_partial(to_dev(b, True), out)
    torch.cuda.synchronize()
    ref = oracle.tree_sum(oracle.f16_decode(b[:, :wl.P]))
    got = host(out)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "S differs (bits, sign of zero included)"
    assert np.signbit(got[0]) and got[1] == np.float32(5 * 2.0 ** -24)
    plan.close()


def test_combine_rejects_bad_arguments(ga):
    own16 = ga.Plan(2, [100], True)
    part = torch.zeros((2, own16.ld), dtype=torch.float32, device="cuda")
    g = torch.empty(100, dtype=torch.float32, device="cuda")
    with pytest.raises(ga.GAError) as e:
        own16.tree_combine(part, 2, g)
    assert e.value.status == ga.GA_ERR_INVALID
    own = ga.Plan(2, [100], False)
    with pytest.raises(ga.GAError) as e:
        own.tree_combine(part, 0, g)
    assert e.value.status == ga.GA_ERR_INVALID
    with pytest.raises(ga.GAError) as e:
        own.tree_combine(part, 2)
    assert e.value.status == ga.GA_ERR_INVALID
    own.close()
    own16.close()
