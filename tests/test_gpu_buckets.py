"""GPU parity of the multi-bucket lazy allreduce (GradientFlow, arXiv
abstract: lazy allreduce; computation/communication overlap): reducing every
bucket of a schedule, each after its layers are ready, gives bit for bit the
oracle's dense step (FireCaffe sec. 6 tree, momentum SGD) and the one-launch
zero-copy reduction, including when a producer on another stream writes the
layers last-first while the buckets are being reduced."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_same_bits, device_layers, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MIS = {"aligned": lambda w, l: 0, "mixed": lambda w, l: (3 * w + l) % 4}


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


CASES = [
    (1, [3], 1),
    (3, workloads.WORKLOADS["tiny"].numels, 1),
    (3, workloads.WORKLOADS["tiny"].numels, 4096),
    (16, [8, 1, 5000, 7, 4096, 333, 64], 1),
    (16, [8, 1, 5000, 7, 4096, 333, 64], 10000),
    (128, [2048, 16, 4099, 520], 1),
    (5, [4104] * 6 + [1000], 1 << 40),
]


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels,threshold", CASES)
@pytest.mark.parametrize("mis", list(MIS))
@pytest.mark.parametrize("cap", [0, 3])
def test_buckets_equal_whole_reduce(ga, fp16, W, numels, threshold, mis, cap):
    wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer")
    plan = ga.Plan(W, numels, fp16)
    bk = ga.Buckets(plan, threshold)
    assert bk.count == len(ga.bucket_boundaries(numels, fp16, threshold))
    assert bk.ranges[0][0] + bk.ranges[0][1] == len(numels) and bk.ranges[-1][2] == 0
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    w1, v1 = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    g1 = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    for step in (1, 2):
        b = workloads.grad_bucket(wl, step, plan.ld)
        buf, ptrs = device_layers(b[:, :wl.P], numels, MIS[mis])
        g_ref = oracle.dense_step(b, wl.P, fp16, wl.lr, wl.mu, w_ref, v_ref)
        for i in range(bk.count):
            ev = torch.cuda.Event()
            ev.record()
            bk.reduce_layers(i, ptrs, ev, gd, wd, vd, wl.lr, wl.mu, max_workgroups=cap)
        plan.tree_reduce_layers(ptrs, g1, w1, v1, wl.lr, wl.mu)
        torch.cuda.synchronize()
        assert_same_bits(host(gd), g_ref, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")
        assert_same_bits(host(gd), host(g1), "gbar vs one launch")
        assert_same_bits(host(wd), host(w1), "w vs one launch")


@pytest.mark.parametrize("fp16", [False, True])
def test_overlapped_producer(ga, fp16):
    """A producer stream writes the layers last-first, behind a slow matmul
    per layer, and records an event when a bucket is complete; the buckets are
    reduced on another stream after their event.  A reduction that ran early
    would read the zeroed tensors."""
    W, numels = 8, [4096, 8, 2048, 1000, 8192, 520, 3000]
    wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer")
    plan = ga.Plan(W, numels, fp16)
    bk = ga.Buckets(plan, 2000 * (2 if fp16 else 4))
    assert bk.count == 4
    b = workloads.grad_bucket(wl, 1, plan.ld)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    g_ref = oracle.dense_step(b, wl.P, fp16, wl.lr, wl.mu, w_ref, v_ref)
    buf, ptrs = device_layers(b[:, :wl.P], numels)
    stage = buf.clone()
    isz = 2 if fp16 else 4
    starts = (host(ptrs) - buf.data_ptr()) // isz
    buf.zero_()
    wd, vd = to_dev(workloads.weights(wl)), to_dev(np.zeros(wl.P, np.float32))
    gd = torch.zeros(wl.P, dtype=torch.float32, device="cuda")
    a = torch.randn(1536, 1536, device="cuda")
    producer, reducer = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    bucket_of_first = {f: i for i, (f, n, e0, e1) in enumerate(bk.ranges)}
    events = []
    with torch.cuda.stream(producer):
        for l in range(len(numels) - 1, -1, -1):
            for _ in range(4):
                a = torch.tanh(a @ a * 1e-3)
            for w in range(W):
                s = int(starts[w * len(numels) + l])
                buf[s:s + numels[l]].copy_(stage[s:s + numels[l]])
            if l in bucket_of_first:
                ev = torch.cuda.Event()
                ev.record(producer)
                events.append((bucket_of_first[l], ev))
    with torch.cuda.stream(reducer):
        for i, ev in events:
            bk.reduce_layers(i, ptrs, ev, gd, wd, vd, wl.lr, wl.mu, max_workgroups=2)
    torch.cuda.synchronize()
    assert [i for i, _ in events] == list(range(bk.count))
    assert_same_bits(host(gd), g_ref, "gbar")
    assert_same_bits(host(wd), w_ref, "w")
    assert_same_bits(host(vd), v_ref, "v")


def test_bucket_errors(ga):
    plan = ga.Plan(4, [64, 64], False)
    bk = ga.Buckets(plan, 1)
    assert bk.count == 2
    ptrs = torch.zeros(8, dtype=torch.int64, device="cuda")
    g = torch.zeros(129, dtype=torch.float32, device="cuda")
    with pytest.raises(ga.GAError, match="out of range"):
        bk.reduce_layers(2, ptrs, None, g)
    with pytest.raises(ga.GAError, match="misaligned"):
        bk.reduce_layers(0, ptrs, None, g[1:])
    with pytest.raises(ga.GAError, match="neither"):
        bk.reduce_layers(0, ptrs, None)
    with pytest.raises(ga.GAError, match="max_workgroups"):
        bk.reduce_layers(0, ptrs, None, g, max_workgroups=-1)
