"""GPU parity of zero-copy fusion: the dense tree reduce and the chunk norms
reading every worker's per-layer tensors through the layer table, against the
oracle run on the fused (concatenated) gradients."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, assert_close, assert_same_bits, device_layers, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MIS = {"aligned": lambda w, l: 0, "unaligned": lambda w, l: 1 + l, "mixed": lambda w, l: (3 * w + l) % 4}


@pytest.fixture(scope="module")
def ga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gradient_aggregation_amd as ga
    return ga


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("W,numels", [(1, [3]), (3, workloads.WORKLOADS["tiny"].numels),
                                      (16, [8, 1, 5000, 7, 4096, 333]), (63, [4096, 1, 515]), (64, [777, 4096, 9]),
                                      (128, [2048, 10, 4099])])
@pytest.mark.parametrize("mis", list(MIS))
def test_tree_reduce_layers(ga, fp16, W, numels, mis):
    wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer")
    plan = ga.Plan(W, numels, fp16)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    gd = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    for step in (1, 2):
        b = workloads.grad_bucket(wl, step, plan.ld)
        buf, ptrs = device_layers(b[:, :wl.P], numels, MIS[mis])
        g_ref = oracle.dense_step(b, wl.P, fp16, wl.lr, wl.mu, w_ref, v_ref)
        plan.tree_reduce_layers(ptrs, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        assert_same_bits(host(gd), g_ref, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        assert_same_bits(host(vd), v_ref, "v")


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("C,numels", [(64, workloads.WORKLOADS["tiny"].numels), (256, [1000, 17, 3000, 8, 40]),
                                      (8, [5, 11, 100]),
                                      # chunks split into 2048-element norm parts: the last
                                      # chunk's second part empty; a ragged third part
                                      (2304, [5000, 3, 9000, 250]), (6144, [20000, 37, 4003])])
@pytest.mark.parametrize("mis", list(MIS))
@pytest.mark.parametrize("lazy", [False, True])
def test_chunk_norm_layers(ga, fp16, C, numels, mis, lazy):
    W = 5
    wl = workloads.custom(W, numels, fp16, sigma=1e-2, scale_mode="layer", chunk=C, rho=0.25)
    plan = ga.Plan(W, numels, fp16, chunk=C, keep_ratio=0.25)
    k = plan.k
    r_ref = np.zeros((W, plan.ld), np.float32)
    w_ref = workloads.weights(wl)
    v_ref = np.zeros(wl.P, np.float32)
    wd, vd = to_dev(w_ref.copy()), to_dev(v_ref.copy())
    rd, keys = plan.empty_residual(), plan.empty_keys()
    idx = torch.empty((W, max(k, 1)), dtype=torch.int32, device="cuda")
    masks = [torch.zeros((W, plan.mask_words), dtype=torch.int32, device="cuda") for _ in range(2)]
    gd = torch.empty(wl.P, dtype=torch.float32, device="cuda")
    for step in (1, 2, 3):
        b = workloads.grad_bucket(wl, step, plan.ld)
        buf, ptrs = device_layers(b[:, :wl.P], numels, MIS[mis])
        res = oracle.sparse_step(b, wl.P, fp16, C, k, r_ref, wl.lr, wl.mu, w_ref, v_ref)
        cur, prev = masks[step % 2], masks[(step + 1) % 2]
        plan.chunk_norm_layers(ptrs, rd, keys, prev if (lazy and step > 1) else None)
        plan.chunk_topk(keys, idx, cur)
        plan.sparse_gather_reduce(rd, cur, not lazy, gd, wd, vd, wl.lr, wl.mu)
        torch.cuda.synchronize()
        assert np.all(res.margin > 1e-12)
        assert_close(host(keys), res.keys, KEY_RTOL, "keys")
        assert np.array_equal(host(idx)[:, :k], res.sel_idx)
        assert_same_bits(host(gd), res.gbar, "gbar")
        assert_same_bits(host(wd), w_ref, "w")
        r_got = host(rd)
        if lazy:
            m = host(cur).view(np.uint32)
            n_c = plan.n_chunks
            for w in range(W):
                for c in range(n_c):
                    if (int(m[w, c >> 5]) >> (c & 31)) & 1:
                        r_got[w, c * C:min((c + 1) * C, wl.P)] = 0.0
        assert_same_bits(r_got[:, :wl.P], r_ref[:, :wl.P], "residual")


def test_layers_equal_bucket_path_alexnet_shape(ga):
    """Same layer list as the benchmark (16 AlexNet tensors, W=8): the layer
    table and the packed bucket give bitwise identical keys and sums."""
    wl = workloads.custom(8, workloads.WORKLOADS["alexnet16"].numels, True, sigma=1e-3, chunk=32768, rho=0.1)
    plan = ga.Plan(wl.W, wl.numels, True, chunk=32768, keep_ratio=0.1)
    b = workloads.grad_bucket(wl, 1, plan.ld)
    buf, ptrs = device_layers(b[:, :wl.P], wl.numels)
    bd = to_dev(b, True)
    r1, r2 = plan.empty_residual(), plan.empty_residual()
    k1, k2 = plan.empty_keys(), plan.empty_keys()
    plan.chunk_norm(bd, r1, k1)
    plan.chunk_norm_layers(ptrs, r2, k2)
    g1 = torch.empty(wl.P, device="cuda")
    g2 = torch.empty(wl.P, device="cuda")
    plan.tree_reduce(bd, g1)
    plan.tree_reduce_layers(ptrs, g2)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2) and torch.equal(k1, k2) and torch.equal(g1, g2)
