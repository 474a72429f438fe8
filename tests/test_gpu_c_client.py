"""The C ABI driven from plain C (tests/c/abi_client.c: gcc, libamdhip64, no
Python or torch in the process): all five calls of the path - the fusion of
per-layer tensors into a bucket, the dense tree reduce, the chunk norms with
top-k, the sparse gather-reduce and the standalone momentum-SGD update - on
device buffers the client allocates, compared with the oracle element by
element."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from helpers import KEY_RTOL, assert_close, assert_same_bits

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def client():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = os.path.join(HERE, "c", "abi_client")
    if not os.path.exists(exe):
        import importlib.util
        spec = importlib.util.spec_from_file_location("c_build", os.path.join(HERE, "c", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return exe


def run_client(exe, tmp_path, wl, steps):
    info_ld = (wl.P + 63) // 64 * 64
    with open(tmp_path / "meta.txt", "w") as f:
        f.write("%d %d %d %d %.17g %.9g %.9g %d\n" % (wl.W, len(wl.numels), int(wl.fp16), wl.chunk, wl.rho, wl.lr,
                                                      wl.mu, steps))
        f.write(" ".join(str(n) for n in wl.numels) + "\n")
    buckets = []
    for s in range(1, steps + 1):
        b = workloads.grad_bucket(wl, s, info_ld)
        b.tofile(tmp_path / ("bucket%d.bin" % s))
        buckets.append(b)
    w0 = workloads.weights(wl)
    w0.tofile(tmp_path / "w.bin")
    print("[c-client] W=%d P=%d fp16=%s chunk=%d steps=%d" % (wl.W, wl.P, wl.fp16, wl.chunk, steps), flush=True)
    out = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    return buckets, w0, info_ld


def load(tmp_path, name, dtype):
    return np.fromfile(tmp_path / name, dtype=dtype)


def check_pack_and_sgd(tmp_path, wl, ld, bucket1, gbar, w, v):
    """pack.bin is the oracle's fusion of step 1's per-layer tensors (byte
    for byte, zero padding); w_sgd/v_sgd are one more oracle update of the
    final state with the final mean gradient."""
    offs = np.cumsum([0] + list(wl.numels))
    layers = [[bucket1[r, offs[l]:offs[l + 1]] for l in range(len(wl.numels))] for r in range(wl.W)]
    ref = oracle.pack(layers, ld)
    got = load(tmp_path, "pack.bin", ref.dtype).reshape(wl.W, ld)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), "packed bucket differs"
    w2, v2 = w.copy(), v.copy()
    oracle.sgd(gbar, w2, v2, wl.lr, wl.mu)
    assert_same_bits(load(tmp_path, "w_sgd.bin", np.float32), w2, "standalone SGD w")
    assert_same_bits(load(tmp_path, "v_sgd.bin", np.float32), v2, "standalone SGD v")


@pytest.mark.parametrize("fp16", [False, True])
def test_c_client_dense(client, tmp_path, fp16):
    wl = workloads.custom(5, [1000, 37, 4099], fp16, sigma=1e-2, scale_mode="layer")
    buckets, w0, ld = run_client(client, tmp_path, wl, steps=2)
    w, v = w0.copy(), np.zeros(wl.P, np.float32)
    for b in buckets:
        g = oracle.dense_step(b, wl.P, fp16, wl.lr, wl.mu, w, v)
    assert_same_bits(load(tmp_path, "gbar.bin", np.float32), g, "gbar")
    assert_same_bits(load(tmp_path, "w_out.bin", np.float32), w, "w")
    assert_same_bits(load(tmp_path, "v_out.bin", np.float32), v, "v")
    check_pack_and_sgd(tmp_path, wl, ld, buckets[0], g, w, v)


def test_c_client_sparse(client, tmp_path):
    wl = workloads.custom(4, [3000, 17, 1000], True, sigma=1e-3, scale_mode="chunk", scale_log10=(-4.0, 0.0),
                          chunk=64, rho=0.25)
    buckets, w0, ld = run_client(client, tmp_path, wl, steps=3)
    n_c = (wl.P + wl.chunk - 1) // wl.chunk
    k = oracle.keep_count(n_c, wl.rho)
    w, v = w0.copy(), np.zeros(wl.P, np.float32)
    r = np.zeros((wl.W, ld), np.float32)
    for b in buckets:
        res = oracle.sparse_step(b, wl.P, True, wl.chunk, k, r, wl.lr, wl.mu, w, v)
    assert np.all(res.margin > 1e-12)
    assert np.array_equal(load(tmp_path, "idx.bin", np.int32).reshape(wl.W, k), res.sel_idx)
    assert np.array_equal(load(tmp_path, "mask.bin", np.uint32).reshape(wl.W, -1), res.sel_mask)
    assert_close(load(tmp_path, "keys.bin", np.float64).reshape(wl.W, n_c), res.keys, KEY_RTOL, "keys")
    assert_same_bits(load(tmp_path, "resid.bin", np.float32).reshape(wl.W, ld)[:, :wl.P], r[:, :wl.P], "residual")
    assert_same_bits(load(tmp_path, "gbar.bin", np.float32), res.gbar, "gbar")
    assert_same_bits(load(tmp_path, "w_out.bin", np.float32), w, "w")
    assert_same_bits(load(tmp_path, "v_out.bin", np.float32), v, "v")
    check_pack_and_sgd(tmp_path, wl, ld, buckets[0], res.gbar, w, v)
