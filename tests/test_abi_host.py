"""The C-ABI library on the host: it loads, exports every declared function,
and its plan arithmetic and argument validation behave as declared.  No kernel
is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gradagg.h")


@pytest.fixture(scope="module")
def ga():
    import gradient_aggregation_amd as ga
    if not os.path.exists(ga.LIB_PATH):
        from gradient_aggregation_amd import build
        build.build()
    return ga


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ga_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(ga):
    names = _declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(ga.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert ga.lib().ga_abi_version() == 4


def test_status_strings(ga):
    for s, n in enumerate(["GA_OK", "GA_ERR_INVALID", "GA_ERR_ALIGN", "GA_ERR_DEVICE", "GA_ERR_UNSUPPORTED"]):
        assert ga.status_name(s) == n


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_plan_sizes_match_formulas(ga, name):
    wl = workloads.WORKLOADS[name]
    info = ga.compute_info(wl.W, wl.numels, wl.fp16, wl.chunk, wl.rho)
    assert info.P == wl.P and info.W == wl.W and info.n_layers == len(wl.layers)
    assert info.ld == (wl.P + 63) // 64 * 64
    if wl.chunk:
        n_c = (wl.P + wl.chunk - 1) // wl.chunk
        assert info.n_chunks == n_c and info.k == oracle.keep_count(n_c, wl.rho)
        assert info.mask_words == (n_c + 31) // 32
    if name == "alexnet128_sparse":
        assert (info.n_chunks, info.k, info.mask_words) == (1861, 187, 59)


def test_keep_count_agrees_with_oracle(ga):
    rng = np.random.default_rng(0)
    for _ in range(300):
        P = int(rng.integers(8, 200000))
        C = int(rng.integers(1, 64)) * 8
        rho = float(rng.random()) if rng.random() < 0.8 else float(rng.integers(0, 11)) / 10
        info = ga.compute_info(3, [P], True, C, rho)
        assert info.k == oracle.keep_count(info.n_chunks, rho)


@pytest.mark.parametrize("args,status", [
    (dict(W=0), 1), (dict(W=1025), 1), (dict(numels=[]), 1), (dict(numels=[5, 0]), 1),
    (dict(chunk=-8), 1), (dict(rho=-0.1), 1), (dict(rho=1.5), 1), (dict(rho=float("nan")), 1),
    (dict(chunk=12), 4), (dict(chunk=8, numels=[8 * 70000]), 4),
])
def test_plan_validation(ga, args, status):
    a = dict(W=4, numels=[100, 28], fp16=False, chunk=64, rho=0.5)
    a.update(args)
    with pytest.raises(ga.GAError) as e:
        ga.compute_info(a["W"], a["numels"], a["fp16"], a["chunk"], a["rho"])
    assert e.value.status == status
    assert ga.lib().ga_last_error().decode()


def test_calls_reject_null_plan_without_launching(ga):
    L = ga.lib()
    assert L.ga_tree_reduce(None, None, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_chunk_norm(None, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_chunk_topk(None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_sparse_gather_reduce(None, None, None, 1, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_bucket_pack(None, None, None, None) == ga.GA_ERR_INVALID
    h = ga.History()
    assert L.ga_chunk_norm_deferred(None, None, None, 0, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_sparse_gather_reduce_deferred(None, None, None, 0, None, None, None, None, None, None,
                                              None) == ga.GA_ERR_INVALID
    assert L.ga_residual_flush(None, None, None, 0, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_chunk_norm_deferred(None, 8, ctypes.byref(h), 0, 16, 8, None) == ga.GA_ERR_INVALID
    assert L.ga_reduce_variant(None, None, 0, 0, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_tree_reduce_layers(None, None, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_chunk_norm_layers(None, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_tree_partial(None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_tree_combine(None, None, 1, None, None, None, None, None) == ga.GA_ERR_INVALID
    assert L.ga_sgd_momentum_apply(-1, None, None, None, None, None) == ga.GA_ERR_INVALID
    s = ga.SGD(0.01, 0.9)
    assert L.ga_sgd_momentum_apply(0, None, None, None, ctypes.byref(s), None) == ga.GA_OK
    assert L.ga_sgd_momentum_apply(16, 8, 16, 32, ctypes.byref(s), None) == ga.GA_ERR_ALIGN


def test_history_struct_matches_header(ga):
    """The binding's ga_history has the header's layout (age, GA_MAX_AGE + 1
    mask pointers, GA_MAX_AGE layer-table pointers)."""
    src = open(HEADER).read()
    m = re.search(r"#define GA_MAX_AGE (\d+)", src)
    assert m and int(m.group(1)) == ga.MAX_AGE
    assert ctypes.sizeof(ga.History) == 8 + 8 * (2 * ga.MAX_AGE + 1)
    assert ga.History.d_masks.offset == 8 and ga.History.d_layer_ptrs.offset == 8 + 8 * (ga.MAX_AGE + 1)


def test_product_path_has_no_cpu_fallback(ga):
    """The binding refuses to run without a GPU instead of computing on the host."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    with pytest.raises(RuntimeError):
        ga.Plan(4, [100], False)


def test_library_does_not_link_the_oracle(ga):
    """The product package never refers to the oracle or the input generator."""
    src_dir = os.path.join(ROOT, "gradient_aggregation_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read().lower()
                assert "oracle" not in text and "workloads" not in text, f
    out = os.popen("ldd %s" % ga.LIB_PATH).read()
    assert "oracle" not in out and "gagen" not in out


def test_size_limits_are_inclusive(ga):
    info = ga.compute_info(ga.MAX_WORKERS, [8 * ga.MAX_CHUNKS], True, 8, 0.1)
    assert info.n_chunks == ga.MAX_CHUNKS and info.W == ga.MAX_WORKERS
    with pytest.raises(ga.GAError) as e:
        ga.compute_info(2, [8 * ga.MAX_CHUNKS + 1], True, 8, 0.1)
    assert e.value.status == ga.GA_ERR_UNSUPPORTED


def test_element_limit(ga):
    """P up to GA_MAX_ELEMENTS per worker (summed over layers), not one more;
    the standalone SGD call has the same limit and checks it before any
    pointer."""
    half = ga.MAX_ELEMENTS // 2
    info = ga.compute_info(ga.MAX_WORKERS, [half, half], False, 0, 0.0)
    assert info.P == ga.MAX_ELEMENTS
    for numels in ([ga.MAX_ELEMENTS + 1], [half, half, 1]):
        with pytest.raises(ga.GAError) as e:
            ga.compute_info(2, numels, True, 0, 0.0)
        assert e.value.status == ga.GA_ERR_UNSUPPORTED
    L = ga.lib()
    s = ga.SGD(0.01, 0.9)
    assert L.ga_sgd_momentum_apply(ga.MAX_ELEMENTS + 1, 16, 16, 16, ctypes.byref(s), None) == ga.GA_ERR_UNSUPPORTED


def test_header_is_plain_c_and_client_links(ga):
    """include/gradagg.h compiles as C11 with gcc and a C program links against
    the library (the client itself runs in the GPU tests)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_build", os.path.join(ROOT, "tests", "c", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build()
    assert os.path.exists(exe)
