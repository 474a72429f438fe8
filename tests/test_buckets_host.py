"""Multi-bucket lazy allreduce schedule on the host: the rule that cuts the
layer list into buckets (GradientFlow, arXiv abstract: lazy allreduce fuses
many communication operations; computation and communication overlap).  The
rule is stated in include/gradagg.h at ga_bucket_boundaries; this file checks
the library against a plain statement of it and against the properties any
bucket schedule of a backward pass must have.  No kernel is launched."""
import os

import numpy as np
import pytest

import workloads


@pytest.fixture(scope="module")
def ga():
    import gradient_aggregation_amd as ga
    if not os.path.exists(ga.LIB_PATH):
        from gradient_aggregation_amd import build
        build.build()
    return ga


def greedy(numels, esz, threshold):
    """Walk from the last layer down; close at an 8-aligned layer start once
    the bucket holds >= threshold bytes; layer 0 closes the last bucket."""
    offs = np.concatenate([[0], np.cumsum(numels)])
    firsts, acc = [], 0
    for l in range(len(numels) - 1, -1, -1):
        acc += numels[l] * esz
        if l == 0 or (acc >= threshold and offs[l] % 8 == 0):
            firsts.append(l)
            acc = 0
    return firsts


def check_properties(numels, esz, threshold, firsts):
    L = len(numels)
    offs = np.concatenate([[0], np.cumsum(numels)])
    assert firsts[-1] == 0
    assert all(a > b for a, b in zip(firsts, firsts[1:])), "buckets run from the last layer down"
    ends = [L] + firsts[:-1]
    covered = []
    for f, e in zip(firsts, ends):
        covered.extend(range(f, e))
        assert offs[f] % 8 == 0, "bucket start not 8-aligned"
        nbytes = int(offs[e] - offs[f]) * esz
        if f != 0:
            assert nbytes >= threshold, "a bucket other than the last is below the threshold"
    assert sorted(covered) == list(range(L)), "every layer in exactly one bucket"


@pytest.mark.parametrize("fp16", [False, True])
@pytest.mark.parametrize("threshold", [1, 64, 4096, 1 << 20, 25 << 20, 1 << 40])
@pytest.mark.parametrize("name", ["tiny", "nin", "googlenet", "alexnet16"])
def test_workload_schedules(ga, name, fp16, threshold):
    numels = workloads.WORKLOADS[name].numels
    esz = 2 if fp16 else 4
    firsts = ga.bucket_boundaries(numels, fp16, threshold)
    assert firsts == greedy(numels, esz, threshold)
    check_properties(numels, esz, threshold, firsts)
    if threshold >= 1 << 40:
        assert firsts == [0]


def test_random_layer_lists(ga):
    rng = np.random.default_rng(7)
    for _ in range(300):
        L = int(rng.integers(1, 40))
        numels = [int(x) for x in rng.integers(1, 3000, L)]
        if rng.random() < 0.5:
            numels = [8 * ((n + 7) // 8) for n in numels]
        fp16 = bool(rng.random() < 0.5)
        thr = int(rng.integers(1, 20000))
        firsts = ga.bucket_boundaries(numels, fp16, thr)
        assert firsts == greedy(numels, 2 if fp16 else 4, thr)
        check_properties(numels, 2 if fp16 else 4, thr, firsts)


def test_one_layer_per_bucket_when_aligned(ga):
    numels = [8, 16, 24, 800]
    assert ga.bucket_boundaries(numels, False, 1) == [3, 2, 1, 0]


def test_unaligned_starts_merge(ga):
    # offsets 0, 3, 10, 17: no start but 0 is a multiple of 8, one bucket
    assert ga.bucket_boundaries([3, 7, 7, 40], False, 1) == [0]


@pytest.mark.parametrize("args", [(0, [1], 4, 1), (2, [1, 0], 4, 1), (1, [5], 3, 1), (1, [5], 4, 0)])
def test_invalid_arguments(ga, args):
    import ctypes
    n, numels, esz, thr = args
    arr = (ctypes.c_int64 * max(len(numels), 1))(*numels)
    first = (ctypes.c_int32 * 4)()
    nb = ctypes.c_int32(0)
    st = ga.lib().ga_bucket_boundaries(n, arr, esz, thr, first, ctypes.byref(nb))
    assert st == ga.GA_ERR_INVALID
    assert ga.lib().ga_last_error().decode()


def test_null_schedule_calls(ga):
    assert ga.lib().ga_buckets_count(None) == 0
    ga.lib().ga_buckets_destroy(None)
    assert ga.lib().ga_bucket_range(None, 0, None, None, None, None) == ga.GA_ERR_INVALID
    assert ga.lib().ga_bucket_reduce_layers(None, 0, None, None, None, None, None, None, 0, None) == ga.GA_ERR_INVALID
