"""Shared helpers for the GPU parity tests: moving numpy inputs to the device
and comparing results with the oracle's to the stated tolerances."""
import numpy as np

# Tolerances for floating-point results (max elementwise relative error, with
# the denominator floored at the smallest normal binary32).  Both sides perform
# the same binary32 operations in the same order, so the observed error is 0.
TOL_FP32 = 1e-6
TOL_FP16_PATH = 2e-3
KEY_RTOL = 1e-12          # binary64 chunk keys: summation order differs


def to_dev(a: np.ndarray, fp16: bool = False):
    import torch
    if fp16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN positions differ"
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)]), "infinities differ"
    if not fin.any():
        return 0.0
    den = np.maximum(np.abs(ref[fin]), np.finfo(np.float32).tiny)
    return float(np.max(np.abs(got[fin] - ref[fin]) / den))


def assert_close(got, ref, tol, name=""):
    err = max_rel(got, ref)
    assert err <= tol, "%s: max relative error %.3g > %.3g" % (name, err, tol)
    return err


def assert_same_bits(got, ref, name=""):
    """Bitwise equality, with +0 and -0 taken as equal and NaNs matched by position."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), name + ": NaN positions differ"
    same = (got == ref) | nan
    if not same.all():
        i = int(np.flatnonzero(~same.ravel())[0])
        raise AssertionError("%s: %d mismatches, first at %d: %r vs %r" % (
            name, int((~same).sum()), i, got.ravel()[i], ref.ravel()[i]))
