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


def device_layers(rows: np.ndarray, numels, misalign=lambda w, l: 0):
    """Copy each worker's gradient row, split into layers of `numels` elements,
    into separate places of one device buffer, layer (w, l) starting
    misalign(w, l) elements past a 16-byte boundary with gaps between layers.
    Returns (buffer, int64 tensor of the W*L layer addresses, worker-major)."""
    import torch
    W = rows.shape[0]
    isz = rows.dtype.itemsize
    ti = {2: torch.int16, 4: torch.int32}[isz]
    ni = {2: np.int16, 4: np.int32}[isz]
    pad = 16 // isz
    total = sum(n + 3 * pad for n in numels) * W
    buf = torch.zeros(total, dtype=ti, device="cuda")
    offs = np.cumsum([0] + list(numels))
    ptrs, off = [], 0
    for w in range(W):
        for l, n in enumerate(numels):
            s = off + misalign(w, l) % pad
            src = np.ascontiguousarray(rows[w, offs[l]:offs[l + 1]]).view(ni)
            buf[s:s + n].copy_(torch.from_numpy(src))
            ptrs.append(buf.data_ptr() + s * isz)
            off += n + 2 * pad
            off += (-off) % pad
    return buf, torch.tensor(ptrs, dtype=torch.int64, device="cuda")
