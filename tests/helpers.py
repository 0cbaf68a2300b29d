"""Shared helpers for the GPU parity tests (no WKV arithmetic here)."""
import numpy as np

# Tolerance of the fp32 GPU path against the fp64 oracle: |x - r| <= RTOL * max(|r|, FLOOR),
# i.e. relative error 1e-4, with an absolute floor of 1e-5 below |r| = 0.1.
RTOL = 1e-4
FLOOR = 0.1


def max_violation(got, ref, rtol=RTOL, floor=FLOOR):
    """Largest |got - ref| / (rtol * max(|ref|, floor)); <= 1 means within tolerance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError("shape %s != %s" % (got.shape, ref.shape))
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref) / (rtol * np.maximum(np.abs(ref), floor))))


def assert_wkv_close(got, ref, what="", rtol=RTOL, floor=FLOOR):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    v = max_violation(got, ref, rtol, floor)
    if not v <= 1.0:
        err = np.abs(got - ref) / (rtol * np.maximum(np.abs(ref), floor))
        err = np.where(np.isfinite(err), err, np.inf)
        idx = np.unravel_index(int(np.argmax(err)), err.shape)
        raise AssertionError("%s: tolerance exceeded %.3gx at %s: got %r, oracle %r"
                             % (what, v, idx, float(got[idx]), float(ref[idx])))
    return v


# Spacing of the representable numbers next to x in a 16-bit output format (mantissa bits
# after the leading one; smallest normal exponent): one unit in the last place.
_FMT = {"bfloat16": (7, -126), "float16": (10, -14)}


def fmt_ulp(x, fmt):
    mant, emin = _FMT[fmt]
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** emin)))
    return 2.0 ** (e - mant)


def assert_io_close(got, ref, fmt, what="", rtol=RTOL, floor=FLOOR):
    """A 16-bit output against the fp64 oracle on the same (exactly widened) inputs: within
    the fp32 tolerance plus one unit in the last place of the format (a faithfully rounded
    result of a computation accurate to the fp32 tolerance). Returns the largest fraction of
    that allowance used."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError("shape %s != %s" % (got.shape, ref.shape))
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        raise AssertionError("%s: non-finite output" % what)
    allow = rtol * np.maximum(np.abs(ref), floor) + fmt_ulp(ref, fmt)
    r = np.abs(got - ref) / allow
    v = float(np.max(r))
    if not v <= 1.0:
        idx = np.unravel_index(int(np.argmax(r)), r.shape)
        raise AssertionError("%s: allowance exceeded %.3gx at %s: got %r, oracle %r"
                             % (what, v, idx, float(got[idx]), float(ref[idx])))
    return v
