"""Small test-side helpers (bit handling and comparison), independent of both
the oracle and the HIP library."""
from __future__ import annotations

import numpy as np


def bf16_to_f32(a) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(a) -> np.ndarray:
    return bf16_to_f32(a).astype(np.float64)


def f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def bf16_of_exact(v: float) -> int:
    """bf16 bits of a value that is exactly representable in bf16."""
    b = f32_bits(v)
    assert b & 0xFFFF == 0, v
    return b >> 16


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 values (as float64): 2^(max(floor(log2|v|), -126) - 7)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, -126), -126)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def ulp_diff(got_bits, ref_bits) -> np.ndarray:
    """|got - ref| in units of ulp(ref), both bf16 bit arrays (finite values)."""
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    return np.abs(g - r) / bf16_ulp(r)


def check_y(got_bits, ref_bits, max_ulps=2.0, abs_tol=1e-2):
    """Normalized-output tolerance: |got - ref| <= max(max_ulps * ulp(ref), abs_tol).

    Returns (ok, max_ulp_error, n_bad, first_bad_index)."""
    g = bf16_to_f64(got_bits).ravel()
    r = bf16_to_f64(ref_bits).ravel()
    err = np.abs(g - r)
    tol = np.maximum(max_ulps * bf16_ulp(r), abs_tol)
    bad = ~(err <= tol)
    ulps = err / bf16_ulp(r)
    first = int(np.argmax(bad)) if bad.any() else -1
    return (not bad.any()), float(np.nanmax(ulps)) if ulps.size else 0.0, int(bad.sum()), first


# -- an independent nearest-bf16 search (table lookup, not the oracle's method) --
_POS_BITS = np.arange(0x0000, 0x7F80, dtype=np.uint16)       # +0 .. max finite
_POS_VALS = bf16_to_f64(_POS_BITS)                            # ascending
_MAX = _POS_VALS[-1]
_OVF_MID = (_MAX + 2.0 ** 128) / 2.0                          # exact in binary64


def nearest_bf16(t) -> np.ndarray:
    """Round binary64 values to the nearest bf16 by searching the sorted table of
    all finite bf16 values; exact ties go to the even bit pattern.  NaN maps to
    0x7FC0, overflow to +-Inf."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t).ravel()
    out = np.zeros(a.shape, dtype=np.uint16)
    fin = np.isfinite(a) & (a < _OVF_MID)
    af = a[fin]
    hi = np.clip(np.searchsorted(_POS_VALS, af, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, None)
    hv, lv = _POS_VALS[hi], _POS_VALS[lo]
    below_max = af <= _MAX
    # beyond the largest finite value but below the overflow midpoint: max finite
    d_lo = af - lv
    d_hi = hv - af
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_BITS[hi] & 1) == 0))
    exact = _POS_VALS[hi] == af
    res = np.where(exact | pick_hi, _POS_BITS[hi], _POS_BITS[lo])
    res = np.where(below_max, res, _POS_BITS[-1])
    out[fin] = res
    out[~fin] = 0x7F80
    out[np.isnan(a)] = 0x7FC0
    neg = np.signbit(t.ravel()) & ~np.isnan(a)
    out[neg] |= 0x8000
    return out.reshape(t.shape)


def near_bf16_tie(t, rel=2.0 ** -40) -> np.ndarray:
    """True where |t| lies within rel (relative) of the midpoint of the two
    finite bf16 values that bracket it."""
    a = np.abs(np.asarray(t, dtype=np.float64))
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 1, len(_POS_VALS) - 1)
    mid = (_POS_VALS[hi - 1] + _POS_VALS[hi]) / 2.0
    tol = rel * np.maximum(a, 2.0 ** -133)
    return np.abs(a - mid) <= tol
