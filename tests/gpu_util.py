"""Helpers for the GPU parity tests: device transfer of bf16 bit arrays, running
a workload through the C ABI, and the oracle comparison at the contract's bar
(residual_out bit-exact; y within max(2 ulp, 1e-2)) plus the tighter quality
the kernels reach inside it.  The comparison itself needs no GPU; a CPU test
checks that it rejects planted errors."""
from __future__ import annotations

import sys
import time

import numpy as np

from util import bf16_to_f64, bf16_ulp, check_y, ulp_diff


def log(*a):
    print("[gpu-test %s]" % time.strftime("%H:%M:%S"), *a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; torch.cuda.is_available() is False")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(dev or "cuda:0")


def to_host(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def workload_flags(rn, wl) -> int:
    f = rn.RN_RMS if wl.is_rms else 0
    if wl.op == "fused" and wl.gate_layout is not None:
        f |= rn.RN_GATE
    if wl.has_weight:
        f |= rn.RN_WEIGHT
    if wl.has_bias:
        f |= rn.RN_BIAS
    return f


def launch_workload(rn, wl, d: dict, y, ro=None, stream=None):
    """Enqueue one pass of the workload on device tensors d -> y (and ro)."""
    flags = workload_flags(rn, wl)
    if wl.op == "fused":
        rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d.get("gate"), d.get("weight"),
                             d.get("bias"), d["scale"], d["shift"], wl.B, wl.L, wl.D, flags,
                             wl.gate_layout or (0, 0), wl.ss_layout, wl.eps, stream)
    else:
        rn.norm_scale_shift_fwd(y, d["x"], d.get("weight"), d.get("bias"), d["scale"],
                                d["shift"], wl.B, wl.L, wl.D, flags, wl.ss_layout, wl.eps, stream)


# What the kernels achieve beyond the contract, asserted so that a regression
# inside the contract's loose absolute floor cannot pass unnoticed.  The
# kernels compute t = n * (1 + scale) + shift in binary32: with |n| up to a
# few units, its error against the binary64 oracle is a few binary32 ulps of
# n, about 2^-20 absolute, so (a) wherever |y| >= 2^-6 (bf16 ulp >= 2^-13)
# the rounded results differ by at most one bf16 ulp (only next to a
# rounding boundary), and (b) everywhere the difference is at most one ulp
# of the oracle's value plus 2^-14 -- far below the contract's 1e-2 floor,
# which is about 80 ulps at |y| = 2^-6.
QUALITY_FLOOR = 2.0 ** -6
QUALITY_MAX_ULP = 1.0
QUALITY_ABS = 2.0 ** -14
# Full-size workloads: at most this fraction of y may differ in any bit
# (measured: 99.998 % bit-identical; one element in ~5e4 sits close enough to
# a bf16 rounding boundary for the binary32 result to round the other way).
FULL_SIZE_MIN_IDENTICAL = 0.9995


def compare_outputs(y_gpu, y_ref, ro_gpu=None, ro_ref=None, what="", min_identical=None):
    """Assert the contract (residual_out bit-exact; y within max(2 ulp, 1e-2))
    and the quality the kernels have inside it: at most 1 ulp wherever
    |y_ref| >= 2^-6, at most 1 ulp + 2^-14 everywhere, and, if
    min_identical is given, at least that fraction of y bit-identical.

    Returns statistics of y: max ulp error where |y_ref| >= 1 (where the ulp
    term of the tolerance is the binding one), max ulp error where
    |y_ref| >= 2^-6, max absolute error, and the fraction of bit-identical
    elements."""
    if ro_ref is not None:
        diff = np.flatnonzero(ro_gpu.ravel() != ro_ref.ravel())
        assert diff.size == 0, "%s residual_out differs at %d elements (first flat index %d: gpu %04x oracle %04x)" % (
            what, diff.size, diff[0], ro_gpu.ravel()[diff[0]], ro_ref.ravel()[diff[0]])
    yg = y_gpu.ravel()
    yr = y_ref.ravel()
    idx = np.flatnonzero(yg != yr)
    stats = {"ulp_ge1": 0.0, "ulp_ge_1_64": 0.0, "abs": 0.0, "identical": 1.0 - idx.size / max(1, yg.size)}
    if min_identical is not None:
        assert stats["identical"] >= min_identical, "%s: only %.5f%% of y bit-identical (floor %.5f%%)" % (
            what, 100 * stats["identical"], 100 * min_identical)
    if idx.size == 0:
        return stats
    ok, _, n_bad, first = check_y(yg[idx], yr[idx])
    assert ok, "%s y outside tolerance at %d elements (first flat index %d: gpu %04x oracle %04x)" % (
        what, n_bad, idx[first], yg[idx[first]], yr[idx[first]])
    ref = np.abs(bf16_to_f64(yr[idx]))
    ulps = ulp_diff(yg[idx], yr[idx])
    absd = np.abs(bf16_to_f64(yg[idx]) - bf16_to_f64(yr[idx]))
    big = ref >= QUALITY_FLOOR
    bad = np.flatnonzero(big & (ulps > QUALITY_MAX_ULP))
    assert bad.size == 0, "%s: y differs by %.0f ulp where |y| >= 2^-6 (flat index %d: gpu %04x oracle %04x)" % (
        what, ulps[bad[0]], idx[bad[0]], yg[idx[bad[0]]], yr[idx[bad[0]]])
    lim = bf16_ulp(bf16_to_f64(yr[idx])) + QUALITY_ABS
    bad = np.flatnonzero(absd > lim)
    assert bad.size == 0, "%s: y differs by %.3g (> 1 ulp + 2^-14) (flat index %d: gpu %04x oracle %04x)" % (
        what, absd[bad[0]], idx[bad[0]], yg[idx[bad[0]]], yr[idx[bad[0]]])
    stats["abs"] = float(absd.max())
    if (ref >= 1).any():
        stats["ulp_ge1"] = float(ulps[ref >= 1].max())
    if big.any():
        stats["ulp_ge_1_64"] = float(ulps[big].max())
    return stats
