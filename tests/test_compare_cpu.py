"""The GPU parity comparison rejects errors the contract's loose floor would
let through (CPU only: planted errors in copies of oracle outputs, no GPU).

The contract bar is max(2 bf16 ulps, 1e-2); its absolute floor is about 80
ulps at |y| = 2^-6, so by itself it would pass a kernel that lost tens of
ulps on every output below |y| ~ 0.64.  compare_outputs also asserts what the
kernels reach (1 ulp where |y| >= 2^-6, 1 ulp + 2^-14 everywhere, a floor on
the bit-identical fraction of full-size workloads); each planted error below
fails one of those while passing the contract alone."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import FULL_SIZE_MIN_IDENTICAL, compare_outputs
from util import bf16_to_f64, check_y


@pytest.fixture(scope="module")
def y_ref():
    """Oracle output of one small fused workload (16 rows x 5120)."""
    wl = synth.WORKLOADS["fused_ln_b1_l16_d5120"]
    inp = synth.make_inputs(wl, threads=1)
    y, ro, _ = oracle.Oracle().run_workload(wl, inp)
    return y.ravel().copy(), ro.ravel().copy()


def _plant(y, mask, ulps):
    """Move the masked finite bf16 values `ulps` units away from zero (the bit
    pattern of a finite bf16 value of one sign is monotonic in its magnitude)."""
    out = y.copy()
    out[mask] = (out[mask].astype(np.int32) + ulps).astype(np.uint16)
    return out


def _band(y, lo, hi):
    a = np.abs(bf16_to_f64(y))
    return (a >= lo) & (a < hi)


def test_exact_copy_passes(y_ref):
    y, ro = y_ref
    st = compare_outputs(y.copy(), y, ro.copy(), ro, "copy", min_identical=FULL_SIZE_MIN_IDENTICAL)
    assert st["identical"] == 1.0


def test_one_ulp_passes(y_ref):
    y, _ = y_ref
    m = np.zeros(y.size, bool)
    m[::5000] = True                       # 17 elements, 1 ulp each
    compare_outputs(_plant(y, m, 1), y, what="1 ulp", min_identical=FULL_SIZE_MIN_IDENTICAL)


@pytest.mark.parametrize("lo,hi", [(2.0 ** -6, 2.0 ** -4), (2.0 ** -4, 0.48)])
def test_four_ulps_on_small_outputs_fail(y_ref, lo, hi):
    y, _ = y_ref
    m = _band(y, lo, hi)
    assert m.sum() > 100
    bad = _plant(y, m, 4)
    assert check_y(bad, y)[0], "the contract bar alone passes this error"
    with pytest.raises(AssertionError, match="ulp where"):
        compare_outputs(bad, y, what="planted")


def test_tiny_outputs_bounded_absolutely(y_ref):
    """Below 2^-6 the ulp shrinks; 16 ulps at |y| in [2^-8, 2^-7) is 2^-11,
    far over 1 ulp + 2^-14 yet inside the contract's 1e-2."""
    y, _ = y_ref
    m = _band(y, 2.0 ** -8, 2.0 ** -7)
    assert m.sum() > 10
    bad = _plant(y, m, 16)
    assert check_y(bad, y)[0]
    with pytest.raises(AssertionError, match="2\\^-14"):
        compare_outputs(bad, y, what="planted tiny")


def test_identical_floor(y_ref):
    """One element in 500 off by one ulp: within every per-element bound, but
    below the full-size workloads' bit-identical floor."""
    y, _ = y_ref
    m = np.zeros(y.size, bool)
    m[::500] = True
    bad = _plant(y, m, 1)
    compare_outputs(bad, y, what="per-element bounds only")
    with pytest.raises(AssertionError, match="bit-identical"):
        compare_outputs(bad, y, what="floor", min_identical=FULL_SIZE_MIN_IDENTICAL)


def test_residual_bit_flip_fails(y_ref):
    y, ro = y_ref
    bad = ro.copy()
    bad[123] ^= 1
    with pytest.raises(AssertionError, match="residual_out differs"):
        compare_outputs(y.copy(), y, bad, ro, "residual")
