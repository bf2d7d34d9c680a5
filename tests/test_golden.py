"""Hand-worked rows (tests/golden/worked_rows.txt) against the oracle (CPU)
and against the HIP path through the C ABI (GPU).

Every value in the fixture is a small dyadic number and every expected output
follows exactly from the definition, as derived in the fixture next to each
case; none was produced by either implementation.  The oracle, which rounds
its binary64 result once, must reproduce every bit; the HIP path must
reproduce residual_out bit for bit and y within the contract's bar."""
import numpy as np
import pytest

from golden_cases import load_cases
from util import bf16_to_f64, check_y

CASES = load_cases()
IDS = [c["name"] for c in CASES]


def _op_rows(lay, B, L):
    kind, frames = lay
    return {0: 1, 1: B * L, 2: B * frames}[kind]


def test_fixture_is_consistent():
    """Sizes in every case agree with its layouts, so a bad fixture cannot pass
    silently."""
    assert len(CASES) == 9
    for c in CASES:
        B, L, D = c["B"], c["L"], c["D"]
        n = B * L * D
        assert c["op"] in ("fused", "nss") and c["norm"] in ("layer", "rms"), c["name"]
        assert c["x"].size == n and c["expect.y"].size == n, c["name"]
        ss = _op_rows(c["layout.ss"], B, L) * D
        assert c["scale"].size == ss and c["shift"].size == ss, c["name"]
        for k in ("weight", "bias"):
            assert k not in c or c[k].size == D, c["name"]
        if c["op"] == "fused":
            assert c["residual"].size == n and c["expect.residual_out"].size == n, c["name"]
            assert c["gate"].size == _op_rows(c["layout.gate"], B, L) * D, c["name"]
        else:
            assert "residual" not in c and "gate" not in c, c["name"]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_oracle_reproduces_worked_rows(orc, case):
    c = case
    common = dict(B=c["B"], L=c["L"], D=c["D"], is_rms=c["norm"] == "rms",
                  ss_layout=c["layout.ss"], eps=c["eps"])
    if c["op"] == "fused":
        y, ro, _ = orc.fused(c["x"], c["residual"], c["gate"], c.get("weight"), c.get("bias"),
                             c["scale"], c["shift"], gate_layout=c["layout.gate"], **common)
        np.testing.assert_array_equal(ro.ravel(), c["expect.residual_out"])
    else:
        y, _ = orc.nss(c["x"], c.get("weight"), c.get("bias"), c["scale"], c["shift"], **common)
    np.testing.assert_array_equal(y.ravel(), c["expect.y"])


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_hip_path_reproduces_worked_rows(case):
    from gpu_util import log, require_gpu, to_dev, to_host
    import torch
    dev = require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    c = case
    log("golden case %s: B %d L %d D %d %s/%s" % (c["name"], c["B"], c["L"], c["D"], c["op"], c["norm"]))
    B, L, D = c["B"], c["L"], c["D"]
    flags = rn.RN_RMS if c["norm"] == "rms" else 0
    flags |= rn.RN_WEIGHT if "weight" in c else 0
    flags |= rn.RN_BIAS if "bias" in c else 0
    d = {k: to_dev(c[k], dev) for k in ("x", "residual", "gate", "weight", "bias", "scale", "shift")
         if k in c}
    y = torch.full((B * L * D,), float("nan"), dtype=torch.bfloat16, device=dev)
    if c["op"] == "fused":
        flags |= rn.RN_GATE
        ro = torch.full_like(y, float("nan"))
        rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d["gate"], d.get("weight"),
                             d.get("bias"), d["scale"], d["shift"], B, L, D, flags,
                             c["layout.gate"], c["layout.ss"], c["eps"])
    else:
        rn.norm_scale_shift_fwd(y, d["x"], d.get("weight"), d.get("bias"), d["scale"],
                                d["shift"], B, L, D, flags, c["layout.ss"], c["eps"])
    torch.cuda.synchronize()
    if c["op"] == "fused":
        np.testing.assert_array_equal(to_host(ro), c["expect.residual_out"])
    got = to_host(y)
    ok, max_ulps, n_bad, first = check_y(got, c["expect.y"])
    assert ok, "%s: y[%d] = %r, expected %r" % (c["name"], first, bf16_to_f64(got[first]),
                                                bf16_to_f64(c["expect.y"][first]))
