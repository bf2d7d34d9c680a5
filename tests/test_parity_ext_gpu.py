"""Parity of the extended entry points (binary32 weight/bias, binary32 and
FP8 E4M3 outputs, per-batch modulation) with the CPU oracle on the GPU.

Bars:
  * residual_out bit-exact, as for the bf16 entry points;
  * bf16 y: max(2 ulp, 1e-2), as for the bf16 entry points;
  * binary32 y: |y - t| <= 2^-14 * max(1, |t|) against the oracle's binary32
    rounding of its binary64 t.  The kernel evaluates (h - mean) * rstd
    [* w + b] * (1 + scale) + shift in binary32 with a binary32 mean and
    variance: about ten roundings of relative size 2^-24 on terms of magnitude
    |n| <= 8 for these inputs, i.e. a few times 2^-20 absolute; 2^-14 leaves a
    wide margin while still catching any wrong term (a wrong term moves y by
    the size of a bf16 modulation value, >= 2^-10 here);
  * FP8 y: the per-row scale within 2^-20 relative of the oracle's, and every
    element's decoded value within one E4M3 step of the oracle's (the binary32
    t can sit on the other side of an E4M3 rounding boundary from the binary64
    one), with at least 99.9 % of the codes identical.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import compare_outputs, log, require_gpu, to_dev, to_host
from util import bf16_to_f64

pytestmark = pytest.mark.gpu

BCAST, ROW, FRAME = 0, 1, 2
THREADS = max(1, min(16, os.cpu_count() or 1))
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.fixture(scope="module")
def rn():
    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    return rn


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def e4m3_step(dec):
    a = np.abs(dec)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -6, np.exp2(e - 3), 2.0 ** -9)


def check_y_f32(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = 2.0 ** -14 * np.maximum(1.0, np.abs(ref.astype(np.float64)))
    bad = err > tol
    assert not bad.any(), "%s: binary32 y off by %g at %d elements" % (what, err.max(), bad.sum())
    return float(err.max())


def check_y_fp8(q_gpu, s_gpu, q_ref, s_ref, what, min_same=0.999):
    np.testing.assert_allclose(s_gpu, s_ref, rtol=2.0 ** -20, atol=0, err_msg=what)
    dg = E4M3[q_gpu.ravel()]
    dr = E4M3[q_ref.ravel()]
    bad = np.abs(dg - dr) > e4m3_step(dr) * (1 + 1e-12)
    assert not bad.any(), "%s: %d FP8 codes more than one step away" % (what, bad.sum())
    same = float(np.mean(q_gpu.ravel() == q_ref.ravel()))
    assert same >= min_same, "%s: only %.4f%% of FP8 codes identical" % (what, 100 * same)
    return same


def _problem(seed, fused, gate_layout, aff, ss_layout, B, L, D):
    R = B * L

    def rows(lay):
        return {BCAST: 1, ROW: R, FRAME: B * lay[1]}[lay[0]]

    rng = np.random.default_rng(seed)
    inp = {"x": synth.random_bf16((R, D), seed, 1)}
    if fused:
        inp["residual"] = synth.random_bf16((R, D), seed, 2)
        if gate_layout is not None:
            inp["gate"] = synth.random_bf16((rows(gate_layout), D), seed, 3, dist=synth.UNIFORM,
                                            a=0.0, b=1.0)
    if aff in (1, 2):
        inp["weight"] = synth.random_bf16((D,), seed, 4, a=1.0, b=0.05)
        if aff == 2:
            inp["bias"] = synth.random_bf16((D,), seed, 5, a=0.0, b=0.1)
    if aff in (3, 4):  # binary32, not bf16 values
        inp["weight"] = (1.0 + 0.05 * rng.standard_normal(D)).astype(np.float32)
        if aff == 4:
            inp["bias"] = (0.1 * rng.standard_normal(D)).astype(np.float32)
    inp["scale"] = synth.random_bf16((rows(ss_layout), D), seed, 6, a=0.0, b=0.1)
    inp["shift"] = synth.random_bf16((rows(ss_layout), D), seed, 7, a=0.0, b=0.1)
    return inp


def _run(rn, orc, seed, fused, rms, gate_layout, aff, ss_layout, B, L, D, y_dtype, eps=1e-6):
    """One problem through the _ex entry point and the oracle; checks and
    returns a short statistic."""
    inp = _problem(seed, fused, gate_layout, aff, ss_layout, B, L, D)
    return _run_inputs(rn, orc, inp, fused, rms, gate_layout, aff, ss_layout, B, L, D, y_dtype,
                       eps, seed)


def _run_inputs(rn, orc, inp, fused, rms, gate_layout, aff, ss_layout, B, L, D, y_dtype,
                eps=1e-6, seed=-1):
    """_run on given inputs (a dict as _problem returns)."""
    aff32 = aff in (3, 4)
    d = {}
    for k, v in inp.items():
        d[k] = f32_dev(v) if v.dtype == np.float32 else to_dev(v)
    R = B * L
    flags = (rn.RN_RMS if rms else 0) | (rn.RN_WEIGHT if aff else 0) | \
        (rn.RN_BIAS if aff in (2, 4) else 0)
    ydt = {0: torch.bfloat16, 1: torch.float32, 2: torch.float8_e4m3fn}[y_dtype]
    y = torch.empty((R, D), dtype=ydt, device="cuda")
    ys = torch.empty((R,), dtype=torch.float32, device="cuda") if y_dtype == 2 else None
    case = "seed=%d fused=%s rms=%s gate=%s aff=%d ss=%s B=%d L=%d D=%d y=%d eps=%g" % (
        seed, fused, rms, gate_layout, aff, ss_layout, B, L, D, y_dtype, eps)
    adt = rn.RN_DTYPE_F32 if aff32 else rn.RN_DTYPE_BF16
    if fused:
        if gate_layout is not None:
            flags |= rn.RN_GATE
        ro = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        rn.resnorm_fused_fwd_ex(y, ro, d["x"], d["residual"], d.get("gate"), d.get("weight"),
                                d.get("bias"), d["scale"], d["shift"], B, L, D, flags,
                                gate_layout or (BCAST, 0), ss_layout, eps, adt, y_dtype, ys)
        torch.cuda.synchronize()
        res = orc.fused(inp["x"], inp["residual"], inp.get("gate"), inp.get("weight"),
                        inp.get("bias"), inp["scale"], inp["shift"], B, L, D, rms,
                        gate_layout or (BCAST, 0), ss_layout, eps, affine_f32=aff32,
                        y_dtype=y_dtype, threads=THREADS)
        y_ref, ro_ref = res[0], res[1]
        assert np.array_equal(to_host(ro), ro_ref), case + ": residual_out not bit-exact"
    else:
        rn.norm_scale_shift_fwd_ex(y, d["x"], d.get("weight"), d.get("bias"), d["scale"],
                                   d["shift"], B, L, D, flags, ss_layout, eps, adt, y_dtype, ys)
        torch.cuda.synchronize()
        res = orc.nss(inp["x"], inp.get("weight"), inp.get("bias"), inp["scale"], inp["shift"],
                      B, L, D, rms, ss_layout, eps, affine_f32=aff32, y_dtype=y_dtype,
                      threads=THREADS)
        y_ref = res[0]
    if y_dtype == 0:
        return compare_outputs(to_host(y), y_ref, what=case)
    if y_dtype == 1:
        return check_y_f32(y.cpu().numpy(), y_ref, case)
    return check_y_fp8(y.view(torch.uint8).cpu().numpy(), ys.cpu().numpy(), y_ref, res[-1], case)


WIDTHS = [8, 520, 1000, 5120, 8200, 10240, 16384]


@pytest.mark.parametrize("D", WIDTHS)
def test_affine_f32_matrix(rn, orc, D):
    """binary32 weight / weight+bias, both norms, fused and norm-only, bf16 y."""
    log("fp32 affine matrix D=%d" % D)
    k = 0
    for rms in (False, True):
        for aff in (3, 4):
            for fused in (True, False):
                sl = [(BCAST, 0), (ROW, 0), (FRAME, 3)][k % 3]
                gl = (FRAME, 3) if fused and k % 2 else ((BCAST, 0) if fused else None)
                _run(rn, orc, 500 + k + D, fused, rms, gl, aff, sl, 2, 6, D, 0)
                k += 1


@pytest.mark.parametrize("y_dtype", [1, 2])
@pytest.mark.parametrize("D", WIDTHS)
def test_output_dtypes_matrix(rn, orc, D, y_dtype):
    """binary32 and FP8 y across norms, ops, every affine variant and layouts."""
    log("output dtype %d matrix D=%d" % (y_dtype, D))
    k = 0
    for rms in (False, True):
        for aff in (0, 1, 2, 3, 4):
            for fused in (True, False):
                sl = [(BCAST, 0), (ROW, 0), (FRAME, 3)][k % 3]
                gl = (ROW, 0) if fused and k % 2 else ((BCAST, 0) if fused else None)
                _run(rn, orc, 700 + k + D, fused, rms, gl, aff, sl, 2, 6, D, y_dtype)
                k += 1


def _random_cases(n, seed):
    """n seeded random problems: row widths spread over 8..16384 (half of them
    within 8 elements of a multiple of 512, where shapes change), 1..~3000
    rows, every flag, layout, affine type, output type, and four eps values."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        if rng.random() < 0.5:
            D = int(rng.integers(1, 2049)) * 8
        else:
            D = int(np.clip(512 * int(rng.integers(1, 33)) + 8 * int(rng.integers(-1, 2)), 8, 16384))
        B = int(rng.integers(1, 4))
        F = int(rng.choice([1, 2, 3, 5]))
        L = F * max(1, int(np.exp(rng.uniform(0, np.log(1000))) / F))
        if B * L * D > 8_000_000:
            continue
        fused = bool(rng.random() < 0.6)
        lay = lambda: [(BCAST, 0), (ROW, 0), (FRAME, F)][int(rng.integers(0, 3))]  # noqa: E731
        gl = (lay() if rng.random() < 0.75 else None) if fused else None
        cases.append(dict(fused=fused, rms=bool(rng.random() < 0.5), gate_layout=gl,
                          aff=int(rng.integers(0, 5)), ss_layout=lay(), B=B, L=L, D=D,
                          y_dtype=int(rng.choice([0, 0, 0, 1, 2])),
                          eps=float(rng.choice([1e-6, 1e-5, 0.0, 1e-2]))))
    return cases


# Power-of-two row widths (D = 4096, 8192, 16384, where every shape covers
# the row exactly): odd row counts (the last workgroup partly empty), one
# wave per row with weight and bias in LDS, the multi-row norm-only shapes,
# several waves per row, every output type.
# (B, L, D, fused, aff, y dtype, rms, gate layout, scale/shift layout)
POW2 = [
    (1, 1023, 4096, True, 0, 0, False, (BCAST, 0), (BCAST, 0)),
    (1, 1023, 4096, True, 4, 2, True, (FRAME, 3), (FRAME, 3)),
    (1, 3073, 4096, False, 2, 1, False, None, (BCAST, 0)),     # 4 rows per wave
    (1, 1025, 8192, True, 3, 0, True, (BCAST, 0), (BCAST, 0)),
    (2, 1028, 8192, False, 4, 2, False, None, (FRAME, 257)),    # 4 rows per wave, per frame
    (1, 513, 16384, True, 0, 1, False, (ROW, 0), (BCAST, 0)),
    (1, 771, 16384, False, 0, 0, True, None, (ROW, 0)),
    (3, 5, 4096, True, 2, 0, False, (BCAST, 0), (ROW, 0)),
]


@pytest.mark.parametrize("case", POW2)
def test_power_of_two_widths(rn, orc, case):
    B, L, D, fused, aff, y_dtype, rms, gl, sl = case
    log("power-of-two width: B=%d L=%d D=%d fused=%s aff=%d y=%d rms=%s gate=%s ss=%s" % case)
    _run(rn, orc, 2100 + D // 512 + aff + y_dtype, fused, rms, gl, aff, sl, B, L, D, y_dtype)


# The fused op with weight and one wave per row stages weight and bias in
# LDS: every affine type and output type, 1023 rows (the last workgroup of
# four rows has one empty slot, whose wave still takes part in the LDS fill
# and the barrier), ragged and full rows, broadcast and per-frame layouts.
# (L, D, aff, y dtype, rms, gate layout, scale/shift layout)
LDS_AFFINE = [
    (1023, 5120, 1, 0, False, (BCAST, 0), (BCAST, 0)),
    (1023, 5120, 2, 1, True, (FRAME, 3), (FRAME, 3)),
    (1023, 5120, 3, 2, False, (BCAST, 0), (FRAME, 3)),
    (1023, 5120, 4, 0, False, (FRAME, 3), (BCAST, 0)),
    (1023, 5120, 4, 1, True, (BCAST, 0), (BCAST, 0)),
    (1023, 5120, 4, 2, True, (BCAST, 0), (FRAME, 3)),
    (1023, 3000, 4, 0, True, (BCAST, 0), (BCAST, 0)),
    (1023, 3000, 2, 2, False, (FRAME, 3), (BCAST, 0)),
    (1023, 1000, 3, 1, False, (BCAST, 0), (FRAME, 3)),
    (1023, 1000, 1, 0, True, None, (BCAST, 0)),
]


@pytest.mark.parametrize("case", LDS_AFFINE)
def test_fused_affine_lds(rn, orc, case):
    L, D, aff, y_dtype, rms, gl, sl = case
    flags = rn.RN_WEIGHT | (rn.RN_BIAS if aff in (2, 4) else 0) | (rn.RN_GATE if gl else 0)
    info = rn.describe_launch(1, L, D, flags, True, gl or (BCAST, 0), sl,
                              affine_dtype=rn.RN_DTYPE_F32 if aff in (3, 4) else rn.RN_DTYPE_BF16)
    assert (info["waves_per_row"], info["rows_per_wave"]) == (1, 1)
    log("fused affine, weight/bias in LDS: L=%d D=%d aff=%d y=%d rms=%s gate=%s ss=%s" % case)
    _run(rn, orc, 1900 + D + 7 * aff + y_dtype, True, rms, gl, aff, sl, 1, L, D, y_dtype)


# Multi-row shapes (the norm-only op with weight on large problems): odd row
# counts (a partly empty last workgroup), ragged rows, every W, affine and
# output type, broadcast, per-frame (164 tokens per frame) and per-batch
# scale/shift.  (B, L, D, aff, scale/shift layout, y dtype, rms, expected W)
MULTI_ROW = [
    (1, 12599, 1000, 4, (BCAST, 0), 0, False, 1),
    (1, 12599, 1000, 1, (BCAST, 0), 2, True, 1),
    (1, 8195, 3000, 2, (BCAST, 0), 1, True, 2),
    (1, 8200, 5120, 4, (FRAME, 50), 0, False, 2),
    (2, 4100, 5120, 3, (FRAME, 1), 2, False, 2),
    (1, 8200, 9000, 3, (FRAME, 50), 1, False, 4),
    (1, 8195, 9000, 2, (BCAST, 0), 0, True, 4),
]


@pytest.mark.parametrize("case", MULTI_ROW)
def test_multi_row_shapes(rn, orc, case):
    B, L, D, aff, sl, y_dtype, rms, w = case
    flags = rn.RN_WEIGHT | (rn.RN_BIAS if aff in (2, 4) else 0) | (rn.RN_RMS if rms else 0)
    info = rn.describe_launch(B, L, D, flags, False, (BCAST, 0), sl,
                              affine_dtype=rn.RN_DTYPE_F32 if aff in (3, 4) else rn.RN_DTYPE_BF16)
    assert (info["rows_per_wave"], info["waves_per_row"]) == (4, w)
    log("multi-row: B=%d L=%d D=%d aff=%d ss=%s y=%d rms=%s" % case[:7])
    _run(rn, orc, 1700 + D + aff, False, rms, None, aff, sl, B, L, D, y_dtype)


def test_random_matrix(rn, orc):
    """400 seeded random problems through the _ex entry points against the
    oracle, each at the bar of its output type; the planner picks whatever
    shape each problem gets (all four waves-per-row families are exercised)."""
    cases = _random_cases(400, 4321)
    seen = set()
    for k, c in enumerate(cases):
        flags = (rn.RN_RMS if c["rms"] else 0) | (rn.RN_WEIGHT if c["aff"] else 0) | \
            (rn.RN_BIAS if c["aff"] in (2, 4) else 0) | (rn.RN_GATE if c["gate_layout"] else 0)
        info = rn.describe_launch(c["B"], c["L"], c["D"], flags, c["fused"],
                                  c["gate_layout"] or (BCAST, 0), c["ss_layout"],
                                  rn.RN_DTYPE_F32 if c["aff"] in (3, 4) else rn.RN_DTYPE_BF16)
        seen.add(info["waves_per_row"])
        log("random case %d: %s" % (k, c))
        _run(rn, orc, 1000 + k, c["fused"], c["rms"], c["gate_layout"], c["aff"], c["ss_layout"],
             c["B"], c["L"], c["D"], c["y_dtype"], c["eps"])
    assert seen == {1, 2, 4, 10}, seen


@pytest.mark.parametrize("B", [2, 4])
def test_per_batch_modulation(rn, orc, B):
    """Per-batch gate and scale/shift, (B, 1, C) and (B, C), through the tensor
    API: mapped to the per-frame layout with one frame per batch; also the
    explicit (B, 1, 1, C) frame layout."""
    D, L = 5120, 40
    inp = _problem(900 + B, True, (FRAME, 1), 0, (FRAME, 1), B, L, D)
    d = {k: to_dev(v) for k, v in inp.items()}
    x3 = d["x"].view(B, L, D)
    r3 = d["residual"].view(B, L, D)
    y_ref, ro_ref, _ = orc.fused(inp["x"], inp["residual"], inp["gate"], None, None, inp["scale"],
                                 inp["shift"], B, L, D, False, (FRAME, 1), (FRAME, 1), 1e-6)
    for shape in ((B, 1, D), (B, D), (B, 1, 1, D)):
        y, ro = rn.fused_residual_norm_scale_shift(
            r3, x3, d["gate"].view(*shape), None, None, d["scale"].view(*shape),
            d["shift"].view(*shape), "layer", 1e-6)
        torch.cuda.synchronize()
        compare_outputs(to_host(y).reshape(-1, D), y_ref, to_host(ro).reshape(-1, D), ro_ref,
                        "per-batch %s" % (shape,))
    # norm-only, RMS, per-batch (B, C)
    y_ref, _ = orc.nss(inp["x"], None, None, inp["scale"], inp["shift"], B, L, D, True, (FRAME, 1))
    y = rn.norm_scale_shift(x3, None, None, d["scale"].view(B, D), d["shift"].view(B, D), "rms")
    torch.cuda.synchronize()
    compare_outputs(to_host(y).reshape(-1, D), y_ref, what="per-batch nss")


def test_tensor_api_dtypes(rn, orc):
    """The tensor-level API picks the affine dtype from the weight tensors and
    the output type from out_dtype; FP8 returns the per-row scales."""
    B, L, D = 1, 64, 5120
    inp = _problem(950, True, (BCAST, 0), 4, (BCAST, 0), B, L, D)
    x3 = to_dev(inp["x"]).view(B, L, D)
    r3 = to_dev(inp["residual"]).view(B, L, D)
    g, sc, sh = to_dev(inp["gate"]), to_dev(inp["scale"]), to_dev(inp["shift"])
    w, bb = f32_dev(inp["weight"]), f32_dev(inp["bias"])
    y8, ro, s = rn.fused_residual_norm_scale_shift(r3, x3, g, w, bb, sc, sh, "layer", 1e-6,
                                                   out_dtype=torch.float8_e4m3fn)
    y32, ro32 = rn.fused_residual_norm_scale_shift(r3, x3, g, w, bb, sc, sh, "layer", 1e-6,
                                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y8.dtype == torch.float8_e4m3fn and s.shape == (L,) and y32.dtype == torch.float32
    yr8, ror, _, sr = orc.fused(inp["x"], inp["residual"], inp["gate"], inp["weight"], inp["bias"],
                                inp["scale"], inp["shift"], B, L, D, False, affine_f32=True,
                                y_dtype=2)
    check_y_fp8(y8.view(torch.uint8).cpu().numpy().reshape(L, D), s.cpu().numpy(), yr8, sr, "api fp8")
    assert np.array_equal(to_host(ro).reshape(-1, D), ror)
    yr32, _, _ = orc.fused(inp["x"], inp["residual"], inp["gate"], inp["weight"], inp["bias"],
                           inp["scale"], inp["shift"], B, L, D, False, affine_f32=True, y_dtype=1)
    check_y_f32(y32.cpu().numpy().reshape(L, D), yr32, "api f32")
    with pytest.raises(TypeError):
        rn.fused_residual_norm_scale_shift(r3, x3, g, w, bb.to(torch.bfloat16), sc, sh)


@pytest.mark.parametrize("y_dtype,aff", [(0, 4), (2, 0), (1, 0)])
def test_full_size_ext(rn, orc, y_dtype, aff):
    """The WAN2.2 shape (B 1, L 176400, D 5120, broadcast modulation), every row:
    the fused LayerNorm with binary32 weight+bias (the pages' "fused affine"
    call), and the headline fused op with FP8 and binary32 outputs."""
    log("full size ext y=%d aff=%d" % (y_dtype, aff))
    B, L, D = 1, 176400, 5120
    wl = synth.WORKLOADS["fused_ln_b1_l90000_d5120"]
    inp = {"x": synth.fill(wl.dists[synth.X], 11, L * D, threads=THREADS).reshape(L, D),
           "residual": synth.fill(wl.dists[synth.RES], 11, L * D, threads=THREADS).reshape(L, D),
           "gate": synth.fill(wl.dists[synth.GATE], 11, D).reshape(1, D),
           "scale": synth.fill(wl.dists[synth.SCALE], 11, D).reshape(1, D),
           "shift": synth.fill(wl.dists[synth.SHIFT], 11, D).reshape(1, D)}
    rng = np.random.default_rng(11)
    if aff == 4:
        inp["weight"] = (1.0 + 0.05 * rng.standard_normal(D)).astype(np.float32)
        inp["bias"] = (0.1 * rng.standard_normal(D)).astype(np.float32)
    d = {k: (f32_dev(v) if v.dtype == np.float32 else to_dev(v)) for k, v in inp.items()}
    ydt = {0: torch.bfloat16, 1: torch.float32, 2: torch.float8_e4m3fn}[y_dtype]
    y = torch.empty((L, D), dtype=ydt, device="cuda")
    ro = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    ys = torch.empty((L,), dtype=torch.float32, device="cuda") if y_dtype == 2 else None
    flags = rn.RN_GATE | ((rn.RN_WEIGHT | rn.RN_BIAS) if aff else 0)
    rn.resnorm_fused_fwd_ex(y, ro, d["x"], d["residual"], d["gate"], d.get("weight"),
                            d.get("bias"), d["scale"], d["shift"], B, L, D, flags, (BCAST, 0),
                            (BCAST, 0), 1e-6, rn.RN_DTYPE_F32 if aff else rn.RN_DTYPE_BF16,
                            y_dtype, ys)
    torch.cuda.synchronize()
    res = orc.fused(inp["x"], inp["residual"], inp["gate"], inp.get("weight"), inp.get("bias"),
                    inp["scale"], inp["shift"], B, L, D, False, affine_f32=bool(aff),
                    y_dtype=y_dtype, threads=THREADS)
    assert np.array_equal(to_host(ro), res[1])
    if y_dtype == 0:
        st = compare_outputs(to_host(y), res[0], what="full-size fp32 affine")
        log("full size fp32 affine: max %.0f ulp where |y|>=1" % st["ulp_ge1"])
    elif y_dtype == 1:
        log("full size f32 y: max abs err %.3g" % check_y_f32(y.cpu().numpy(), res[0], "full f32"))
    else:
        same = check_y_fp8(y.view(torch.uint8).cpu().numpy(), ys.cpu().numpy(), res[0], res[3],
                           "full fp8")
        log("full size fp8 y: %.4f%% codes identical" % (100 * same))


def test_tensors_over_4gib(rn, orc):
    """Activations larger than 4 GiB (B 1, L 540677, D 4096: 4.4 GB per bf16
    tensor, 8.9 GB for a binary32 y), so byte offsets pass 2^32 both in the
    bf16 tensors (from row 524288) and in the binary32 output (from row
    262144): the rows on either side of each boundary, the first and the last
    rows, against the oracle (residual_out bit-exact, y at its bar)."""
    B, L, D = 1, 540677, 4096
    R = B * L
    wid = 77
    specs = {"x": synth.TensorSpec(synth.X, synth.NORMAL, 0.0, 1.0),
             "residual": synth.TensorSpec(synth.RES, synth.NORMAL, 0.0, 1.0)}
    mod = {"gate": synth.fill(synth.TensorSpec(synth.GATE, synth.UNIFORM, 0.0, 1.0), wid, D),
           "scale": synth.fill(synth.TensorSpec(synth.SCALE, synth.NORMAL, 0.0, 0.1), wid, D),
           "shift": synth.fill(synth.TensorSpec(synth.SHIFT, synth.NORMAL, 0.0, 0.1), wid, D)}
    log("over 4 GiB: generating %d x %d inputs" % (R, D))
    dev = {}
    for k, spec in specs.items():
        t = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        for a in range(0, R, 65536):
            b = min(R, a + 65536)
            host = synth.fill(spec, wid, (b - a) * D, idx0=a * D, threads=THREADS)
            t[a:b].copy_(torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).view(b - a, D))
        dev[k] = t
    dm = {k: to_dev(v.reshape(1, D)) for k, v in mod.items()}
    ro = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
    assert ro.numel() * 2 > 2 ** 32
    args = (dev["x"], dev["residual"], dm["gate"], None, None, dm["scale"], dm["shift"], B, L, D,
            rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6)
    log("over 4 GiB: bf16 y")
    rn.resnorm_fused_fwd(y, ro, *args)
    torch.cuda.synchronize()

    def rows_of(t, r0, n):
        return t[r0:r0 + n].contiguous()

    def oracle_rows(r0, n, y_dtype):
        xs = synth.fill(specs["x"], wid, n * D, idx0=r0 * D).reshape(n, D)
        rs = synth.fill(specs["residual"], wid, n * D, idx0=r0 * D).reshape(n, D)
        return orc.fused(xs, rs, mod["gate"].reshape(1, D), None, None, mod["scale"].reshape(1, D),
                         mod["shift"].reshape(1, D), B, L, D, False, (BCAST, 0), (BCAST, 0), 1e-6,
                         row0=r0, nrows=n, y_dtype=y_dtype)

    samples = [0, 262144 - 64, 524288 - 64, R - 64]
    for r0 in samples:
        y_ref, ro_ref, _ = oracle_rows(r0, 128 if r0 != R - 64 else 64, 0)
        n = y_ref.shape[0]
        compare_outputs(to_host(rows_of(y, r0, n)), y_ref, to_host(rows_of(ro, r0, n)), ro_ref,
                        "over 4 GiB, rows %d..%d" % (r0, r0 + n))
    del y
    log("over 4 GiB: binary32 y")
    y32 = torch.empty((R, D), dtype=torch.float32, device="cuda")
    ro.zero_()
    rn.resnorm_fused_fwd_ex(y32, ro, *args, rn.RN_DTYPE_BF16, rn.RN_DTYPE_F32)
    torch.cuda.synchronize()
    for r0 in samples:
        y_ref, ro_ref, _ = oracle_rows(r0, 128 if r0 != R - 64 else 64, 1)
        n = y_ref.shape[0]
        assert np.array_equal(to_host(rows_of(ro, r0, n)), ro_ref), r0
        check_y_f32(rows_of(y32, r0, n).cpu().numpy(), y_ref, "over 4 GiB f32, rows %d" % r0)
    del y32, ro, dev
    torch.cuda.empty_cache()


def test_degenerate_rows_ext_outputs(rn, orc):
    """Rows holding an infinity or a NaN, a residual sum that overflows to
    Inf, an all-zero row and a constant row, with binary32 and FP8 E4M3 y:
    NaN exactly where the oracle's is (NaN-ness, not payload or sign), equal
    infinities, the per-row FP8 scales equal (NaN / Inf included), and every
    finite element at its usual bar."""
    D, L = 1024, 6
    x = synth.random_bf16((L, D), 78, 1)
    r = synth.random_bf16((L, D), 78, 2)
    x[0, 5] = 0x7F80
    x[1, 7] = 0x7FC0
    x[2, :] = 0x7F7F
    r[2, :] = 0x7F7F
    x[3, :] = 0
    r[3, :] = 0
    x[4, :] = 0x3FC0
    r[4, :] = 0
    g = np.full((1, D), 0x3F80, np.uint16)
    sc = synth.random_bf16((1, D), 78, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 78, 7, a=0.0, b=0.1)
    d = {k: to_dev(v) for k, v in (("x", x), ("r", r), ("g", g), ("sc", sc), ("sh", sh))}
    for rms in (False, True):
        flags = (rn.RN_RMS if rms else 0) | rn.RN_GATE
        ro = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
        y32 = torch.empty((L, D), dtype=torch.float32, device="cuda")
        rn.resnorm_fused_fwd_ex(y32, ro, d["x"], d["r"], d["g"], None, None, d["sc"], d["sh"], 1, L,
                                D, flags, (BCAST, 0), (BCAST, 0), 1e-6, y_dtype=rn.RN_DTYPE_F32)
        y8 = torch.empty((L, D), dtype=torch.float8_e4m3fn, device="cuda")
        ys = torch.empty((L,), dtype=torch.float32, device="cuda")
        rn.resnorm_fused_fwd_ex(y8, ro, d["x"], d["r"], d["g"], None, None, d["sc"], d["sh"], 1, L,
                                D, flags, (BCAST, 0), (BCAST, 0), 1e-6,
                                y_dtype=rn.RN_DTYPE_FP8_E4M3, y_scale=ys)
        torch.cuda.synchronize()
        what = "rms=%s" % rms
        ref32 = orc.fused(x, r, g, None, None, sc, sh, 1, L, D, rms, y_dtype=1)[0]
        got32 = y32.cpu().numpy()
        assert np.array_equal(np.isnan(got32), np.isnan(ref32)), what + " f32 NaN positions"
        inf = np.isinf(ref32)
        assert np.array_equal(got32[inf], ref32[inf]), what + " f32 infinities"
        fin = np.isfinite(ref32)
        check_y_f32(got32[fin], ref32[fin], what + " f32")
        q_ref, _, _, s_ref = orc.fused(x, r, g, None, None, sc, sh, 1, L, D, rms, y_dtype=2)
        q_got, s_got = y8.view(torch.uint8).cpu().numpy(), ys.cpu().numpy()
        assert np.array_equal(np.isnan(s_got), np.isnan(s_ref)), what + " scale NaN"
        assert np.array_equal(np.isinf(s_got), np.isinf(s_ref)), what + " scale Inf"
        sf = np.isfinite(s_ref)
        np.testing.assert_allclose(s_got[sf], s_ref[sf], rtol=2.0 ** -20, atol=0)
        dg, dr = E4M3[q_got], E4M3[q_ref]
        assert np.array_equal(np.isnan(dg), np.isnan(dr)), what + " FP8 NaN positions"
        ok = np.isnan(dr) | (np.abs(dg - dr) <= e4m3_step(np.where(np.isnan(dr), 0, dr)) * (1 + 1e-12))
        assert ok.all(), what + " FP8 codes more than one step away"


def _near_constant_rows(D):
    """Rows whose spread is a few bf16 ulps of their mean (|mean| / std up to
    ~9000): all equal but one element one ulp up; a few elements one ulp up
    or down; a large value with one element one ulp up."""
    rows = []
    r = np.full(D, 0x3F80, np.uint16)          # 1.0 ...
    r[D // 3] = 0x3F81                         # ... and one 1.0078125
    rows.append(r)
    r = np.full(D, 0xC040, np.uint16)          # -3.0 ...
    r[::97] = 0xC041                           # ... a few one ulp below
    r[5::193] = 0xC03F                         # ... and a few one ulp above
    rows.append(r)
    r = np.full(D, 0x447A, np.uint16)          # 1000.0 ...
    r[-1] = 0x447B                             # ... and one 1004.0
    rows.append(r)
    r = np.full(D, 0x3DCD, np.uint16)          # 0.1001 ...
    r[:D // 2] = 0x3DCC                        # ... half of them one ulp lower
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("eps", [1e-6, 0.0])
@pytest.mark.parametrize("D,reps", [(5120, 1), (1000, 1), (5120, 1025)])
def test_near_constant_rows(rn, orc, D, reps, eps):
    """Rows whose values differ by a few bf16 ulps (|mean| >> std): the centred
    values must not carry the binary32 rounding of the mean, which the
    normalisation would magnify by |mean| / std; every output type at its
    bar, both ops (the fused op with the row as residual and x = 0).  Four
    rows reach the ten- and four-waves-per-row shapes; 4100 rows the one-wave
    shapes (a partly filled last workgroup)."""
    rows = np.tile(_near_constant_rows(D), (reps, 1))
    L = rows.shape[0]
    log("near-constant rows: D=%d L=%d eps=%g" % (D, L, eps))
    sc = synth.random_bf16((1, D), 79, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 79, 7, a=0.0, b=0.1)
    zeros = np.zeros((L, D), np.uint16)
    d = {k: to_dev(v) for k, v in (("h", rows), ("z", zeros), ("sc", sc), ("sh", sh))}
    for fused in (False, True):
        for y_dtype in (0, 1, 2):
            what = "near-constant D=%d eps=%g fused=%s y=%d" % (D, eps, fused, y_dtype)
            ydt = {0: torch.bfloat16, 1: torch.float32, 2: torch.float8_e4m3fn}[y_dtype]
            y = torch.empty((L, D), dtype=ydt, device="cuda")
            ys = torch.empty((L,), dtype=torch.float32, device="cuda") if y_dtype == 2 else None
            if fused:
                ro = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
                rn.resnorm_fused_fwd_ex(y, ro, d["z"], d["h"], None, None, None, d["sc"], d["sh"], 1, L,
                                        D, 0, (BCAST, 0), (BCAST, 0), eps, y_dtype=y_dtype, y_scale=ys)
                res = orc.fused(zeros, rows, None, None, None, sc, sh, 1, L, D, False, eps=eps,
                                y_dtype=y_dtype)
            else:
                rn.norm_scale_shift_fwd_ex(y, d["h"], None, None, d["sc"], d["sh"], 1, L, D, 0,
                                           (BCAST, 0), eps, y_dtype=y_dtype, y_scale=ys)
                res = orc.nss(rows, None, None, sc, sh, 1, L, D, False, eps=eps, y_dtype=y_dtype)
            torch.cuda.synchronize()
            if fused:
                assert np.array_equal(to_host(ro), rows), what
            if y_dtype == 0:
                compare_outputs(to_host(y), res[0], what=what)
            elif y_dtype == 1:
                check_y_f32(y.cpu().numpy(), res[0], what)
            else:
                check_y_fp8(y.view(torch.uint8).cpu().numpy(), ys.cpu().numpy(), res[0], res[-1], what)


def _scaled_bf16(bits, k):
    """bf16 values times 2^k, exactly (asserting no bit is lost)."""
    f = ((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * 2.0 ** k).astype(np.float32)
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _tiny_rows(D):
    """Rows of tiny values whose squares underflow binary32: N(0,1) times
    2^-60, 2^-90 and 2^-110 (every value kept in the normal range), 2^-100
    with every seventh element one ulp up (a common offset), and one plain
    N(0,1) row beside them."""
    base = synth.random_bf16((5, D), 83, 1)
    big = np.abs(((base.astype(np.uint32) << 16).view(np.float32))) >= 2.0 ** -12
    base = np.where(big, base, np.uint16(0x3F80))
    off = _scaled_bf16(np.full(D, 0x3F80, np.uint16), -100)
    off[::7] = _scaled_bf16(np.full(D, 0x3F81, np.uint16), -100)[::7]
    return np.stack([_scaled_bf16(base[0], -60), _scaled_bf16(base[1], -90),
                     _scaled_bf16(base[2], -110), off, base[4]])


@pytest.mark.parametrize("eps", [0.0, 1e-35])
@pytest.mark.parametrize("D,reps", [(2048, 1), (2048, 820), (1000, 1), (10240, 820)])
def test_tiny_rows_small_eps(rn, orc, D, reps, eps):
    """Rows whose centred squares underflow binary32, with eps 0 or far below
    their variance: the kernels recompute the variance on the row scaled up
    by a power of two.  Every output type, both ops, LayerNorm and RMSNorm;
    the shapes with four waves per row, four rows per workgroup (also
    ragged) and two waves per row with two rows per workgroup, where one
    row of a workgroup may take the recomputation and another not."""
    rows = np.tile(_tiny_rows(D), (reps, 1))
    L = rows.shape[0]
    log("tiny rows: D=%d L=%d eps=%g" % (D, L, eps))
    sc = synth.random_bf16((1, D), 83, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 83, 7, a=0.0, b=0.1)
    zeros = np.zeros((L, D), np.uint16)
    d = {k: to_dev(v) for k, v in (("h", rows), ("z", zeros), ("sc", sc), ("sh", sh))}
    for rms in (False, True):
        flags = rn.RN_RMS if rms else 0
        for fused in (False, True):
            for y_dtype in (0, 1, 2):
                what = "tiny rows D=%d L=%d rms=%s eps=%g fused=%s y=%d" % (D, L, rms, eps, fused, y_dtype)
                ydt = {0: torch.bfloat16, 1: torch.float32, 2: torch.float8_e4m3fn}[y_dtype]
                y = torch.empty((L, D), dtype=ydt, device="cuda")
                ys = torch.empty((L,), dtype=torch.float32, device="cuda") if y_dtype == 2 else None
                if fused:
                    ro = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
                    rn.resnorm_fused_fwd_ex(y, ro, d["z"], d["h"], None, None, None, d["sc"], d["sh"], 1,
                                            L, D, flags, (BCAST, 0), (BCAST, 0), eps, y_dtype=y_dtype,
                                            y_scale=ys)
                    res = orc.fused(zeros, rows, None, None, None, sc, sh, 1, L, D, rms, eps=eps,
                                    y_dtype=y_dtype)
                else:
                    rn.norm_scale_shift_fwd_ex(y, d["h"], None, None, d["sc"], d["sh"], 1, L, D, flags,
                                               (BCAST, 0), eps, y_dtype=y_dtype, y_scale=ys)
                    res = orc.nss(rows, None, None, sc, sh, 1, L, D, rms, eps=eps, y_dtype=y_dtype)
                torch.cuda.synchronize()
                if fused:
                    assert np.array_equal(to_host(ro), rows), what
                if y_dtype == 0:
                    compare_outputs(to_host(y), res[0], what=what)
                elif y_dtype == 1:
                    check_y_f32(y.cpu().numpy(), res[0], what)
                else:
                    # with eps > 0 the rows scaled by 2^-90, 2^-110 and 2^-100 have a
                    # variance far below eps: their y is the bf16 shift plus a few
                    # 2^-30 and less, so E4M3 rounding ties are common there (as for a
                    # constant row), each within one step
                    q, qs = y.view(torch.uint8).cpu().numpy(), ys.cpu().numpy()
                    tie = np.isin(np.arange(L) % 5, (1, 2, 3)) if eps > 0 else np.zeros(L, bool)
                    check_y_fp8(q[~tie], qs[~tie], res[0][~tie], res[-1][~tie], what)
                    if tie.any():
                        check_y_fp8(q[tie], qs[tie], res[0][tie], res[-1][tie], what + " (ties)",
                                    min_same=0.97)


def test_maximum_row_count(rn, orc):
    """B * L = 2^31 - 1 rows (the largest the ABI accepts) at D = 8: 34 GB per
    tensor and a grid of 2^29 workgroups.  The inputs are a seeded block of
    65536 rows tiled over the tensor on the device; sampled rows (the first,
    around 2^30, the last) against the oracle, for the norm-only op, the
    norm-only op with weight (four rows per wave, 2^27 workgroups) and the
    fused op (per-batch scale/shift, broadcast gate)."""
    D, T = 8, 65536
    L = (1 << 31) - 1
    info = rn.describe_launch(1, L, D, 0, False)
    assert info["grid_blocks"] == (L + info["rows_per_block"] - 1) // info["rows_per_block"]
    tiles = {k: synth.random_bf16((T, D), 31, t) for k, t in (("x", 1), ("residual", 2))}
    g = synth.random_bf16((1, D), 31, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    sc = synth.random_bf16((1, D), 31, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 31, 7, a=0.0, b=0.1)
    dg, dsc, dsh = to_dev(g), to_dev(sc), to_dev(sh)

    def tiled(k):
        t = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
        tile = to_dev(tiles[k])
        full = (L // T) * T
        t[:full].view(-1, T, D).copy_(tile.unsqueeze(0).expand(L // T, T, D))
        t[full:].copy_(tile[:L - full])
        return t

    samples = [0, (1 << 30) - 5, L - 20]

    def host_rows(k, r0, n):
        return tiles[k][np.arange(r0, r0 + n) % T]

    log("maximum rows: norm-only, %d rows" % L)
    x = tiled("x")
    y = torch.empty_like(x)
    rn.norm_scale_shift_fwd(y, x, None, None, dsc, dsh, 1, L, D, 0, (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    for r0 in samples:
        n = min(20, L - r0)
        xs = host_rows("x", r0, n)
        y_ref, _ = orc.nss(xs, None, None, sc, sh, 1, L, D, False, row0=r0, nrows=n)
        compare_outputs(to_host(y[r0:r0 + n]), y_ref, what="max rows nss at %d" % r0)
    log("maximum rows: norm-only with weight (four rows per wave)")
    w = synth.random_bf16((D,), 31, 4, a=1.0, b=0.05)
    info_w = rn.describe_launch(1, L, D, rn.RN_WEIGHT, False)
    assert info_w["rows_per_wave"] == 4
    rn.norm_scale_shift_fwd(y, x, to_dev(w), None, dsc, dsh, 1, L, D, rn.RN_WEIGHT, (BCAST, 0),
                            1e-6)
    torch.cuda.synchronize()
    for r0 in samples:
        n = min(20, L - r0)
        y_ref, _ = orc.nss(host_rows("x", r0, n), w, None, sc, sh, 1, L, D, False, row0=r0, nrows=n)
        compare_outputs(to_host(y[r0:r0 + n]), y_ref, what="max rows nss+w at %d" % r0)
    del y
    log("maximum rows: fused")
    r = tiled("residual")
    y = torch.empty_like(x)
    ro = torch.empty_like(x)
    rn.resnorm_fused_fwd(y, ro, x, r, dg, None, None, dsc, dsh, 1, L, D, rn.RN_GATE, (BCAST, 0),
                         (FRAME, 1), 1e-6)
    torch.cuda.synchronize()
    for r0 in samples:
        n = min(20, L - r0)
        y_ref, ro_ref, _ = orc.fused(host_rows("x", r0, n), host_rows("residual", r0, n), g, None,
                                     None, sc, sh, 1, L, D, False, (BCAST, 0), (FRAME, 1), 1e-6,
                                     row0=r0, nrows=n)
        compare_outputs(to_host(y[r0:r0 + n]), y_ref, to_host(ro[r0:r0 + n]), ro_ref,
                        "max rows fused at %d" % r0)
    del x, r, y, ro
    torch.cuda.empty_cache()


def test_two_dimensional_grid_ten_waves(rn, orc):
    """Ten waves per row (640-thread workgroups: per-row gate, D = 2560) over
    6,711,887 rows, just past the 6,710,886 workgroups one grid dimension can
    hold, so the launch spills into a second dimension: rows either side of
    the seam and the last rows against the oracle (five 34 GB tensors)."""
    D, T = 2560, 4096
    L = 6711887
    flags = rn.RN_GATE
    info = rn.describe_launch(1, L, D, flags, True, (ROW, 0), (BCAST, 0))
    assert info["waves_per_row"] == 10 and info["block_threads"] == 640
    seam = (2 ** 32 - 1) // 640
    assert info["grid_blocks"] > seam
    tiles = {k: synth.random_bf16((T, D), 32, t) for k, t in (("x", 1), ("residual", 2))}
    tiles["gate"] = synth.random_bf16((T, D), 32, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    sc = synth.random_bf16((1, D), 32, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 32, 7, a=0.0, b=0.1)

    def tiled(k):
        t = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
        tile = to_dev(tiles[k])
        full = (L // T) * T
        t[:full].view(-1, T, D).copy_(tile.unsqueeze(0).expand(L // T, T, D))
        t[full:].copy_(tile[:L - full])
        return t

    log("two-dimensional grid: %d rows x %d, ten waves per row" % (L, D))
    dev = {k: tiled(k) for k in ("x", "residual", "gate")}
    y = torch.empty_like(dev["x"])
    ro = torch.empty_like(dev["x"])
    rn.resnorm_fused_fwd(y, ro, dev["x"], dev["residual"], dev["gate"], None, None, to_dev(sc),
                         to_dev(sh), 1, L, D, flags, (ROW, 0), (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    for r0 in (0, seam - 3, L - 4):
        n = min(8, L - r0)
        rows = np.arange(r0, r0 + n) % T
        # a per-row gate: the sampled rows as a problem of their own (rows are
        # independent, and with broadcast scale/shift nothing else depends on r)
        y_ref, ro_ref, _ = orc.fused(tiles["x"][rows], tiles["residual"][rows], tiles["gate"][rows],
                                     None, None, sc, sh, 1, n, D, False, (ROW, 0), (BCAST, 0), 1e-6)
        compare_outputs(to_host(y[r0:r0 + n]), y_ref, to_host(ro[r0:r0 + n]), ro_ref,
                        "2D grid rows %d..%d" % (r0, r0 + n))
    del dev, y, ro
    torch.cuda.empty_cache()


def test_rescaled_statistics_ext_outputs(rn, orc):
    """Rows whose binary32 sums overflow (magnitudes 2^100 and 2^126), mixed
    with ordinary rows, with binary32 and FP8 outputs and binary32
    weight/bias, on shapes with one, two, four and ten waves per row, and on
    multi-row shapes (where a wave's consecutive rows mix the two kinds): the
    rescaled statistics and, for FP8, the row maximum that follows them in
    the same workgroup."""
    cases = [(5120, 2048, False, None, 0), (3072, 300, False, None, 0), (4096, 200, False, None, 0),
             (2560, 64, True, (ROW, 0), 0), (5120, 600, True, (BCAST, 0), 4),
             (5120, 8195, False, None, 4), (1000, 12599, False, None, 2)]
    for k, (D, L, fused, gl, aff) in enumerate(cases):
        for y_dtype in (1, 2):
            inp = _problem(1500 + k, fused, gl, aff, (BCAST, 0), 1, L, D)
            rows = np.arange(L)
            big, huge = rows % 3 == 1, rows % 7 == 3
            inp["x"][big] = (inp["x"][big] & 0x807F) | 0x7180
            inp["x"][huge] = (inp["x"][huge] & 0x807F) | 0x7E80
            if fused:
                inp["residual"][big | huge] = 0
                if gl is not None and gl[0] == ROW:
                    inp["gate"][big | huge] = 0x3F80
            flags = (rn.RN_GATE if gl is not None else 0) | \
                (rn.RN_WEIGHT | rn.RN_BIAS if aff else 0)
            info = rn.describe_launch(1, L, D, flags, fused, gl or (BCAST, 0), (BCAST, 0))
            log("rescaled statistics ext: D=%d L=%d fused=%s aff=%d y=%d W=%d K=%d" % (
                D, L, fused, aff, y_dtype, info["waves_per_row"], info["rows_per_wave"]))
            _run_inputs(rn, orc, inp, fused, False, gl, aff, (BCAST, 0), 1, L, D, y_dtype)


def test_hip_graph_lds_and_multi_row(rn, orc):
    """The LDS-staged fused kernel (binary32 weight + bias, one wave per row)
    and a multi-row norm-only kernel (bf16 weight + bias, 4 rows per wave)
    captured in one HIP graph and replayed three times with new input
    contents, eager work between replays, each replay against the oracle."""
    B, D = 1, 5120
    LA, LB = 600, 2458                        # 2458 x 5120 >= 12 Mi elements
    WB = rn.RN_WEIGHT | rn.RN_BIAS
    ia = rn.describe_launch(B, LA, D, rn.RN_GATE | WB, True, affine_dtype=rn.RN_DTYPE_F32)
    ib = rn.describe_launch(B, LB, D, WB, False)
    assert (ia["waves_per_row"], ia["rows_per_wave"]) == (1, 1)
    assert ib["rows_per_wave"] == 4

    def dev_like(a):
        dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
        return torch.empty(a.shape, dtype=dt, device="cuda")

    pa = _problem(1, True, (BCAST, 0), 4, (BCAST, 0), B, LA, D)
    pb = _problem(2, False, None, 2, (BCAST, 0), B, LB, D)
    da = {k: dev_like(v) for k, v in pa.items()}
    db = {k: dev_like(v) for k, v in pb.items()}
    ya = torch.empty((LA, D), dtype=torch.bfloat16, device="cuda")
    ra = torch.empty_like(ya)
    yb = torch.empty((LB, D), dtype=torch.bfloat16, device="cuda")

    def fill(seed):
        inps = (_problem(seed, True, (BCAST, 0), 4, (BCAST, 0), B, LA, D),
                _problem(seed + 100, False, None, 2, (BCAST, 0), B, LB, D))
        for inp, d in zip(inps, (da, db)):
            for k, v in inp.items():
                d[k].copy_(f32_dev(v) if v.dtype == np.float32 else to_dev(v))
        return inps

    def calls():
        rn.resnorm_fused_fwd_ex(ya, ra, da["x"], da["residual"], da["gate"], da["weight"],
                                da["bias"], da["scale"], da["shift"], B, LA, D, rn.RN_GATE | WB,
                                (BCAST, 0), (BCAST, 0), 1e-6, rn.RN_DTYPE_F32)
        rn.norm_scale_shift_fwd(yb, db["x"], db["weight"], db["bias"], db["scale"], db["shift"],
                                B, LB, D, WB, (BCAST, 0), 1e-6)

    fill(3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for seed in (21, 22, 23):
        a, b = fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("graph replay %d: LDS-staged fused and multi-row norm-only" % seed)
        y_ref, ro_ref, _ = orc.fused(a["x"], a["residual"], a["gate"], a["weight"], a["bias"],
                                     a["scale"], a["shift"], B, LA, D, False, (BCAST, 0), (BCAST, 0),
                                     1e-6, affine_f32=True, threads=THREADS)
        compare_outputs(to_host(ya), y_ref, to_host(ra), ro_ref, "graph replay %d fused" % seed)
        yb_ref, _ = orc.nss(b["x"], b["weight"], b["bias"], b["scale"], b["shift"], B, LB, D, False,
                            (BCAST, 0), 1e-6, threads=THREADS)
        compare_outputs(to_host(yb), yb_ref, what="graph replay %d nss" % seed)
        torch.add(da["x"], 1.0).sum().item()      # eager work between replays
