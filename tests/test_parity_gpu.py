"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Bar: residual_out bit-exact; y within max(2 bf16 ulps of the oracle's value,
1e-2) element by element.  Inputs are the seeded synthetic workloads (the
pages' shapes: sglang PR #36349, "Microbenchmark"; sglang PR #33144,
"Accuracy Tests") and small random problems spanning every specialisation,
layout and ragged row width.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (FULL_SIZE_MIN_IDENTICAL, compare_outputs, launch_workload, log,
                      require_gpu, to_dev, to_host, workload_flags)
from util import bf16_to_f64

pytestmark = pytest.mark.gpu

BCAST, ROW, FRAME = 0, 1, 2
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def rn():
    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    return rn


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _run_full(rn, orc, wl, check_rows=None, min_identical=None):
    import torch
    log("workload %s: generating inputs" % wl.name)
    inp = synth.make_inputs(wl, threads=THREADS)
    d = {k: to_dev(v) for k, v in inp.items()}
    y = torch.empty_like(d["x"])
    ro = torch.empty_like(d["x"]) if wl.op == "fused" else None
    log("workload %s: launching (B=%d L=%d D=%d)" % (wl.name, wl.B, wl.L, wl.D))
    launch_workload(rn, wl, d, y, ro)
    torch.cuda.synchronize()
    yh = to_host(y)
    roh = to_host(ro) if ro is not None else None
    del d, y, ro
    log("workload %s: oracle on %d rows x %d threads" % (wl.name, wl.R, THREADS))
    y_ref, ro_ref, _ = orc.run_workload(wl, inp, threads=THREADS)
    st = compare_outputs(yh, y_ref, roh, ro_ref, wl.name, min_identical=min_identical)
    log("workload %s: OK  %sy: max %.0f ulp where |y|>=1, max %.0f ulp where "
        "|y|>=2^-6, max abs err %.3g, %.5f%% bit-identical"
        % (wl.name, "residual_out bit-exact; " if roh is not None else "", st["ulp_ge1"], st["ulp_ge_1_64"], st["abs"], 100 * st["identical"]))
    return inp, yh, roh


@pytest.mark.parametrize("name", ["fused_ln_b1_l16_d5120", "fused_rms_w_b2_l16_d10240",
                                  "fused_ln_b2_l16_d5120", "nss_ln_b1_l16_d5120",
                                  "nss_ln_b2_l16_d5120"])
def test_small_workloads_all_rows(rn, orc, name):
    _run_full(rn, orc, synth.WORKLOADS[name])


@pytest.mark.parametrize("name", ["fused_ln_b1_l90000_d5120", "fused_rms_w_b1_l90000_d10240",
                                  "nss_ln_b1_l176400_d5120", "fused_ln_frame_b1_f49_l176400_d5120",
                                  "nss_ln_b1_l90000_d5120"])
def test_full_size_workloads_all_rows(rn, orc, name):
    """Every row of the full-size workloads, in the launch configuration the
    benchmark times, against the oracle; at most 0.05 % of y may differ in
    any bit."""
    _run_full(rn, orc, synth.WORKLOADS[name], min_identical=FULL_SIZE_MIN_IDENTICAL)


def _small_problem(seed, fused, rms, gate_layout, aff, ss_layout, B, L, D):
    R = B * L

    def rows(lay):
        return {BCAST: 1, ROW: R, FRAME: B * lay[1]}[lay[0]]

    inp = {"x": synth.random_bf16((R, D), seed, 1)}
    if fused:
        inp["residual"] = synth.random_bf16((R, D), seed, 2)
        if gate_layout is not None:
            inp["gate"] = synth.random_bf16((rows(gate_layout), D), seed, 3, dist=synth.UNIFORM,
                                            a=0.0, b=1.0)
    if aff >= 1:
        inp["weight"] = synth.random_bf16((D,), seed, 4, a=1.0, b=0.05)
    if aff >= 2:
        inp["bias"] = synth.random_bf16((D,), seed, 5, a=0.0, b=0.1)
    inp["scale"] = synth.random_bf16((rows(ss_layout), D), seed, 6, a=0.0, b=0.1)
    inp["shift"] = synth.random_bf16((rows(ss_layout), D), seed, 7, a=0.0, b=0.1)
    return inp


def _check_small(rn, orc, seed, fused, rms, gate_layout, aff, ss_layout, B, L, D):
    import torch
    inp = _small_problem(seed, fused, rms, gate_layout, aff, ss_layout, B, L, D)
    d = {k: to_dev(v) for k, v in inp.items()}
    flags = (rn.RN_RMS if rms else 0) | (rn.RN_WEIGHT if aff >= 1 else 0) | (rn.RN_BIAS if aff >= 2 else 0)
    y = torch.empty_like(d["x"])
    case = "seed=%d fused=%s rms=%s gate=%s aff=%d ss=%s B=%d L=%d D=%d" % (
        seed, fused, rms, gate_layout, aff, ss_layout, B, L, D)
    if fused:
        if gate_layout is not None:
            flags |= rn.RN_GATE
        ro = torch.empty_like(d["x"])
        rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d.get("gate"), d.get("weight"),
                             d.get("bias"), d["scale"], d["shift"], B, L, D, flags,
                             gate_layout or (BCAST, 0), ss_layout, 1e-6)
        torch.cuda.synchronize()
        y_ref, ro_ref, _ = orc.fused(inp["x"], inp["residual"], inp.get("gate"), inp.get("weight"),
                                     inp.get("bias"), inp["scale"], inp["shift"], B, L, D, rms,
                                     gate_layout or (BCAST, 0), ss_layout, 1e-6)
        compare_outputs(to_host(y), y_ref, to_host(ro), ro_ref, case)
    else:
        rn.norm_scale_shift_fwd(y, d["x"], d.get("weight"), d.get("bias"), d["scale"], d["shift"],
                                B, L, D, flags, ss_layout, 1e-6)
        torch.cuda.synchronize()
        y_ref, _ = orc.nss(inp["x"], inp.get("weight"), inp.get("bias"), inp["scale"],
                           inp["shift"], B, L, D, rms, ss_layout, 1e-6)
        compare_outputs(to_host(y), y_ref, what=case)


LAYOUTS = [(BCAST, 0), (ROW, 0), (FRAME, 3)]
WIDTHS = [8, 64, 136, 520, 1000, 4104, 5120, 8192, 8200, 10240, 16384]


@pytest.mark.parametrize("D", WIDTHS)
def test_specialisation_matrix(rn, orc, D):
    """Every flag combination (is_rms x has_gate x affine none/weight/weight+bias,
    fused and norm-only) at one row width, cycling through the layouts; B=2,
    L=6, F=3.  Widths include exact fits of each register-cache width and
    ragged rows whose tail lanes are masked."""
    log("specialisation matrix D=%d" % D)
    B, L = 2, 6
    k = 0
    for rms in (False, True):
        for aff in (0, 1, 2):
            for gate in (True, False):
                gl = LAYOUTS[k % 3] if gate else None
                sl = LAYOUTS[(k // 3 + k) % 3]
                _check_small(rn, orc, 100 + k + D, True, rms, gl, aff, sl, B, L, D)
                k += 1
            _check_small(rn, orc, 200 + k + D, False, rms, None, aff, LAYOUTS[k % 3], B, L, D)
            k += 1


def test_all_layout_pairs(rn, orc):
    """Every gate layout x scale/shift layout pair, both norms, several frame counts."""
    for rms in (False, True):
        for gl in LAYOUTS + [(FRAME, 1), (FRAME, 6)]:
            for sl in LAYOUTS + [(FRAME, 2), (FRAME, 6)]:
                _check_small(rn, orc, 7, True, rms, gl, 0, sl, 2, 6, 64)
                _check_small(rn, orc, 8, True, rms, gl, 2, sl, 3, 12, 320)


def test_residual_every_bf16_x(rn, orc):
    """residual_out for every bf16 bit pattern of x against 64 residual values
    and 16 gates (per-row gate layout): bit-exact with the oracle; NaN outputs
    compared as NaN."""
    import torch
    xs = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(11)
    res_vals = rng.integers(0, 1 << 16, 256).astype(np.uint16)
    res_vals = res_vals[(res_vals & 0x7F80) != 0x7F80][:64]
    gates = np.concatenate([np.array([0x0000, 0x3F80, 0x3F00, 0x3F40], np.uint16),
                            rng.integers(0x3C00, 0x3F80, 12).astype(np.uint16)])
    D = 1024
    X = np.tile(xs, len(res_vals) * len(gates)).reshape(-1, D)
    Rr = np.repeat(np.repeat(res_vals, len(xs)), len(gates)).reshape(-1, D)
    G = np.tile(np.repeat(gates, len(xs)), len(res_vals)).reshape(-1, D)
    R = X.shape[0]
    log("residual brute force: %d rows of %d" % (R, D))
    zeros = np.zeros((1, D), np.uint16)
    dx, dr, dg, dz = to_dev(X), to_dev(Rr), to_dev(G), to_dev(zeros)
    y = torch.empty_like(dx)
    ro = torch.empty_like(dx)
    rn.resnorm_fused_fwd(y, ro, dx, dr, dg, None, None, dz, dz, 1, R, D, rn.RN_GATE,
                         (ROW, 0), (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    got = to_host(ro)
    ref = orc.residual(Rr, G, X)
    gnan = (got & 0x7FFF) > 0x7F80
    rnan = (ref & 0x7FFF) > 0x7F80
    bad = (gnan != rnan) | (~gnan & (got != ref))
    assert not bad.any(), "x %04x res %04x gate %04x: gpu %04x oracle %04x" % (
        X[bad][0], Rr[bad][0], G[bad][0], got[bad][0], ref[bad][0])


def test_residual_products_below_the_normal_range(rn, orc):
    """residual_out for every bf16 x against residuals of either sign at and
    near zero and gates down to 2^-33, where gate * x falls below the binary32
    normal range or underflows: bit-exact with the oracle's one rounding of
    the exact sum, including the -0 of a product that underflows below a +0
    residual."""
    import torch
    xs = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    res_vals = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0040, 0x807F, 0x0080, 0x8080,
                         0x0100, 0x3F80], np.uint16)
    gates = np.array([0x3580, 0xB580, 0x2F00, 0xAF00, 0x3A80, 0x37C0, 0x3F80, 0x0001], np.uint16)
    D = 1024
    X = np.tile(xs, len(res_vals) * len(gates)).reshape(-1, D)
    Rr = np.repeat(np.repeat(res_vals, len(xs)), len(gates)).reshape(-1, D)
    G = np.tile(np.repeat(gates, len(xs)), len(res_vals)).reshape(-1, D)
    R = X.shape[0]
    log("residual below the normal range: %d rows of %d" % (R, D))
    zeros = np.zeros((1, D), np.uint16)
    dx, dr, dg, dz = to_dev(X), to_dev(Rr), to_dev(G), to_dev(zeros)
    y = torch.empty_like(dx)
    ro = torch.empty_like(dx)
    rn.resnorm_fused_fwd(y, ro, dx, dr, dg, None, None, dz, dz, 1, R, D, rn.RN_GATE,
                         (ROW, 0), (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    got = to_host(ro)
    ref = orc.residual(Rr, G, X)
    gnan = (got & 0x7FFF) > 0x7F80
    rnan = (ref & 0x7FFF) > 0x7F80
    bad = (gnan != rnan) | (~gnan & (got != ref))
    assert not bad.any(), "x %04x res %04x gate %04x: gpu %04x oracle %04x (%d)" % (
        X[bad][0], Rr[bad][0], G[bad][0], got[bad][0], ref[bad][0], int(bad.sum()))
    assert ((Rr == 0x0000) & (ref == 0x8000)).any()     # the underflowed -0 case occurs


def test_determinism_permutation_and_norm_of_residual(rn, orc):
    """Reruns are bitwise identical; permuting rows permutes the outputs bit-
    exactly (broadcast layouts); the fused y equals the norm-only op applied to
    the fused op's residual_out, bit-exactly."""
    import torch
    B, L, D = 1, 512, 5120
    inp = _small_problem(21, True, False, (BCAST, 0), 0, (BCAST, 0), B, L, D)
    d = {k: to_dev(v) for k, v in inp.items()}

    def run(dd):
        y = torch.empty_like(dd["x"])
        ro = torch.empty_like(dd["x"])
        rn.resnorm_fused_fwd(y, ro, dd["x"], dd["residual"], dd["gate"], None, None, dd["scale"],
                             dd["shift"], B, L, D, rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6)
        return y, ro

    y1, ro1 = run(d)
    y2, ro2 = run(d)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(ro1.view(torch.int16), ro2.view(torch.int16))
    perm = np.random.default_rng(3).permutation(L)
    dp = dict(d)
    dp["x"] = to_dev(inp["x"][perm])
    dp["residual"] = to_dev(inp["residual"][perm])
    y3, ro3 = run(dp)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(y3), to_host(y1)[perm])
    assert np.array_equal(to_host(ro3), to_host(ro1)[perm])
    yn = torch.empty_like(y1)
    rn.norm_scale_shift_fwd(yn, ro1, None, None, d["scale"], d["shift"], B, L, D, 0, (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(yn.view(torch.int16), y1.view(torch.int16))


def test_in_place_aliasing(rn, orc):
    """y == x and residual_out == residual give the out-of-place results."""
    import torch
    B, L, D = 2, 40, 10240
    inp = _small_problem(31, True, True, (BCAST, 0), 1, (ROW, 0), B, L, D)
    d = {k: to_dev(v) for k, v in inp.items()}
    flags = rn.RN_RMS | rn.RN_GATE | rn.RN_WEIGHT
    y = torch.empty_like(d["x"])
    ro = torch.empty_like(d["x"])
    rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d["gate"], d["weight"], None, d["scale"],
                         d["shift"], B, L, D, flags, (BCAST, 0), (ROW, 0), 1e-6)
    xi, ri = d["x"].clone(), d["residual"].clone()
    rn.resnorm_fused_fwd(xi, ri, xi, ri, d["gate"], d["weight"], None, d["scale"], d["shift"],
                         B, L, D, flags, (BCAST, 0), (ROW, 0), 1e-6)
    xn = d["x"].clone()
    yn = torch.empty_like(xn)
    rn.norm_scale_shift_fwd(yn, xn, d["weight"], None, d["scale"], d["shift"], B, L, D,
                            rn.RN_RMS | rn.RN_WEIGHT, (ROW, 0), 1e-6)
    rn.norm_scale_shift_fwd(xn, xn, d["weight"], None, d["scale"], d["shift"], B, L, D,
                            rn.RN_RMS | rn.RN_WEIGHT, (ROW, 0), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(xi.view(torch.int16), y.view(torch.int16))
    assert torch.equal(ri.view(torch.int16), ro.view(torch.int16))
    assert torch.equal(xn.view(torch.int16), yn.view(torch.int16))


@pytest.mark.parametrize("D", [8, 1000, 8200])
def test_ragged_rows_leave_neighbours_untouched(rn, orc, D):
    """Outputs are written only inside their rows: guard rows after the last
    row (and the whole buffers beyond it) keep their contents, for row widths
    whose tail lanes are masked by the per-row buffer range."""
    import torch
    B, L = 1, 7
    inp = _small_problem(41, True, False, (BCAST, 0), 0, (BCAST, 0), B, L, D)
    d = {k: to_dev(v) for k, v in inp.items()}
    guard = 5
    y_buf = torch.full((L + guard, D), 3.0, dtype=torch.bfloat16, device="cuda")
    ro_buf = torch.full((L + guard, D), -3.0, dtype=torch.bfloat16, device="cuda")
    rn.resnorm_fused_fwd(y_buf[:L], ro_buf[:L], d["x"], d["residual"], d["gate"], None, None,
                         d["scale"], d["shift"], B, L, D, rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    assert torch.all(y_buf[L:] == 3.0) and torch.all(ro_buf[L:] == -3.0)
    y_ref, ro_ref, _ = orc.fused(inp["x"], inp["residual"], inp["gate"], None, None, inp["scale"],
                                 inp["shift"], B, L, D, False)
    compare_outputs(to_host(y_buf[:L]), y_ref, to_host(ro_buf[:L]), ro_ref, "ragged D=%d" % D)


def test_empty_and_side_stream(rn, orc):
    """B*L = 0 enqueues nothing; a call on a non-default stream is ordered on it."""
    import torch
    D = 256
    z = torch.zeros((1, D), dtype=torch.bfloat16, device="cuda")
    y = torch.full((4, D), 7.0, dtype=torch.bfloat16, device="cuda")
    rn.norm_scale_shift_fwd(y, z, None, None, z, z, 0, 4, D, 0, (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    inp = _small_problem(51, False, False, None, 0, (BCAST, 0), 1, 64, D)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d = {k: to_dev(v) for k, v in inp.items()}
        y = torch.empty_like(d["x"])
        rn.norm_scale_shift_fwd(y, d["x"], None, None, d["scale"], d["shift"], 1, 64, D, 0,
                                (BCAST, 0), 1e-6, stream=s)
    s.synchronize()
    y_ref, _ = orc.nss(inp["x"], None, None, inp["scale"], inp["shift"], 1, 64, D, False)
    compare_outputs(to_host(y), y_ref, what="side stream")


def test_default_stream_is_torchs_current_stream(rn, orc):
    """Without stream=, a call goes to torch's current stream of the operands'
    device: the same handle torch reports, outside and inside a
    torch.cuda.stream() context, and the call made there is ordered on it."""
    import torch
    assert rn._stream(None, 0) == torch.cuda.current_stream(0).cuda_stream
    assert rn._stream(None) == torch.cuda.current_stream().cuda_stream
    D = 512
    inp = _small_problem(52, False, False, None, 0, (BCAST, 0), 1, 64, D)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert rn._stream(None, 0) == s.cuda_stream != torch.cuda.default_stream(0).cuda_stream
        assert rn._stream(None) == s.cuda_stream
        d = {k: to_dev(v) for k, v in inp.items()}
        y = torch.empty_like(d["x"])
        rn.norm_scale_shift_fwd(y, d["x"], None, None, d["scale"], d["shift"], 1, 64, D, 0,
                                (BCAST, 0), 1e-6)
    s.synchronize()
    y_ref, _ = orc.nss(inp["x"], None, None, inp["scale"], inp["shift"], 1, 64, D, False)
    compare_outputs(to_host(y), y_ref, what="current stream")


def test_binding_refuses_device_tensors_it_cannot_pass(rn):
    """The binding's checks on GPU tensors, before any library call: element
    type, contiguity, one device for all operands; a refused call leaves the
    outputs untouched."""
    import torch
    D, L = 512, 8
    dev = torch.device("cuda:0")
    x = torch.randn((L, D), device=dev).to(torch.bfloat16)
    row = torch.zeros((1, D), dtype=torch.bfloat16, device=dev)
    y = torch.full((L, D), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(TypeError, match="y must be torch.bfloat16"):
        rn.norm_scale_shift_fwd(y.to(torch.float16), x, None, None, row, row, 1, L, D, 0)
    with pytest.raises(ValueError, match="x must be contiguous"):
        rn.norm_scale_shift_fwd(y, torch.randn((D, L), device=dev).to(torch.bfloat16).t(), None,
                                None, row, row, 1, L, D, 0)
    with pytest.raises(ValueError, match="shift is on cpu but other operands are on cuda:0"):
        rn.norm_scale_shift_fwd(y, x, None, None, row, row.cpu(), 1, L, D, 0)
    with pytest.raises(TypeError, match="weight must be torch.float32"):
        rn.norm_scale_shift_fwd_ex(y, x, row.view(-1), None, row, row, 1, L, D, rn.RN_WEIGHT,
                                   affine_dtype=rn.RN_DTYPE_F32)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # int addresses pass through to the library, which checks them itself
    rn.norm_scale_shift_fwd(y.data_ptr(), x, None, None, row, row, 1, L, D, 0)
    torch.cuda.synchronize()
    assert not bool((y == 7.0).all())


def test_repeated_calls_and_prepared_calls(rn, orc):
    """The library keeps each thread's last validated call with its launch
    plan, and rn.prepare checks a call once: alternating two problems (A, B,
    A, B) must launch each with its own arguments every time, a repeated
    identical call must pick up new input contents, and a prepared call must
    give the direct call's bits."""
    import torch
    D = 5120
    probs = []
    for seed, L in ((61, 96), (62, 40)):
        inp = _small_problem(seed, True, False, (BCAST, 0), 0, (BCAST, 0), 1, L, D)
        d = {k: to_dev(v) for k, v in inp.items()}
        y, ro = torch.empty_like(d["x"]), torch.empty_like(d["x"])
        ref = orc.fused(inp["x"], inp["residual"], inp["gate"], None, None, inp["scale"],
                        inp["shift"], 1, L, D, False, (BCAST, 0), (BCAST, 0), 1e-6)
        probs.append((inp, d, y, ro, L, ref))

    def call(p):
        inp, d, y, ro, L, ref = p
        rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d["gate"], None, None, d["scale"],
                             d["shift"], 1, L, D, rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6)

    for k in range(4):
        p = probs[k % 2]
        p[2].fill_(float("nan"))
        p[3].fill_(float("nan"))
        call(p)
        torch.cuda.synchronize()
        compare_outputs(to_host(p[2]), p[5][0], to_host(p[3]), p[5][1], "alternating call %d" % k)
    # the same call again after new inputs were written into the same buffers
    inp, d, y, ro, L, _ = probs[0]
    x2 = synth.random_bf16((L, D), 63, 1)
    d["x"].copy_(to_dev(x2))
    call(probs[0])
    call(probs[0])
    torch.cuda.synchronize()
    ref2 = orc.fused(x2, inp["residual"], inp["gate"], None, None, inp["scale"], inp["shift"], 1, L,
                     D, False, (BCAST, 0), (BCAST, 0), 1e-6)
    compare_outputs(to_host(y), ref2[0], to_host(ro), ref2[1], "repeat after new inputs")
    # a prepared call gives the direct call's bits, also after new inputs
    y_direct = y.clone()
    y.fill_(float("nan"))
    launch = rn.prepare(rn.resnorm_fused_fwd, y, ro, d["x"], d["residual"], d["gate"], None, None,
                        d["scale"], d["shift"], 1, L, D, rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6)
    launch()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_direct.view(torch.int16))
    d["x"].copy_(to_dev(inp["x"]))
    launch()
    torch.cuda.synchronize()
    compare_outputs(to_host(y), probs[0][5][0], to_host(ro), probs[0][5][1], "prepared call")
    # the _ex form through prepare: binary32 output against the oracle's binary32
    # y, at the binary32-output tests' bound (2^-14 relative, absolute below 1)
    y32 = torch.empty((L, D), dtype=torch.float32, device="cuda")
    launch32 = rn.prepare(rn.norm_scale_shift_fwd_ex, y32, d["x"], None, None, d["scale"], d["shift"],
                          1, L, D, 0, (BCAST, 0), 1e-6, y_dtype=rn.RN_DTYPE_F32)
    launch32()
    torch.cuda.synchronize()
    ref32 = orc.nss(inp["x"], None, None, inp["scale"], inp["shift"], 1, L, D, False, (BCAST, 0),
                    1e-6, y_dtype=oracle.Y_F32)[0]
    got = y32.cpu().numpy().astype(np.float64).ravel()
    want = np.asarray(ref32, dtype=np.float64).ravel()
    assert np.all(np.abs(got - want) <= 2.0 ** -14 * np.maximum(1.0, np.abs(want)))


def test_gpu_norm_invariants(rn, orc):
    """Pure-norm GPU outputs (scale = shift = 0, no affine) at D >= 512.

    The exact normalised row t has mean 0 and variance 1 (RMS 1) up to the eps
    term; the oracle pins that on t to 1e-3.  A bf16 output y differs from t by
    at most half an ulp, i.e. |y - t| <= 2^-8 |t|, so its row variance can move
    by up to (2 * 2^-8 + 2^-16) * mean(t^2) and its mean by 2^-8 * mean|t| --
    and it does, systematically, because y tends to stay on the input's own bf16
    grid when the row scale is close to 1.  So the GPU rows are held to those
    bounds (plus 1e-3), and their moments must also agree with the moments of
    the oracle's bf16 rows to 1e-3."""
    import torch
    q = 2.0 ** -8
    for D in (512, 5120, 10240):
        L = 64
        x = synth.random_bf16((L, D), 61, 1)
        z = np.zeros((1, D), np.uint16)
        dx, dz = to_dev(x), to_dev(z)
        for rms in (False, True):
            y = torch.empty_like(dx)
            rn.norm_scale_shift_fwd(y, dx, None, None, dz, dz, 1, L, D,
                                    rn.RN_RMS if rms else 0, (BCAST, 0), 1e-6)
            torch.cuda.synchronize()
            t = bf16_to_f64(to_host(y))
            ref = bf16_to_f64(orc.nss(x, None, None, z, z, 1, L, D, rms)[0])
            if rms:
                ms = (t * t).mean(1)
                assert np.all(np.abs(ms - 1) <= 2 * q + q * q + 1e-3)
                assert np.all(np.abs(ms - (ref * ref).mean(1)) <= 1e-3)
            else:
                assert np.all(np.abs(t.mean(1)) <= q * np.abs(t).mean(1) + 1e-3)
                assert np.all(np.abs(t.var(1) - 1) <= 2 * q + q * q + 1e-3)
                assert np.all(np.abs(t.mean(1) - ref.mean(1)) <= 1e-3)
                assert np.all(np.abs(t.var(1) - ref.var(1)) <= 1e-3)


def test_mean_offset_rows(rn, orc):
    """Rows with a large common offset (|mean| >> std) stay within tolerance: the
    kernel centres the register-resident row before squaring."""
    import torch
    D, L = 5120, 32
    base = synth.random_bf16((L, D), 71, 1)
    xf = (base.astype(np.uint32) << 16).view(np.float32) + np.float32(300.0)
    x = ((xf.view(np.uint32) + 0x7FFF + ((xf.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    sc = synth.random_bf16((1, D), 71, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 71, 7, a=0.0, b=0.1)
    y = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    rn.norm_scale_shift_fwd(y, to_dev(x), None, None, to_dev(sc), to_dev(sh), 1, L, D, 0,
                            (BCAST, 0), 1e-6)
    torch.cuda.synchronize()
    y_ref, _ = orc.nss(x, None, None, sc, sh, 1, L, D, False)
    compare_outputs(to_host(y), y_ref, what="mean offset 300")




# a few hundred rows, a mid-size and a large problem, and odd counts that
# reach the multi-row threshold (12 Mi elements) from D = 1536 and D = 512
SHAPE_ROWS = ((2, 263), (2, 600), (2, 1031), (1, 8195), (1, 24579))


def _shape_cases(rn):
    """One (B, L, D, fused, flags, scale/shift layout) per compiled (waves per
    row, vectors per lane, rows per wave, rows per workgroup) shape, at the
    first row count and row width that select it."""
    seen = {}
    flag_sets = [(False, 0), (True, rn.RN_GATE), (True, rn.RN_GATE | rn.RN_WEIGHT),
                 (True, rn.RN_GATE | rn.RN_WEIGHT | rn.RN_BIAS), (False, rn.RN_WEIGHT | rn.RN_BIAS)]
    for B, L in SHAPE_ROWS:
        for D in range(8, 16385, 8):
            for fused, flags in flag_sets:
                for sl in ((BCAST, 0), (ROW, 0)):
                    gl = (FRAME, 1) if flags & rn.RN_GATE else (BCAST, 0)
                    i = rn.describe_launch(B, L, D, flags, fused, gl, sl)
                    key = (i["waves_per_row"], i["vec_per_lane"], i["rows_per_wave"], i["rows_per_block"])
                    if key not in seen:
                        seen[key] = (B, L, D, fused, flags, sl)
    return seen


def test_every_compiled_shape(rn, orc):
    """Every compiled (waves per row, vectors per lane, rows per wave, rows per
    workgroup) shape the planner can pick, at the first row width that selects it (a ragged
    row for most), with odd L (so the last workgroup of a shape with several
    rows per workgroup is partly empty)."""
    cases = _shape_cases(rn)
    assert len(cases) == 37, sorted(cases)
    for (w, vpt, k, rpb), (B, L, D, fused, flags, sl) in sorted(cases.items()):
        log("shape W=%d VPT=%d K=%d rows/workgroup %d via B=%d L=%d D=%d fused=%s flags=%d ss=%s" % (
            w, vpt, k, rpb, B, L, D, fused, flags, sl))
        aff = 2 if flags & rn.RN_BIAS else (1 if flags & rn.RN_WEIGHT else 0)
        gl = (FRAME, 1) if flags & rn.RN_GATE else None
        for rms in (False, True):
            _check_small(rn, orc, 300 + w * 16 + vpt + k, fused, rms, gl, aff, sl, B, L, D)


def test_hip_graph_capture_and_replay(rn, orc):
    """The entry points can be captured in a HIP graph (torch.cuda.CUDAGraph):
    three calls (fused, norm-only, FP8 output) captured once and replayed with
    new input contents each time, each replay checked against the oracle, with
    eager work and synchronisation between replays."""
    import torch
    B, L, D = 1, 48, 5120
    shapes = {"x": (L, D), "residual": (L, D), "gate": (1, D), "scale": (1, D), "shift": (1, D)}
    bufs = {k: torch.empty(s, dtype=torch.bfloat16, device="cuda") for k, s in shapes.items()}
    y = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty_like(y)
    yn = torch.empty_like(y)
    y8 = torch.empty((L, D), dtype=torch.float8_e4m3fn, device="cuda")
    ys = torch.empty((L,), dtype=torch.float32, device="cuda")

    def calls():
        rn.resnorm_fused_fwd(y, ro, bufs["x"], bufs["residual"], bufs["gate"], None, None,
                             bufs["scale"], bufs["shift"], B, L, D, rn.RN_GATE, (BCAST, 0),
                             (BCAST, 0), 1e-6)
        rn.norm_scale_shift_fwd(yn, ro, None, None, bufs["scale"], bufs["shift"], B, L, D, 0,
                                (BCAST, 0), 1e-6)
        rn.resnorm_fused_fwd_ex(y8, ro, bufs["x"], ro, bufs["gate"], None, None, bufs["scale"],
                                bufs["shift"], B, L, D, rn.RN_GATE, (BCAST, 0), (BCAST, 0), 1e-6,
                                y_dtype=rn.RN_DTYPE_FP8_E4M3, y_scale=ys)

    def fill(seed):
        inp = _small_problem(seed, True, False, (BCAST, 0), 0, (BCAST, 0), B, L, D)
        for k in shapes:
            bufs[k].copy_(to_dev(inp[k]))
        return inp

    fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for seed in (11, 12, 13):
        inp = fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, ro_ref, _ = orc.fused(inp["x"], inp["residual"], inp["gate"], None, None,
                                     inp["scale"], inp["shift"], B, L, D, False)
        compare_outputs(to_host(y), y_ref, None, None, "graph replay %d y" % seed)
        yn_ref, _ = orc.nss(ro_ref, None, None, inp["scale"], inp["shift"], B, L, D, False)
        compare_outputs(to_host(yn), yn_ref, what="graph replay %d nss" % seed)
        # the third call read residual_out in place of the residual (aliasing)
        q, _, _, s8 = orc.fused(inp["x"], ro_ref, inp["gate"], None, None, inp["scale"],
                                inp["shift"], B, L, D, False, y_dtype=2)
        np.testing.assert_allclose(ys.cpu().numpy(), s8, rtol=2.0 ** -20)
        same = np.mean(y8.view(torch.uint8).cpu().numpy() == q)
        assert same > 0.999, same
        # eager work between replays
        torch.add(bufs["x"], 1.0).sum().item()


def test_degenerate_rows(rn, orc):
    """Rows with an Inf or NaN element, residual sums that overflow binary32 to
    Inf, all-zero rows, rows of bf16 subnormals, constant rows and rows of
    large magnitude (2^50; 2^100 and 2^126 with random signs, whose binary32
    sums overflow and take the rescaled path; the bf16 maximum, constant),
    through both ops and both norms: residual_out bit-exact (NaN compared as
    NaN); y NaN exactly where the oracle's is, equal infinities, and the
    usual bar on every finite element."""
    import torch
    D, L = 1024, 10
    x = synth.random_bf16((L, D), 77, 1)
    r = synth.random_bf16((L, D), 77, 2)
    x[0, 5] = 0x7F80                      # +Inf in x
    x[1, 7] = 0x7FC0                      # NaN in x
    r[2, 3] = 0xFF80                      # -Inf in the residual
    x[3, :] = 0x7F7F                      # bf16 max: residual + x overflows to +Inf
    r[3, :] = 0x7F7F
    x[4, :] = 0
    r[4, :] = 0
    x[5, :] = np.arange(D, dtype=np.uint16) % 0x7F + 1   # positive bf16 subnormals
    r[5, :] = 0
    x[6, :] = 0x3FC0                      # 1.5 everywhere
    r[6, :] = 0
    x[7, :] = (x[7, :] & 0x807F) | 0x5880  # random signs and mantissas, magnitude 2^50
    r[7, :] = 0
    x[8, :] = (x[8, :] & 0x807F) | 0x7180  # magnitude 2^100: squares overflow binary32
    r[8, :] = 0
    x[9, :] = (x[9, :] & 0x807F) | 0x7E80  # magnitude 2^126: sums overflow too
    r[9, :] = 0
    g = synth.random_bf16((1, D), 77, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    g[0, :] = 0x3F80                      # gate 1: rows keep their designed sums
    sc = synth.random_bf16((1, D), 77, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), 77, 7, a=0.0, b=0.1)
    d = {k: to_dev(v) for k, v in (("x", x), ("r", r), ("g", g), ("sc", sc), ("sh", sh))}

    def same(got, ref, what):
        gnan = (got & 0x7FFF) > 0x7F80
        rnan = (ref & 0x7FFF) > 0x7F80
        assert np.array_equal(gnan, rnan), "%s: NaN positions differ at %s" % (
            what, np.argwhere(gnan != rnan)[:4].tolist())
        inf_r = (ref & 0x7FFF) == 0x7F80
        assert np.array_equal(got[inf_r], ref[inf_r]), what + ": infinities differ"
        fin = ~rnan & ~inf_r
        compare_outputs(got[fin], ref[fin], what=what)

    for rms in (False, True):
        flags = (rn.RN_RMS if rms else 0) | rn.RN_GATE
        y = torch.empty_like(d["x"])
        ro = torch.empty_like(d["x"])
        rn.resnorm_fused_fwd(y, ro, d["x"], d["r"], d["g"], None, None, d["sc"], d["sh"], 1, L, D,
                             flags, (BCAST, 0), (BCAST, 0), 1e-6)
        torch.cuda.synchronize()
        y_ref, ro_ref, _ = orc.fused(x, r, g, None, None, sc, sh, 1, L, D, rms)
        same(to_host(ro), ro_ref, "fused rms=%s residual_out" % rms)
        same(to_host(y), y_ref, "fused rms=%s y" % rms)
        assert (ro_ref[3] == 0x7F80).all()
        yn = torch.empty_like(d["x"])
        rn.norm_scale_shift_fwd(yn, d["x"], None, None, d["sc"], d["sh"], 1, L, D,
                                rn.RN_RMS if rms else 0, (BCAST, 0), 1e-6)
        torch.cuda.synchronize()
        yn_ref, _ = orc.nss(x, None, None, sc, sh, 1, L, D, rms)
        same(to_host(yn), yn_ref, "norm-only rms=%s y" % rms)
        assert not np.isnan(bf16_to_f64(yn_ref[[3, 8, 9]])).any()


def test_rescaled_statistics_every_wave_count(rn, orc):
    """Rows of magnitude 2^100 and 2^126 (random signs and mantissas), whose
    binary32 sums overflow, interleaved with ordinary rows, for one, two
    (two rows per workgroup: an overflowing row next to an ordinary one),
    four and ten waves per row, both norms, fused and norm-only: every row
    against the oracle."""
    import torch
    cases = [(5120, 2048, False, None), (3072, 300, False, None), (4096, 200, False, None),
             (2560, 64, True, (ROW, 0))]
    for D, L, fused, gl in cases:
        x = synth.random_bf16((L, D), 90 + D, 1)
        r = synth.random_bf16((L, D), 90 + D, 2)
        rows = np.arange(L)
        big = rows % 3 == 1
        huge = rows % 7 == 3
        x[big] = (x[big] & 0x807F) | 0x7180
        x[huge] = (x[huge] & 0x807F) | 0x7E80
        r[big | huge] = 0
        g = synth.random_bf16((L if gl else 1, D), 90 + D, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
        if gl:
            g[big | huge] = 0x3F80                # gate 1: residual_out = x on those rows
        sc = synth.random_bf16((1, D), 90 + D, 6, a=0.0, b=0.1)
        sh = synth.random_bf16((1, D), 90 + D, 7, a=0.0, b=0.1)
        d = {k: to_dev(v) for k, v in (("x", x), ("r", r), ("g", g), ("sc", sc), ("sh", sh))}
        for rms in (False, True):
            flags = rn.RN_RMS if rms else 0
            if fused:
                flags |= rn.RN_GATE
            info = rn.describe_launch(1, L, D, flags, fused, gl or (BCAST, 0), (BCAST, 0))
            what = "D=%d L=%d fused=%s rms=%s W=%d RPB=%d" % (D, L, fused, rms, info["waves_per_row"],
                                                             info["rows_per_block"])
            log("rescaled statistics: " + what)
            y = torch.empty_like(d["x"])
            if fused:
                ro = torch.empty_like(d["x"])
                rn.resnorm_fused_fwd(y, ro, d["x"], d["r"], d["g"], None, None, d["sc"], d["sh"], 1,
                                     L, D, flags, gl, (BCAST, 0), 1e-6)
                torch.cuda.synchronize()
                y_ref, ro_ref, _ = orc.fused(x, r, g, None, None, sc, sh, 1, L, D, rms, gl,
                                             (BCAST, 0), 1e-6)
                compare_outputs(to_host(y), y_ref, to_host(ro), ro_ref, what)
            else:
                rn.norm_scale_shift_fwd(y, d["x"], None, None, d["sc"], d["sh"], 1, L, D, flags,
                                        (BCAST, 0), 1e-6)
                torch.cuda.synchronize()
                y_ref, _ = orc.nss(x, None, None, sc, sh, 1, L, D, rms)
                compare_outputs(to_host(y), y_ref, what=what)
