"""Pins of the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something the pages or the mathematics fix: a library routine
(torch's CPU bf16 cast, torch.nn.functional.layer_norm / rms_norm in float64),
a closed form, an exact special case, an independent brute-force evaluator, or
an invariant.  They are plain functions so that the mutation test can run the
same pins against deliberately broken builds of the oracle.

Where the readings come from (the pages never print the formula):
  * operand order residual, x, gate, weight, bias, scale, shift and the names
    of the two ops: sglang PR #36349, "Microbenchmark" (reproduction snippet);
  * eps = 1e-6 and broadcast operands as one dense (1, C) row: sglang
    PR #33144, "Modifications";
  * per-row scale/shift and the 4D per-frame layout: sglang PR #33144,
    "Modifications" and "Accuracy Tests";
  * frame-major token order (49 frames x 3600 tokens): sglang PR #36349,
    "Microbenchmark".
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from util import bf16_of_exact, bf16_to_f32, bf16_to_f64, near_bf16_tie, nearest_bf16

BCAST, ROW, FRAME = 0, 1, 2


def _zeros(rows, D):
    return np.zeros((rows, D), dtype=np.uint16)


def _const(rows, D, v):
    return np.full((rows, D), bf16_of_exact(v), dtype=np.uint16)


def _bits(values):
    return np.array([bf16_of_exact(float(v)) for v in np.ravel(values)],
                    dtype=np.uint16).reshape(np.shape(values))


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _nss_t(o, x, D, is_rms, eps, scale=None, shift=None, weight=None, bias=None,
           ss_layout=(BCAST, 0), B=1):
    rows = x.shape[0]
    sc = _zeros(1, D) if scale is None else scale
    sh = _zeros(1, D) if shift is None else shift
    return o.nss(x, weight, bias, sc, sh, B, rows // B, D, is_rms, ss_layout, eps, want_t=True)


# --------------------------------------------------------------------------- rounding

def pin_round_f32_vs_torch(o, stride: int = 1, threads: int = 8):
    """binary32 -> bf16 (nearest, ties to even) equals torch's CPU cast on every
    binary32 bit pattern (stride 1 = all 2^32; NaN compared as NaN)."""
    chunk = 1 << 26
    if stride == 1:
        starts = range(0, 1 << 32, chunk)
    else:
        starts = [0]
    from concurrent.futures import ThreadPoolExecutor

    def one(s0):
        if stride == 1:
            bits = np.arange(s0, s0 + chunk, dtype=np.uint64).astype(np.uint32)
        else:
            hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
            lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF,
                             0x4000, 0xC000], dtype=np.uint32)
            extra = np.arange(0, 1 << 32, stride, dtype=np.uint64).astype(np.uint32)
            bits = np.concatenate([(hi[:, None] | lows[None, :]).ravel(), extra])
        f = bits.view(np.float32)
        got = o.f32_to_bf16(f)
        ref = _torch_bf16_bits(f)
        nan = np.isnan(f)
        bad = (got != ref) & ~nan
        bad |= nan & ((got & 0x7FFF) <= 0x7F80)
        if bad.any():
            i = int(np.argmax(bad))
            return "f32 bits %08x: oracle %04x torch %04x" % (bits[i], got[i], ref[i])
        return None

    with ThreadPoolExecutor(max_workers=threads) as ex:
        for msg in ex.map(one, list(starts)):
            assert msg is None, msg


def pin_round_f64(o, n: int = 200000, seed: int = 1):
    """binary64 -> bf16 equals an independent nearest-value search over the table
    of all finite bf16 values, on random magnitudes over the whole range, on
    exact midpoints (ties to even), just above/below them, at the overflow
    boundary and in the subnormal range."""
    rng = np.random.default_rng(seed)
    t = rng.standard_normal(n) * np.exp2(rng.integers(-140, 129, n).astype(np.float64))
    # exact midpoints between neighbouring finite bf16 values, both signs
    b = rng.integers(0, 0x7F7F, n // 4).astype(np.uint16)
    lo = bf16_to_f64(b)
    hi = bf16_to_f64(b + 1)
    mid = (lo + hi) / 2
    t = np.concatenate([t, mid, -mid, np.nextafter(mid, np.inf), np.nextafter(mid, 0),
                        [0.0, -0.0, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -135,
                         float(np.nextafter(2.0 ** -134, 1)),
                         (bf16_to_f64(np.array([0x7F7F]))[0] + 2.0 ** 128) / 2,
                         float(np.nextafter((bf16_to_f64(np.array([0x7F7F]))[0] + 2.0 ** 128) / 2, 0)),
                         2.0 ** 128, -2.0 ** 129, np.inf, -np.inf]])
    got = o.f64_to_bf16(t)
    ref = nearest_bf16(t)
    bad = got != ref
    assert not bad.any(), "t=%r oracle %04x table %04x" % (
        t[np.argmax(bad)], got[np.argmax(bad)], ref[np.argmax(bad)])
    assert o.f64_to_bf16(np.array([np.nan]))[0] == 0x7FC0


# --------------------------------------------------------------------------- residual

def _residual_grid(n_res: int, seed: int):
    special = [0.0, 1.0, -1.0, 0.5, -2.0, 3.0, 2.0 ** -10, -7.25, 2.0 ** 16, -2.0 ** 100,
               2.0 ** -127, -2.0 ** -133]
    rng = np.random.default_rng(seed)
    vals = _bits(special).tolist()
    rand = rng.integers(0, 1 << 16, 4 * n_res).astype(np.uint16)
    rand = rand[((rand & 0x7F80) != 0x7F80)][: max(0, n_res - len(vals))]
    return np.array(vals + rand.tolist(), dtype=np.uint16)[:n_res]


def pin_residual_vs_torch(o, n_res: int = 64, n_gate: int = 16, seed: int = 2):
    """residual_out = bf16(f32(res) + f32(gate) * f32(x)) equals torch's
    (res.float() + gate.float() * x.float()).to(bfloat16) for every bf16 x
    against a grid of residuals and gates (NaN compared as NaN)."""
    xs = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    res = _residual_grid(n_res, seed)
    rng = np.random.default_rng(seed + 1)
    gates = np.concatenate([_bits([0.0, 1.0, 0.5, 0.75]),
                            rng.integers(0x3C00, 0x3F80, n_gate - 4).astype(np.uint16)])
    X = np.broadcast_to(xs[None, :], (len(res), len(xs)))
    Rr = np.broadcast_to(res[:, None], X.shape)
    xf = torch.from_numpy(bf16_to_f32(X).copy())
    rf = torch.from_numpy(bf16_to_f32(Rr).copy())
    for g in gates:
        G = np.full(X.shape, g, dtype=np.uint16)
        got = o.residual(Rr, G, X)
        gf = float(bf16_to_f32(np.array([g]))[0])
        ref = (rf + gf * xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = (got & 0x7FFF) > 0x7F80
        rnan = (ref & 0x7FFF) > 0x7F80
        bad = (nan != rnan) | (~nan & (got != ref))
        assert not bad.any(), "gate %04x: x %04x res %04x: oracle %04x torch %04x" % (
            g, X[bad][0], Rr[bad][0], got[bad][0], ref[bad][0])
    # no gate == gate 1
    got1 = o.residual(Rr, np.full(X.shape, 0x3F80, np.uint16), X)
    got0 = o.residual(Rr, None, X)
    assert np.array_equal(got1, got0)


def _f32_nearest(q, zero_negative: bool) -> float:
    """The binary32 value nearest the rational q, ties to the even
    significand, with gradual underflow (quantum 2^-149 below 2^-126); a
    result that rounds to zero keeps the sign of q, and q = 0 gives -0 only
    when zero_negative."""
    from fractions import Fraction
    if q == 0:
        return -0.0 if zero_negative else 0.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    m = n.numerator // n.denominator
    rem = n - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    v = float(m * quantum)
    return -v if q < 0 else v


def pin_residual_one_rounding(o, n: int = 6000, seed: int = 11):
    """Where gate * x falls below the binary32 normal range (bf16 subnormal or
    tiny x, small gates, residuals of either sign near zero), residual_out is
    the exact residual + gate * x rounded once to binary32 (exact rational
    arithmetic, nearest-even with gradual underflow; an exact zero sum is -0
    only when both the residual and the product are -0), then to bf16 by
    torch's cast.  Includes products that underflow to zero below a +0
    residual, where rounding the product first would return +0 instead of
    the -0 of the exact sum."""
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    sign = lambda k: rng.integers(0, 2, k).astype(np.uint16) << 15  # noqa: E731
    x = np.concatenate([rng.integers(1, 0x80, n).astype(np.uint16),             # bf16 subnormals
                        rng.integers(0x0080, 0x0A00, n).astype(np.uint16)]) | sign(2 * n)
    g = np.concatenate([rng.integers(0x2F00, 0x3F80, 2 * n).astype(np.uint16)]) | sign(2 * n)
    r = np.concatenate([np.zeros(n // 2, np.uint16), rng.integers(1, 0x0300, 2 * n - n // 2).astype(np.uint16)])
    r = r | sign(2 * n)
    # the case that separates one rounding from two: -2^-133 * 2^-20 below +0
    x = np.concatenate([x, _bits([-2.0 ** -133, 2.0 ** -133, -2.0 ** -130])])
    g = np.concatenate([g, _bits([2.0 ** -20, -2.0 ** -20, 2.0 ** -30])])
    r = np.concatenate([r, _bits([0.0, 0.0, 0.0])])
    got = o.residual(r, g, x)
    xf, gf, rf = (bf16_to_f32(v).astype(np.float64) for v in (x, g, r))
    ref32 = np.empty(len(x), np.float32)
    for i in range(len(x)):
        prod = Fraction(gf[i]) * Fraction(xf[i])
        prod_negative_zero = prod == 0 and (math.copysign(1.0, gf[i]) * math.copysign(1.0, xf[i]) < 0)
        q = Fraction(rf[i]) + prod
        ref32[i] = _f32_nearest(q, prod_negative_zero and math.copysign(1.0, rf[i]) < 0)
    ref = torch.from_numpy(ref32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = got != ref
    assert not bad.any(), "x %04x gate %04x res %04x: oracle %04x exact %04x (%d cases)" % (
        x[bad][0], g[bad][0], r[bad][0], got[bad][0], ref[bad][0], int(bad.sum()))
    assert got[-3] == 0x8000 and got[-2] == 0x8000, (hex(got[-3]), hex(got[-2]))


def pin_residual_gate_zero(o, seed: int = 3):
    """gate = 0 leaves the residual stream unchanged (finite x, no -0 residuals)."""
    rng = np.random.default_rng(seed)
    x = synth.random_bf16((4096,), seed, 1)
    r = synth.random_bf16((4096,), seed, 2)
    got = o.residual(r, np.zeros_like(r), x)
    assert np.array_equal(got, r)
    # through the fused op too
    D = 64
    xr = x.reshape(-1, D)
    rr = r.reshape(-1, D)
    y, ro, _ = o.fused(xr, rr, _zeros(1, D), None, None, _zeros(1, D), _zeros(1, D), 1,
                       xr.shape[0], D, False)
    assert np.array_equal(ro, rr)
    del rng


# --------------------------------------------------------------------------- closed forms

def pin_closed_forms(o):
    """Rows whose normalisation has a closed form, for LayerNorm and RMSNorm at
    D = 8 and D = 5120 and two eps values (eps inside the square root):
      constant c:      LN -> 0;               RMS -> c / sqrt(c^2 + eps)
      zero row:        0 for both
      alternating +-a: +-a / sqrt(a^2 + eps) for both
      one-hot v:       LN hot (v - v/D)/sqrt(v^2 (D-1)/D^2 + eps), others -(v/D)/sqrt(.)
                       RMS hot v / sqrt(v^2/D + eps), others 0."""
    for D in (8, 5120):
        for eps in (1e-6, 0.25):
            e = float(np.float32(eps))
            for c in (3.0, -0.375, 2.0 ** -10):
                x = _const(2, D, c)
                cv = float(bf16_to_f64(x[:1, :1])[0, 0])
                _, t = _nss_t(o, x, D, False, eps)
                assert np.all(t == 0.0), ("LN const", D, eps, c)
                _, t = _nss_t(o, x, D, True, eps)
                np.testing.assert_allclose(t, cv / math.sqrt(cv * cv + e), rtol=1e-14)
            z = _zeros(1, D)
            for rms in (False, True):
                _, t = _nss_t(o, z, D, rms, eps)
                assert np.all(t == 0.0)
            for a in (2.0, 0.5, 1.5):
                row = np.where(np.arange(D) % 2 == 0, a, -a)
                x = _bits(row)[None, :]
                for rms in (False, True):
                    _, t = _nss_t(o, x, D, rms, eps)
                    np.testing.assert_allclose(t[0], row / math.sqrt(a * a + e), rtol=1e-14)
            for v in (4.0, -1.5):
                x = np.zeros((1, D), dtype=np.uint16)
                x[0, 3] = bf16_of_exact(v)
                _, t = _nss_t(o, x, D, False, eps)
                den = math.sqrt(v * v * (D - 1) / (D * D) + e)
                exp = np.full(D, -(v / D) / den)
                exp[3] = (v - v / D) / den
                np.testing.assert_allclose(t[0], exp, rtol=1e-12)
                _, t = _nss_t(o, x, D, True, eps)
                exp = np.zeros(D)
                exp[3] = v / math.sqrt(v * v / D + e)
                np.testing.assert_allclose(t[0], exp, rtol=1e-14, atol=0)


def pin_modulation(o, seed: int = 4):
    """The modulation is t = n * (1 + scale) + shift with n the (affine) norm:
    scale = -1 gives y == shift bit-exactly; scale = 0, shift = 0 gives the plain
    norm; scale = 1 doubles it exactly; a shift adds to it; weight 1 / bias 0 is
    the same as no affine; weight 2 doubles n exactly; a bias adds to it."""
    D, rows = 256, 6
    x = synth.random_bf16((rows, D), seed, 1)
    sc = synth.random_bf16((1, D), seed, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), seed, 7, a=0.0, b=0.1)
    for rms in (False, True):
        _, n = _nss_t(o, x, D, rms, 1e-6)
        y, _ = _nss_t(o, x, D, rms, 1e-6, scale=_const(1, D, -1.0), shift=sh)
        assert np.array_equal(y, np.broadcast_to(sh, y.shape)), "scale=-1 must give shift"
        _, t = _nss_t(o, x, D, rms, 1e-6, scale=_const(1, D, 1.0))
        assert np.array_equal(t, 2 * n)
        _, t = _nss_t(o, x, D, rms, 1e-6, shift=sh)
        np.testing.assert_allclose(t, n + bf16_to_f64(sh), rtol=0, atol=1e-15)
        _, t = _nss_t(o, x, D, rms, 1e-6, scale=sc)
        np.testing.assert_allclose(t, n * (1 + bf16_to_f64(sc)), rtol=1e-15, atol=1e-300)
        _, t = _nss_t(o, x, D, rms, 1e-6, weight=_const(1, D, 1.0)[0],
                      bias=np.zeros(D, dtype=np.uint16))
        assert np.array_equal(t, n)
        _, t = _nss_t(o, x, D, rms, 1e-6, weight=_const(1, D, 2.0)[0])
        assert np.array_equal(t, 2 * n)
        bb = synth.random_bf16((D,), seed, 5, a=0.0, b=0.1)
        _, t = _nss_t(o, x, D, rms, 1e-6, weight=_const(1, D, 1.0)[0], bias=bb)
        np.testing.assert_allclose(t, n + bf16_to_f64(bb)[None, :], rtol=0, atol=1e-15)
        # affine before modulation: weight 2 with scale 1 and shift s -> 4n + s
        _, t = _nss_t(o, x, D, rms, 1e-6, weight=_const(1, D, 2.0)[0],
                      scale=_const(1, D, 1.0), shift=sh)
        np.testing.assert_allclose(t, 4 * n + bf16_to_f64(sh), rtol=0, atol=1e-14)


def pin_torch_norms(o, seed: int = 5):
    """With scale = shift = 0 the oracle equals torch.nn.functional.layer_norm /
    rms_norm evaluated in float64 (with and without weight/bias), to 1e-12."""
    F = torch.nn.functional
    for D in (8, 64, 1000, 5120):
        rows = 8
        x = synth.random_bf16((rows, D), seed + D, 1)
        w = synth.random_bf16((D,), seed + D, 4, a=1.0, b=0.05)
        bb = synth.random_bf16((D,), seed + D, 5, a=0.0, b=0.1)
        xt = torch.from_numpy(bf16_to_f64(x))
        wt = torch.from_numpy(bf16_to_f64(w))
        bt = torch.from_numpy(bf16_to_f64(bb))
        eps = float(np.float32(1e-6))
        cases = [
            (False, None, None, F.layer_norm(xt, (D,), eps=eps)),
            (False, w, None, F.layer_norm(xt, (D,), weight=wt, eps=eps)),
            (False, w, bb, F.layer_norm(xt, (D,), weight=wt, bias=bt, eps=eps)),
            (True, None, None, F.rms_norm(xt, (D,), eps=eps)),
            (True, w, None, F.rms_norm(xt, (D,), weight=wt, eps=eps)),
        ]
        for rms, ww, bias, ref in cases:
            _, t = _nss_t(o, x, D, rms, 1e-6, weight=ww, bias=bias)
            np.testing.assert_allclose(t, ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_layouts(o, seed: int = 6):
    """Layout addressing.  Scale = -1 makes y equal the shift row an activation
    row reads, so distinct integer shift rows reveal the selected row:
      BCAST: every row reads row 0 (also for every batch at B > 1);
      ROW:   row r reads row r;
      FRAME (B=2, L=12, F=3, frame-major tokens): rows read 0,0,0,0,1,1,1,1,2,2,2,2
             in batch 0 and 3,3,3,3,4,4,4,4,5,5,5,5 in batch 1.
    Gate layouts the same way (x = 1, residual = 0 gives residual_out = gate).
    Equivalences: FRAME(F=1) == BCAST at B=1; ROW with equal rows == BCAST;
    FRAME expanded to (B, L, C) == ROW (all bit-exact)."""
    B, L, D, F = 2, 12, 16, 3
    R = B * L
    x = synth.random_bf16((R, D), seed, 1)
    minus1 = _const(1, D, -1.0)
    expect = {
        BCAST: [0] * R,
        ROW: list(range(R)),
        FRAME: [0] * 4 + [1] * 4 + [2] * 4 + [3] * 4 + [4] * 4 + [5] * 4,
    }
    for kind, nrows in ((BCAST, 1), (ROW, R), (FRAME, B * F)):
        frames = F if kind == FRAME else 0
        sh = _bits(np.repeat(np.arange(1, nrows + 1, dtype=np.float64)[:, None], D, 1))
        sc = np.repeat(minus1, nrows, 0)
        y, _ = o.nss(x, None, None, sc, sh, B, L, D, False, (kind, frames), 1e-6)
        sel = bf16_to_f64(y[:, 0]) - 1
        assert sel.tolist() == expect[kind], (kind, sel.tolist())
        assert np.all(y == y[:, :1])
        # the gate layout, through the residual stream
        ones = _const(R, D, 1.0)
        g = _bits(np.repeat(np.arange(1, nrows + 1, dtype=np.float64)[:, None], D, 1))
        _, ro, _ = o.fused(ones, _zeros(R, D), g, None, None, _zeros(1, D), _zeros(1, D),
                           B, L, D, False, (kind, frames), (BCAST, 0), 1e-6)
        sel = bf16_to_f64(ro[:, 0]) - 1
        assert sel.tolist() == expect[kind], ("gate", kind, sel.tolist())

    res = synth.random_bf16((R, D), seed, 2)
    gate = synth.random_bf16((B * F, D), seed, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    sc = synth.random_bf16((B * F, D), seed, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((B * F, D), seed, 7, a=0.0, b=0.1)
    # FRAME expanded to per-row == ROW
    idx = np.array(expect[FRAME])
    a = o.fused(x, res, gate, None, None, sc, sh, B, L, D, False, (FRAME, F), (FRAME, F), 1e-6)
    b = o.fused(x, res, gate[idx], None, None, sc[idx], sh[idx], B, L, D, False, (ROW, 0),
                (ROW, 0), 1e-6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # FRAME(F=1) == BCAST at B=1; ROW with identical rows == BCAST
    x1, r1 = x[:L], res[:L]
    a = o.fused(x1, r1, gate[:1], None, None, sc[:1], sh[:1], 1, L, D, False, (FRAME, 1),
                (FRAME, 1), 1e-6)
    b = o.fused(x1, r1, gate[:1], None, None, sc[:1], sh[:1], 1, L, D, False, (BCAST, 0),
                (BCAST, 0), 1e-6)
    c = o.fused(x1, r1, np.repeat(gate[:1], L, 0), None, None, np.repeat(sc[:1], L, 0),
                np.repeat(sh[:1], L, 0), 1, L, D, False, (ROW, 0), (ROW, 0), 1e-6)
    for u, v in ((a, b), (b, c)):
        assert np.array_equal(u[0], v[0]) and np.array_equal(u[1], v[1])


def pin_fused_is_nss_of_residual(o, seed: int = 7):
    """The fused op normalises its own bf16 residual output: y_fused equals
    nss(residual_out) bit-exactly, for both norms, with and without weight."""
    B, L, D = 1, 10, 320
    x = synth.random_bf16((L, D), seed, 1)
    r = synth.random_bf16((L, D), seed, 2)
    g = synth.random_bf16((1, D), seed, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    sc = synth.random_bf16((1, D), seed, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), seed, 7, a=0.0, b=0.1)
    w = synth.random_bf16((D,), seed, 4, a=1.0, b=0.05)
    for rms in (False, True):
        for ww in (None, w):
            y, ro, _ = o.fused(x, r, g, ww, None, sc, sh, B, L, D, rms)
            y2, _ = o.nss(ro, ww, None, sc, sh, B, L, D, rms)
            assert np.array_equal(y, y2)


def pin_scale_invariance(o, seed: int = 8):
    """With eps = 0, multiplying a row by 2^k leaves the normalised row bit-identical
    (every binary64 step scales exactly), for both norms."""
    D = 96
    x = synth.random_bf16((5, D), seed, 1)
    xf = bf16_to_f32(x)
    for k in (-3, 1, 5):
        xs = (np.ldexp(xf, k).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        for rms in (False, True):
            _, t0 = _nss_t(o, x, D, rms, 0.0)
            _, t1 = _nss_t(o, xs, D, rms, 0.0)
            assert np.array_equal(t0, t1)


def _ld_norm(h, rms, eps):
    """Independent evaluator in extended precision: one-pass moments
    var = E[h^2] - E[h]^2 (exact for dyadic rows), then normalise."""
    h = h.astype(np.longdouble)
    D = h.shape[1]
    s1 = h.sum(1, keepdims=True)
    s2 = (h * h).sum(1, keepdims=True)
    if rms:
        mean = np.zeros_like(s1)
        var = s2 / D
    else:
        mean = s1 / D
        var = s2 / D - mean * mean
    return (h - mean) / np.sqrt(var + np.longdouble(np.float32(eps)))


def pin_bruteforce_d8(o, alphabet=(-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0), stride: int = 1,
                      threads: int = 8):
    """Every row of D = 8 values from a dyadic alphabet (7^8 = 5,764,801 rows):
    the oracle's binary64 t agrees with the extended-precision evaluator to
    1e-12, and y is the nearest bf16 of it (table search) except within 2^-40 of
    a tie."""
    D = 8
    vals = _bits(list(alphabet))
    idx = np.indices((len(alphabet),) * D, dtype=np.int8).reshape(D, -1).T[::stride]
    x = vals[idx]
    h = bf16_to_f64(x)
    for rms in (False, True):
        for eps in (1e-6, 0.25):
            y, t = o.nss(x, None, None, _zeros(1, D), _zeros(1, D), 1, x.shape[0], D, rms,
                         (BCAST, 0), eps, want_t=True, threads=threads)
            ref = _ld_norm(h, rms, eps)
            err = np.abs(t - ref.astype(np.float64))
            assert float(err.max()) <= 1e-12, (rms, eps, float(err.max()))
            ok = (y == nearest_bf16(t)) | near_bf16_tie(t)
            assert ok.all()


def pin_random_rows_ld(o, rows: int = 100000, D: int = 8, seed: int = 9):
    """Random bf16 rows (N(0,1)): binary64 t within 1e-12 of the extended-precision
    one-pass evaluator (well-conditioned rows)."""
    x = synth.random_bf16((rows, D), seed, 1)
    h = bf16_to_f64(x)
    for rms in (False, True):
        _, t = o.nss(x, None, None, _zeros(1, D), _zeros(1, D), 1, rows, D, rms, (BCAST, 0),
                     1e-6, want_t=True)
        ref = _ld_norm(h, rms, 1e-6).astype(np.float64)
        var = h.var(1) if not rms else (h * h).mean(1)
        good = var > 1e-2
        err = np.abs(t - ref)[good]
        assert float(err.max()) <= 1e-10, float(err.max())


def pin_invariants(o, seed: int = 10):
    """Pure norm rows (scale = shift = 0, no affine): LayerNorm rows have mean 0
    and variance 1, RMSNorm rows have RMS 1, each within 1e-3, for rows with
    variance >= 1e-3; at D in {8, 64, 1000, 5120, 10240}."""
    for D in (8, 64, 1000, 5120, 10240):
        rows = max(4, 40000 // D)
        x = synth.random_bf16((rows, D), seed + D, 1)
        h = bf16_to_f64(x)
        _, t = _nss_t(o, x, D, False, 1e-6)
        keep = h.var(1) >= 1e-3
        assert np.all(np.abs(t.mean(1)[keep]) <= 1e-3)
        assert np.all(np.abs(t.var(1)[keep] - 1) <= 1e-3)
        _, t = _nss_t(o, x, D, True, 1e-6)
        keep = (h * h).mean(1) >= 1e-3
        assert np.all(np.abs(np.sqrt((t * t).mean(1))[keep] - 1) <= 1e-3)


# --------------------------------------------------------------------------- extensions

def _torch_e4m3(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


E4M3_VALUES = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float64).numpy()   # decode table (index = code), from torch


def pin_e4m3_vs_torch(o, stride: int = 1, threads: int = 8):
    """binary64 -> FP8 E4M3 (nearest, ties to even) equals torch's float32 ->
    float8_e4m3fn cast on every binary32 value with |x| < 464 (the inputs torch
    rounds to a finite value); larger magnitudes saturate to +-448; NaN -> 0x7F."""
    from concurrent.futures import ThreadPoolExecutor
    limit = int(np.array([464.0], np.float32).view(np.uint32)[0])
    chunk = 1 << 25
    starts = list(range(0, limit, chunk * stride if stride > 1 else chunk))

    def one(s0):
        if stride == 1:
            mag = np.arange(s0, min(limit, s0 + chunk), dtype=np.uint64).astype(np.uint32)
        else:
            mag = np.arange(s0, min(limit, s0 + chunk * stride), stride, dtype=np.uint64).astype(np.uint32)
        for sign in (0, 0x80000000):
            f = (mag | np.uint32(sign)).view(np.float32)
            got = o.f64_to_e4m3(f.astype(np.float64))
            ref = _torch_e4m3(f)
            bad = got != ref
            if bad.any():
                i = int(np.argmax(bad))
                return "f32 %r: oracle %02x torch %02x" % (float(f[i]), got[i], ref[i])
        return None

    with ThreadPoolExecutor(max_workers=threads) as ex:
        for msg in ex.map(one, starts):
            assert msg is None, msg
    sat = o.f64_to_e4m3(np.array([464.0, 464.00001, 479.9, 480.0, 1e30, np.inf, -500.0, -np.inf]))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE], sat
    assert o.f64_to_e4m3(np.array([np.nan]))[0] == 0x7F
    # values between binary32 neighbours: the table-nearest rule on binary64 inputs
    rng = np.random.default_rng(12)
    t = rng.standard_normal(100000) * np.exp2(rng.integers(-12, 9, 100000).astype(np.float64))
    t = t[np.abs(t) < 460]
    got = o.f64_to_e4m3(t)
    fin = np.arange(0, 127)               # +0 .. 448
    vals = E4M3_VALUES[fin]
    a = np.abs(t)
    hi = np.clip(np.searchsorted(vals, a), 1, 126)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where((dhi < dlo) | ((dhi == dlo) & (fin[hi] % 2 == 0)), fin[hi], fin[lo])
    pick = pick | np.where(np.signbit(t), 0x80, 0)
    assert np.array_equal(got, pick.astype(np.uint8))


def pin_affine_f32(o, seed: int = 13):
    """binary32 weight/bias are used at full precision: with scale = shift = 0
    the oracle equals torch layer_norm / rms_norm in float64 with the float32
    weights widened exactly, to 1e-12; weights that are not bf16 values change
    the result relative to their bf16 rounding."""
    F = torch.nn.functional
    rng = np.random.default_rng(seed)
    for D in (64, 1000, 5120):
        x = synth.random_bf16((6, D), seed + D, 1)
        w = (1.0 + 0.05 * rng.standard_normal(D)).astype(np.float32)
        b = (0.1 * rng.standard_normal(D)).astype(np.float32)
        xt = torch.from_numpy(bf16_to_f64(x))
        eps = float(np.float32(1e-6))
        z = _zeros(1, D)
        _, t = o.nss(x, w, b, z, z, 1, 6, D, False, want_t=True, affine_f32=True)
        ref = F.layer_norm(xt, (D,), weight=torch.from_numpy(w.astype(np.float64)),
                           bias=torch.from_numpy(b.astype(np.float64)), eps=eps)
        np.testing.assert_allclose(t, ref.numpy(), rtol=1e-12, atol=1e-12)
        _, t = o.nss(x, w, None, z, z, 1, 6, D, True, want_t=True, affine_f32=True)
        ref = F.rms_norm(xt, (D,), weight=torch.from_numpy(w.astype(np.float64)), eps=eps)
        np.testing.assert_allclose(t, ref.numpy(), rtol=1e-12, atol=1e-12)
        wb = (w.view(np.uint32) >> 16).astype(np.uint16)   # a bf16 version of w
        _, t16 = o.nss(x, wb, None, z, z, 1, 6, D, True, want_t=True)
        assert not np.array_equal(t, t16)


def pin_y_f32(o, seed: int = 14):
    """The binary32 output is the nearest-even binary32 value of t (numpy's
    IEEE cast), for both ops."""
    D, L = 320, 12
    x = synth.random_bf16((L, D), seed, 1)
    r = synth.random_bf16((L, D), seed, 2)
    g = synth.random_bf16((1, D), seed, 3, dist=synth.UNIFORM, a=0.0, b=1.0)
    sc = synth.random_bf16((1, D), seed, 6, a=0.0, b=0.1)
    sh = synth.random_bf16((1, D), seed, 7, a=0.0, b=0.1)
    for rms in (False, True):
        y, t = o.nss(x, None, None, sc, sh, 1, L, D, rms, want_t=True, y_dtype=1)
        assert y.dtype == np.float32 and np.array_equal(y, t.astype(np.float32))
        y, ro, t = o.fused(x, r, g, None, None, sc, sh, 1, L, D, rms, want_t=True, y_dtype=1)
        assert np.array_equal(y, t.astype(np.float32))
        y16, ro16, _ = o.fused(x, r, g, None, None, sc, sh, 1, L, D, rms)
        assert np.array_equal(ro, ro16)


def pin_fp8_rows(o, seed: int = 15):
    """FP8 output: per-row scale s = max|t| / 448 (binary32) and codes E4M3(t / s).
    With scale = -1 the row is t = shift exactly: a shift row whose largest
    magnitude is 448 gives s = 1 and codes equal to torch's cast of the shift
    values.  Random rows: s is the binary32 rounding of max|t| / 448; the
    largest code decodes to +-448; every element decodes to t within half an
    E4M3 step (2^-4 relative, or s * 2^-10 for subnormals); an all-zero row gives
    s = 0 and zero codes; NaN elements stay out of the maximum and encode as
    torch's cast of NaN, also in a row whose other elements are all zero
    (s = 0)."""
    D = 16
    vals = np.array([448, -3.5, 0.25, 1.0625, 1.1875, -0.001953125, 0, 100, -448, 2 ** -7,
                     13, -17, 0.5, 7.5, 240, -0.75])
    sh = _bits(vals)[None, :]
    x = synth.random_bf16((2, D), seed, 1)
    y, t, s = o.nss(x, None, None, _const(1, D, -1.0), sh, 1, 2, D, False, want_t=True, y_dtype=2)
    assert s.tolist() == [1.0, 1.0]
    ref = _torch_e4m3(bf16_to_f32(sh[0]))
    assert np.array_equal(y[0], ref) and np.array_equal(y[1], ref)
    # random rows
    L, D = 40, 1000
    x = synth.random_bf16((L, D), seed, 1)
    sc = synth.random_bf16((1, D), seed, 6, a=0.0, b=0.1)
    shr = synth.random_bf16((1, D), seed, 7, a=0.0, b=0.1)
    for rms in (False, True):
        y, t, s = o.nss(x, None, None, sc, shr, 1, L, D, rms, want_t=True, y_dtype=2)
        amax = np.abs(t).max(1)
        assert np.array_equal(s, (amax / 448.0).astype(np.float32))
        dec = E4M3_VALUES[y]
        assert np.all(np.abs(dec).max(1) == 448.0)
        err = np.abs(dec * s[:, None].astype(np.float64) - t)
        bound = 2.0 ** -4 * np.abs(t) + s[:, None] * 2.0 ** -10
        assert np.all(err <= bound * (1 + 1e-9))
    z = _zeros(3, D)
    y, _, s = o.nss(z, None, None, _zeros(1, D), _zeros(1, D), 1, 3, D, False, want_t=True,
                    y_dtype=2)
    assert np.all(s == 0) and np.all(y == 0)
    # NaN elements: an RMSNorm row holding +Inf has rstd 0, so with scale = -1
    # and shift = 0 it is t = 0 except NaN (Inf * 0) where the Inf was; a
    # LayerNorm row holding NaN is NaN throughout.  Both rows get s = 0.
    nan_code = _torch_e4m3(np.array([np.nan], np.float32))[0]
    xr = synth.random_bf16((1, D), seed, 2)
    xr[0, 3] = 0x7F80
    y, t, s = o.nss(xr, None, None, _const(1, D, -1.0), _zeros(1, D), 1, 1, D, True, want_t=True,
                    y_dtype=2)
    assert s[0] == 0 and y[0, 3] == nan_code and np.all(np.delete(y[0], 3) == 0)
    assert np.isnan(t[0, 3]) and np.all(np.delete(t[0], 3) == 0)
    xn = synth.random_bf16((1, D), seed, 3)
    xn[0, 9] = 0x7FC0
    y, _, s = o.nss(xn, None, None, sc, shr, 1, 1, D, False, want_t=True, y_dtype=2)
    assert s[0] == 0 and np.all(y[0] == nan_code)
    # a NaN next to finite values: the scale comes from the finite ones
    y, t, s = o.nss(xr, None, None, sc, shr, 1, 1, D, True, want_t=True, y_dtype=2)
    fin = ~np.isnan(t[0])
    assert s[0] == np.float32(np.abs(t[0][fin]).max() / 448.0) and y[0, 3] == nan_code


def pin_golden_worked_rows(o):
    """The hand-worked rows of tests/golden/worked_rows.txt: dyadic inputs whose
    results follow exactly from the definition (residual ties to even, gate 0,
    1/2 and 2, eps inside the square root, the biased variance, uncentred
    RMSNorm, affine before modulation, per-frame and per-row operand rows, a
    constant row, binary32 weight/bias and output, an FP8 row with its scale).
    Every bit of y, residual_out and the FP8 scale must match."""
    from golden_cases import run_oracle
    for c in load_golden():
        y, ro, ys = run_oracle(o, c)
        if ro is not None:
            assert np.array_equal(ro.ravel(), c["expect.residual_out"]), c["name"]
        assert np.array_equal(y.ravel(), c["expect.y"]), c["name"]
        if ys is not None:
            assert np.array_equal(ys.ravel(), c["expect.y_scale"]), c["name"]


def load_golden():
    from golden_cases import load_cases
    return load_cases()

FAST_PINS = [pin_golden_worked_rows, pin_affine_f32, pin_y_f32, pin_fp8_rows, pin_round_f64, pin_residual_gate_zero,
             pin_residual_one_rounding, pin_closed_forms, pin_modulation,
             pin_torch_norms, pin_layouts, pin_fused_is_nss_of_residual, pin_scale_invariance,
             pin_random_rows_ld, pin_invariants]
