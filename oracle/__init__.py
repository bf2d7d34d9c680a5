"""ctypes wrapper of the plain C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg
of the benchmark are the only users.  The product path never imports this
package, and this package never imports the product.

Arrays are numpy ``uint16`` bf16 bit patterns.  Layouts are ``(kind, frames)``
pairs with kind 0 = broadcast (1, C) row, 1 = per-row (B, L, C),
2 = per-frame (B, F, 1, C).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

BCAST, ROW, FRAME = 0, 1, 2
OK, EINVAL = 0, 1
Y_BF16, Y_F32, Y_FP8 = 0, 1, 2
_Y_NP = {Y_BF16: np.uint16, Y_F32: np.float32, Y_FP8: np.uint8}


def build(src: str = SRC, out: str = LIB, force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """One loaded copy of the oracle library (the default one, or a test build)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = build(force=False)
        lib = ctypes.CDLL(path)
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_f32_to_bf16_array.argtypes = [_P, _P, _I64]
        lib.orc_f64_to_bf16_array.argtypes = [_P, _P, _I64]
        lib.orc_residual_array.argtypes = [_P, _P, _P, _P, _I64]
        lib.orc_mod_row.argtypes = [ctypes.c_int, _I64, _I64, _I64]
        lib.orc_mod_row.restype = _I64
        lib.orc_fused.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                  ctypes.c_int, _I64, ctypes.c_int, _I64, ctypes.c_float,
                                  _I64, _I64, _P, _P, _P]
        lib.orc_fused.restype = ctypes.c_int
        lib.orc_nss.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                ctypes.c_int, _I64, ctypes.c_float, _I64, _I64, _P, _P]
        lib.orc_nss.restype = ctypes.c_int
        lib.orc_f64_to_e4m3_array.argtypes = [_P, _P, _I64]
        lib.orc_fused_ex.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                     ctypes.c_int, _I64, ctypes.c_int, _I64, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, _I64, _I64, _P, _P, _P, _P]
        lib.orc_fused_ex.restype = ctypes.c_int
        lib.orc_nss_ex.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                   ctypes.c_int, _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                   _I64, _I64, _P, _P, _P]
        lib.orc_nss_ex.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- conversions ---------------------------------------------------------
    def f64_to_bf16(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.orc_f64_to_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def f32_to_bf16(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.orc_f32_to_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def f64_to_e4m3(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.orc_f64_to_e4m3_array(a.ctypes.data, out.ctypes.data, a.size)
        return out

    def residual(self, res, gate, x) -> np.ndarray:
        res = np.ascontiguousarray(res, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        g = None if gate is None else np.ascontiguousarray(gate, dtype=np.uint16)
        assert res.shape == x.shape and (g is None or g.shape == x.shape)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.orc_residual_array(res.ctypes.data, _ptr(g), x.ctypes.data, out.ctypes.data,
                                    x.size)
        return out

    def mod_row(self, layout, r: int, L: int) -> int:
        return int(self.lib.orc_mod_row(layout[0], layout[1], r, L))

    # -- the two operations --------------------------------------------------
    @staticmethod
    def _affine(a, affine_f32):
        if a is None:
            return None
        return np.ascontiguousarray(a, dtype=np.float32 if affine_f32 else np.uint16)

    def fused(self, x, residual, gate, weight, bias, scale, shift, B, L, D, is_rms,
              gate_layout=(BCAST, 0), ss_layout=(BCAST, 0), eps=1e-6, row0=0, nrows=None,
              want_t=False, threads=1, affine_f32=False, y_dtype=Y_BF16):
        """Rows [row0, row0+nrows): returns (y, residual_out, t or None), plus
        the per-row scales as a 4th item when y_dtype is Y_FP8.

        x and residual hold rows row0 .. row0+nrows-1 ([nrows, D]); modulation
        operands are whole tensors; weight/bias are float32 when affine_f32.
        """
        if nrows is None:
            nrows = B * L - row0
        x = np.ascontiguousarray(x, dtype=np.uint16)
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        assert x.size == nrows * D and residual.size == nrows * D
        ops = [None if a is None else np.ascontiguousarray(a, dtype=np.uint16)
               for a in (gate, scale, shift)]
        w = self._affine(weight, affine_f32)
        b = self._affine(bias, affine_f32)
        y = np.empty((nrows, D), dtype=_Y_NP[y_dtype])
        ys = np.empty(nrows, dtype=np.float32) if y_dtype == Y_FP8 else None
        ro = np.empty((nrows, D), dtype=np.uint16)
        t = np.empty((nrows, D), dtype=np.float64) if want_t else None
        isz = y.itemsize

        def run(a0, a1):
            st = self.lib.orc_fused_ex(
                x.ctypes.data + 2 * a0 * D, residual.ctypes.data + 2 * a0 * D,
                _ptr(ops[0]), _ptr(w), _ptr(b), _ptr(ops[1]), _ptr(ops[2]), B, L, D,
                int(is_rms), gate_layout[0], gate_layout[1], ss_layout[0], ss_layout[1], eps,
                int(bool(affine_f32)), int(y_dtype), row0 + a0, a1 - a0,
                y.ctypes.data + isz * a0 * D, None if ys is None else ys.ctypes.data + 4 * a0,
                ro.ctypes.data + 2 * a0 * D, None if t is None else t.ctypes.data + 8 * a0 * D)
            if st != OK:
                raise ValueError("oracle rejected the arguments (status %d)" % st)

        _split(nrows, threads, run)
        if y_dtype == Y_FP8:
            return y, ro, t, ys
        return y, ro, t

    def nss(self, x, weight, bias, scale, shift, B, L, D, is_rms, ss_layout=(BCAST, 0),
            eps=1e-6, row0=0, nrows=None, want_t=False, threads=1, affine_f32=False,
            y_dtype=Y_BF16):
        """Rows [row0, row0+nrows): returns (y, t or None), plus the per-row
        scales as a 3rd item when y_dtype is Y_FP8."""
        if nrows is None:
            nrows = B * L - row0
        x = np.ascontiguousarray(x, dtype=np.uint16)
        assert x.size == nrows * D
        ops = [None if a is None else np.ascontiguousarray(a, dtype=np.uint16)
               for a in (scale, shift)]
        w = self._affine(weight, affine_f32)
        b = self._affine(bias, affine_f32)
        y = np.empty((nrows, D), dtype=_Y_NP[y_dtype])
        ys = np.empty(nrows, dtype=np.float32) if y_dtype == Y_FP8 else None
        t = np.empty((nrows, D), dtype=np.float64) if want_t else None
        isz = y.itemsize

        def run(a0, a1):
            st = self.lib.orc_nss_ex(
                x.ctypes.data + 2 * a0 * D, _ptr(w), _ptr(b), _ptr(ops[0]), _ptr(ops[1]), B, L,
                D, int(is_rms), ss_layout[0], ss_layout[1], eps, int(bool(affine_f32)),
                int(y_dtype), row0 + a0, a1 - a0, y.ctypes.data + isz * a0 * D,
                None if ys is None else ys.ctypes.data + 4 * a0,
                None if t is None else t.ctypes.data + 8 * a0 * D)
            if st != OK:
                raise ValueError("oracle rejected the arguments (status %d)" % st)

        _split(nrows, threads, run)
        if y_dtype == Y_FP8:
            return y, t, ys
        return y, t

    def run_workload(self, wl, inputs, row0=0, nrows=None, want_t=False, threads=1):
        """Evaluate a synth.Workload on rows [row0, row0+nrows) of its inputs dict."""
        if nrows is None:
            nrows = wl.R - row0
        D = wl.D
        xs = inputs["x"].reshape(-1, D)[row0:row0 + nrows]
        common = dict(B=wl.B, L=wl.L, D=D, is_rms=wl.is_rms, ss_layout=wl.ss_layout,
                      eps=wl.eps, row0=row0, nrows=nrows, want_t=want_t, threads=threads)
        if wl.op == "fused":
            rs = inputs["residual"].reshape(-1, D)[row0:row0 + nrows]
            return self.fused(xs, rs, inputs.get("gate"), inputs.get("weight"),
                              inputs.get("bias"), inputs["scale"], inputs["shift"],
                              gate_layout=wl.gate_layout or (BCAST, 0), **common)
        y, t = self.nss(xs, inputs.get("weight"), inputs.get("bias"), inputs["scale"],
                        inputs["shift"], **common)
        return y, None, t


def _split(n, threads, run):
    threads = max(1, int(threads))
    if threads == 1 or n < 2 * threads:
        run(0, n)
        return
    step = (n + threads - 1) // threads
    with ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(run, a, min(n, a + step)) for a in range(0, n, step)]
        for f in futs:
            f.result()


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
