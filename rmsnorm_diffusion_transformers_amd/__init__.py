"""Fused residual + gate + LayerNorm/RMSNorm + scale/shift for video diffusion
transformers on MI355X (gfx950).

A thin ctypes binding over ``librnorm.so`` (C ABI in ``include/resnorm.h``).
It only marshals arguments: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if the library is not built,
importing this package raises ImportError; if a call is rejected, it raises
``RnError`` with the library's message.

Low level (same names and argument order as the C entry points):
    resnorm_fused_fwd(y, residual_out, x, residual, gate, weight, bias, scale,
                      shift, B, L, D, flags, gate_layout, ss_layout, eps, stream)
    norm_scale_shift_fwd(y, x, weight, bias, scale, shift, B, L, D, flags,
                         ss_layout, eps, stream)
    resnorm_fused_fwd_ex / norm_scale_shift_fwd_ex: the same plus affine_dtype,
    y_dtype and y_scale (binary32 weight/bias; binary32 or FP8 E4M3 y)
    prepare(entry, *args): check a call once; returns a callable that
    enqueues it again (for loops over the same buffers)
Tensor level (operand order of the custom ops flydsl_fused_residual_norm_scale_shift
and flydsl_norm_scale_shift, sglang PR #36349, "Microbenchmark"):
    fused_residual_norm_scale_shift(residual, x, gate, weight, bias, scale, shift,
                                    norm_type, eps) -> (y, residual_out)
    norm_scale_shift(x, weight, bias, scale, shift, norm_type, eps) -> y
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librnorm.so")

RN_OK, RN_EINVAL, RN_EUNSUPPORTED, RN_ELAUNCH = 0, 1, 2, 3
RN_RMS, RN_GATE, RN_WEIGHT, RN_BIAS = 1, 2, 4, 8
RN_BCAST, RN_ROW, RN_FRAME = 0, 1, 2
RN_DTYPE_BF16, RN_DTYPE_F32, RN_DTYPE_FP8_E4M3 = 0, 1, 2
RN_D_MAX = 16384
_STATUS = {0: "RN_OK", 1: "RN_EINVAL", 2: "RN_EUNSUPPORTED", 3: "RN_ELAUNCH"}


class rn_layout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("frames", ctypes.c_int32)]


class rn_ext(ctypes.Structure):
    _fields_ = [("affine_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
                ("y_scale", ctypes.c_void_p)]


class rn_launch_info(ctypes.Structure):
    _fields_ = [("vec_per_lane", ctypes.c_int32), ("waves_per_row", ctypes.c_int32),
                ("waves_per_block", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int64), ("rows_per_wave", ctypes.c_int32)]


class RnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("librnorm.so is not built (expected at %s); build it with "
                          "__graft_entry__.build() or python %s/_build.py" % (LIB_PATH, _HERE))
    # One HIP runtime per process.  torch ships its own copies of the HIP and
    # HSA runtimes; if this library were mapped first, its libamdhip64.so.7
    # would pull in the system copies and torch would then add its own, and
    # with two HSA runtimes in one process one of them can find no device.
    # Importing torch first makes the library resolve to torch's copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, U32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    lib.resnorm_fused_fwd.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, U32,
                                      rn_layout, rn_layout, F32, P]
    lib.resnorm_fused_fwd.restype = ctypes.c_int
    lib.norm_scale_shift_fwd.argtypes = [P, P, P, P, P, P, I64, I64, I64, U32, rn_layout, F32, P]
    lib.norm_scale_shift_fwd.restype = ctypes.c_int
    lib.resnorm_fused_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, U32,
                                         rn_layout, rn_layout, F32, ctypes.POINTER(rn_ext), P]
    lib.resnorm_fused_fwd_ex.restype = ctypes.c_int
    lib.norm_scale_shift_fwd_ex.argtypes = [P, P, P, P, P, P, I64, I64, I64, U32, rn_layout, F32,
                                            ctypes.POINTER(rn_ext), P]
    lib.norm_scale_shift_fwd_ex.restype = ctypes.c_int
    lib.rn_last_error.argtypes = []
    lib.rn_last_error.restype = ctypes.c_char_p
    lib.rn_describe_launch.argtypes = [I64, I64, I64, U32, ctypes.c_int32, rn_layout, rn_layout,
                                       ctypes.POINTER(rn_launch_info)]
    lib.rn_describe_launch.restype = ctypes.c_int
    lib.rn_describe_launch_ex.argtypes = [I64, I64, I64, U32, ctypes.c_int32, rn_layout, rn_layout,
                                          ctypes.POINTER(rn_ext), ctypes.POINTER(rn_launch_info)]
    lib.rn_describe_launch_ex.restype = ctypes.c_int
    lib.rn_version.argtypes = []
    lib.rn_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def last_error() -> str:
    return _lib.rn_last_error().decode()


def version() -> str:
    return _lib.rn_version().decode()


def _check(status: int):
    if status != RN_OK:
        raise RnError(status, last_error())


_torch = None          # torch, imported on first use (the C ABI works without it)
_TORCH_DTYPES = {}     # RN_DTYPE_* -> torch dtype


def _torch_mod():
    global _torch
    if _torch is None:
        import torch
        _TORCH_DTYPES.update({RN_DTYPE_BF16: torch.bfloat16, RN_DTYPE_F32: torch.float32,
                              RN_DTYPE_FP8_E4M3: torch.float8_e4m3fn})
        _torch = torch
    return _torch


def _addr(t, dtype=RN_DTYPE_BF16):
    """Device address of a contiguous CUDA tensor of the given element type
    (or an int address, or None).  Runs on every call, so it sticks to cheap
    attribute checks."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    torch = _torch_mod()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, an int address or None, got %r" % type(t))
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU device (got %s); there is no CPU path" % t.device)
    want = _TORCH_DTYPES[dtype]
    if t.dtype != want:
        raise TypeError("tensor must be %s (got %s)" % (want, t.dtype))
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_code(dt) -> int:
    import torch
    if dt is None or dt == torch.bfloat16:
        return RN_DTYPE_BF16
    if dt == torch.float32:
        return RN_DTYPE_F32
    if dt == torch.float8_e4m3fn:
        return RN_DTYPE_FP8_E4M3
    raise TypeError("unsupported element type %s" % dt)


def _rows(lay, B: int, L: int) -> int:
    kind, frames = (lay.kind, lay.frames) if isinstance(lay, rn_layout) else lay
    return {RN_BCAST: 1, RN_ROW: B * L, RN_FRAME: B * frames}.get(int(kind), 0)


def _check_tensors(named):
    """Host-side checks of the tensors an entry point receives (int addresses
    are passed through unchecked): one common device, and at least as many
    elements as the sizes and layouts make the kernel touch.  `named` is a
    sequence of (name, tensor or address or None, elements needed).  Returns
    the device index (None when only addresses were given)."""
    Tensor = _torch_mod().Tensor
    dev = first = None
    for name, t, need in named:
        if not isinstance(t, Tensor):
            continue
        if t.numel() < need:
            raise ValueError("%s has %d elements; the sizes and layout need %d" % (name, t.numel(), need))
        d = t.get_device()   # GPU index; -1 for host and meta tensors
        if first is None:
            dev, first = d, t
        elif d != dev or (d < 0 and t.device != first.device):
            raise ValueError("%s is on %s but other operands are on %s" % (name, t.device, first.device))
    return dev if dev is not None and dev >= 0 else None


def _stream(stream, device=None):
    """The stream to enqueue on: the given one, else torch's current stream of
    the operands' device."""
    if stream is None:
        return _torch_mod().cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _layout(lay) -> rn_layout:
    if isinstance(lay, rn_layout):
        return lay
    kind, frames = lay
    return rn_layout(int(kind), int(frames))


def _args_fused(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D, flags,
                gate_layout, ss_layout, eps, stream, affine_dtype, y_dtype, y_scale):
    """Checked C arguments of resnorm_fused_fwd_ex."""
    dev = _fused_checks(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                        gate_layout, ss_layout, y_scale)
    ext = rn_ext(int(affine_dtype), int(y_dtype), _addr(y_scale, RN_DTYPE_F32))
    return (_lib.resnorm_fused_fwd_ex,
            (_addr(y, y_dtype), _addr(residual_out), _addr(x), _addr(residual), _addr(gate),
             _addr(weight, affine_dtype), _addr(bias, affine_dtype), _addr(scale), _addr(shift),
             int(B), int(L), int(D), int(flags), _layout(gate_layout), _layout(ss_layout),
             float(eps), ctypes.byref(ext), _stream(stream, dev)), ext)


def _args_nss(y, x, weight, bias, scale, shift, B, L, D, flags, ss_layout, eps, stream,
              affine_dtype, y_dtype, y_scale):
    """Checked C arguments of norm_scale_shift_fwd_ex."""
    dev = _nss_checks(y, x, weight, bias, scale, shift, B, L, D, ss_layout, y_scale)
    ext = rn_ext(int(affine_dtype), int(y_dtype), _addr(y_scale, RN_DTYPE_F32))
    return (_lib.norm_scale_shift_fwd_ex,
            (_addr(y, y_dtype), _addr(x), _addr(weight, affine_dtype), _addr(bias, affine_dtype),
             _addr(scale), _addr(shift), int(B), int(L), int(D), int(flags), _layout(ss_layout),
             float(eps), ctypes.byref(ext), _stream(stream, dev)), ext)


def resnorm_fused_fwd(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                      flags, gate_layout=(RN_BCAST, 0), ss_layout=(RN_BCAST, 0), eps=1e-6,
                      stream=None) -> None:
    """Enqueue the fused op (C entry point of the same name); raises RnError."""
    dev = _fused_checks(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                        gate_layout, ss_layout, None)
    _check(_lib.resnorm_fused_fwd(_addr(y), _addr(residual_out), _addr(x), _addr(residual),
                                  _addr(gate), _addr(weight), _addr(bias), _addr(scale),
                                  _addr(shift), int(B), int(L), int(D), int(flags),
                                  _layout(gate_layout), _layout(ss_layout), float(eps),
                                  _stream(stream, dev)))


def _fused_checks(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                  gate_layout, ss_layout, y_scale):
    B, L, D = int(B), int(L), int(D)
    n, ss = B * L * D, _rows(ss_layout, B, L) * D
    return _check_tensors((("y", y, n), ("residual_out", residual_out, n), ("x", x, n),
                           ("residual", residual, n), ("gate", gate, _rows(gate_layout, B, L) * D),
                           ("weight", weight, D), ("bias", bias, D), ("scale", scale, ss),
                           ("shift", shift, ss), ("y_scale", y_scale, B * L)))


def _nss_checks(y, x, weight, bias, scale, shift, B, L, D, ss_layout, y_scale):
    B, L, D = int(B), int(L), int(D)
    n, ss = B * L * D, _rows(ss_layout, B, L) * D
    return _check_tensors((("y", y, n), ("x", x, n), ("weight", weight, D), ("bias", bias, D),
                           ("scale", scale, ss), ("shift", shift, ss), ("y_scale", y_scale, B * L)))


def norm_scale_shift_fwd(y, x, weight, bias, scale, shift, B, L, D, flags,
                         ss_layout=(RN_BCAST, 0), eps=1e-6, stream=None) -> None:
    """Enqueue the norm-only op (C entry point of the same name); raises RnError."""
    dev = _nss_checks(y, x, weight, bias, scale, shift, B, L, D, ss_layout, None)
    _check(_lib.norm_scale_shift_fwd(_addr(y), _addr(x), _addr(weight), _addr(bias),
                                     _addr(scale), _addr(shift), int(B), int(L), int(D),
                                     int(flags), _layout(ss_layout), float(eps),
                                     _stream(stream, dev)))


def resnorm_fused_fwd_ex(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L,
                         D, flags, gate_layout=(RN_BCAST, 0), ss_layout=(RN_BCAST, 0), eps=1e-6,
                         affine_dtype=RN_DTYPE_BF16, y_dtype=RN_DTYPE_BF16, y_scale=None,
                         stream=None) -> None:
    """Enqueue the fused op with other element types (C entry point of the same
    name): binary32 weight/bias; binary32 or FP8 E4M3 y (FP8 with per-row
    binary32 scales in y_scale)."""
    fn, args, _ext = _args_fused(y, residual_out, x, residual, gate, weight, bias, scale, shift,
                                 B, L, D, flags, gate_layout, ss_layout, eps, stream, affine_dtype,
                                 y_dtype, y_scale)
    _check(fn(*args))


def norm_scale_shift_fwd_ex(y, x, weight, bias, scale, shift, B, L, D, flags,
                            ss_layout=(RN_BCAST, 0), eps=1e-6, affine_dtype=RN_DTYPE_BF16,
                            y_dtype=RN_DTYPE_BF16, y_scale=None, stream=None) -> None:
    """Enqueue the norm-only op with other element types (C entry point of the
    same name)."""
    fn, args, _ext = _args_nss(y, x, weight, bias, scale, shift, B, L, D, flags, ss_layout, eps,
                               stream, affine_dtype, y_dtype, y_scale)
    _check(fn(*args))


def prepare(entry, *args, **kwargs):
    """Check a call once and return a callable that enqueues it again.

    entry is resnorm_fused_fwd, norm_scale_shift_fwd or their _ex forms; the
    other arguments are that entry point's.  Every host-side check runs here
    once (tensor devices, sizes, element types, contiguity) and the stream is
    bound now (torch's current stream of the operands' device unless one is
    given); the returned callable only calls the C entry point with the
    stored arguments and raises RnError on a non-OK status.  For loops that
    call the op on the same buffers every step: the tensors must stay alive
    and keep their storage while the callable is used.  The library keeps the
    last validated problem of each thread, so repeating a call costs the
    launch only."""
    names = {resnorm_fused_fwd: ("fused", False), resnorm_fused_fwd_ex: ("fused", True),
             norm_scale_shift_fwd: ("nss", False), norm_scale_shift_fwd_ex: ("nss", True)}
    if entry not in names:
        raise ValueError("prepare() takes resnorm_fused_fwd, norm_scale_shift_fwd or their _ex forms")
    op, ex = names[entry]
    import inspect
    bound = inspect.signature(entry).bind(*args, **kwargs)
    bound.apply_defaults()
    a = dict(bound.arguments)
    if not ex:
        a.update(affine_dtype=RN_DTYPE_BF16, y_dtype=RN_DTYPE_BF16, y_scale=None)
    if op == "fused":
        fn, cargs, ext = _args_fused(**a)
    else:
        fn, cargs, ext = _args_nss(**a)
    # ctypes objects built once; ext stays referenced by the closure
    conv = tuple(t(v) if isinstance(v, (int, float)) else v for t, v in zip(fn.argtypes, cargs))

    def launch(_fn=fn, _args=conv, _ext=ext):
        st = _fn(*_args)
        if st != RN_OK:
            raise RnError(st, last_error())
    return launch


def describe_launch(B, L, D, flags, fused=True, gate_layout=(RN_BCAST, 0),
                    ss_layout=(RN_BCAST, 0), affine_dtype=RN_DTYPE_BF16) -> dict:
    """Launch shape the library picks for a problem (host-only query;
    rn_describe_launch_ex)."""
    info = rn_launch_info()
    ext = rn_ext(int(affine_dtype), RN_DTYPE_BF16, None)
    _check(_lib.rn_describe_launch_ex(int(B), int(L), int(D), int(flags), int(bool(fused)),
                                      _layout(gate_layout), _layout(ss_layout), ctypes.byref(ext),
                                      ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in rn_launch_info._fields_}


def infer_layout(t, B: int, L: int, D: int) -> tuple:
    """Modulation layout from a tensor's shape, relative to activations [B, L, D]:
    (D,), (1, D), (1, 1, D) -> broadcast; (B, L, D) -> per row; (B, F, 1, D) ->
    per frame with F frames; (B, D) and (B, 1, D) -> per batch (per frame, F = 1)."""
    s = tuple(t.shape)
    if s in ((D,), (1, D), (1, 1, D), (1, 1, 1, D)):
        return (RN_BCAST, 0)
    if s == (B, L, D):
        return (RN_ROW, 0)
    if len(s) == 4 and s[0] == B and s[2] == 1 and s[3] == D and s[1] >= 1:
        return (RN_FRAME, s[1])
    if s in ((B, D), (B, 1, D)):
        return (RN_FRAME, 1)
    raise ValueError("cannot map modulation shape %s onto activations (%d, %d, %d)" % (s, B, L, D))


def _norm_flag(norm_type: str) -> int:
    if norm_type == "layer":
        return 0
    if norm_type == "rms":
        return RN_RMS
    raise ValueError("norm_type must be 'layer' or 'rms' (got %r)" % (norm_type,))


def _bld(x):
    if x.dim() == 3:
        return x.shape
    if x.dim() == 2:
        return (1, x.shape[0], x.shape[1])
    raise ValueError("activations must be [B, L, D] or [L, D] (got %s)" % (tuple(x.shape),))


def _affine_dtype(weight, bias) -> int:
    dts = {_dtype_code(t.dtype) for t in (weight, bias) if t is not None}
    if len(dts) > 1:
        raise TypeError("weight and bias must have the same element type")
    d = dts.pop() if dts else RN_DTYPE_BF16
    if d not in (RN_DTYPE_BF16, RN_DTYPE_F32):
        raise TypeError("weight and bias must be bfloat16 or float32")
    return d


def _new_y(x, y_dtype):
    torch = _torch_mod()
    return torch.empty(x.shape, dtype=_TORCH_DTYPES[y_dtype], device=x.device)


def fused_residual_norm_scale_shift(residual, x, gate, weight, bias, scale, shift,
                                    norm_type: str = "layer", eps: float = 1e-6, *, y=None,
                                    residual_out=None, out_dtype=None, stream=None):
    """residual_out = residual + gate * x; y = norm(residual_out) [* weight + bias]
    * (1 + scale) + shift.  weight/bias may be bfloat16 or float32; y is
    bfloat16 (default), float32, or float8_e4m3fn (out_dtype).  Returns
    (y, residual_out), or (y, residual_out, y_scale) for float8_e4m3fn."""
    import torch
    B, L, D = _bld(x)
    flags = _norm_flag(norm_type)
    if gate is not None:
        flags |= RN_GATE
    if weight is not None:
        flags |= RN_WEIGHT
    if bias is not None:
        flags |= RN_BIAS
    yd = _dtype_code(out_dtype)
    if y is None:
        y = _new_y(x, yd)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    y_scale = torch.empty((B * L,), dtype=torch.float32, device=x.device) \
        if yd == RN_DTYPE_FP8_E4M3 else None
    gl = infer_layout(gate, B, L, D) if gate is not None else (RN_BCAST, 0)
    sl = infer_layout(scale, B, L, D)
    if infer_layout(shift, B, L, D) != sl:
        raise ValueError("scale and shift must share one layout")
    resnorm_fused_fwd_ex(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                         flags, gl, sl, eps, _affine_dtype(weight, bias), yd, y_scale, stream)
    if y_scale is not None:
        return y, residual_out, y_scale
    return y, residual_out


def norm_scale_shift(x, weight, bias, scale, shift, norm_type: str = "layer", eps: float = 1e-6,
                     *, y=None, out_dtype=None, stream=None):
    """y = norm(x) [* weight + bias] * (1 + scale) + shift.  Returns y, or
    (y, y_scale) for out_dtype float8_e4m3fn."""
    import torch
    B, L, D = _bld(x)
    flags = _norm_flag(norm_type)
    if weight is not None:
        flags |= RN_WEIGHT
    if bias is not None:
        flags |= RN_BIAS
    yd = _dtype_code(out_dtype)
    if y is None:
        y = _new_y(x, yd)
    y_scale = torch.empty((B * L,), dtype=torch.float32, device=x.device) \
        if yd == RN_DTYPE_FP8_E4M3 else None
    sl = infer_layout(scale, B, L, D)
    if infer_layout(shift, B, L, D) != sl:
        raise ValueError("scale and shift must share one layout")
    norm_scale_shift_fwd_ex(y, x, weight, bias, scale, shift, B, L, D, flags, sl, eps,
                            _affine_dtype(weight, bias), yd, y_scale, stream)
    if y_scale is not None:
        return y, y_scale
    return y
