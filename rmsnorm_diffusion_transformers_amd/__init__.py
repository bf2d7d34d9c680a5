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
    kind = int(kind)
    if kind == RN_BCAST:
        return 1
    if kind == RN_ROW:
        return B * L
    if kind == RN_FRAME:
        return B * int(frames)
    return 0


def _operands(named):
    """One pass over the operands of an entry point.  `named` is a sequence of
    (name, tensor or int address or None, elements needed, RN_DTYPE_* code).
    A tensor must hold at least as many elements as the sizes and layouts make
    the kernel touch, share one device with the other tensors, have the
    element type of its code (not checked for a code the library does not
    define: the library rejects that) and be contiguous.  Int addresses are
    passed through unchecked.  Returns (GPU index or None, addresses).  Host
    tensors pass the size and device checks and are then refused: there is
    no CPU path."""
    Tensor = _torch_mod().Tensor
    dev = first = None
    ptrs = []
    for name, t, need, code in named:
        if t is None or isinstance(t, int):
            ptrs.append(t)
            continue
        if not isinstance(t, Tensor):
            raise TypeError("%s: expected a torch.Tensor, an int address or None, got %r"
                            % (name, type(t)))
        if t.numel() < need:
            raise ValueError("%s has %d elements; the sizes and layout need %d" % (name, t.numel(), need))
        d = t.get_device()   # GPU index; -1 for host and meta tensors
        if first is None:
            dev, first = d, t
        elif d != dev or (d < 0 and t.device != first.device):
            raise ValueError("%s is on %s but other operands are on %s" % (name, t.device, first.device))
        want = _TORCH_DTYPES.get(code)
        if want is not None and t.dtype != want:
            raise TypeError("%s must be %s (got %s)" % (name, want, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        ptrs.append(t.data_ptr() if d >= 0 else None)
    if first is not None and dev < 0:
        raise ValueError("tensors must be on a GPU device (got %s); there is no CPU path"
                         % first.device)
    return (dev if first is not None else None), ptrs


def _check_tensors(named):
    """_operands over (name, tensor or address or None, elements needed) with
    no element type check; returns the GPU index (None when only addresses
    were given)."""
    return _operands([(n, t, need, None) for n, t, need in named])[0]


_RAW_STREAM = None     # torch's raw current-stream query, when it has one (else False)


def _stream(stream, device=None):
    """The stream to enqueue on: the given one (a torch stream or a raw
    handle), else torch's current stream of the operands' device.  The
    current stream is read through torch's raw-handle query where torch has
    it (about 0.1 us against 1.1 us for building a torch Stream object)."""
    global _RAW_STREAM
    if stream is None:
        torch = _torch_mod()
        if _RAW_STREAM is None:
            _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or False
        if _RAW_STREAM:
            return _RAW_STREAM(torch.cuda.current_device() if device is None else device)
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_LAYOUTS = {}   # (kind, frames) of plain ints -> rn_layout (passed by value; never modified)


def _layout(lay) -> rn_layout:
    if isinstance(lay, rn_layout):
        return lay
    plain = type(lay) is tuple and len(lay) == 2 and type(lay[0]) is int and type(lay[1]) is int
    c = _LAYOUTS.get(lay) if plain else None
    if c is None:
        kind, frames = lay
        c = rn_layout(int(kind), int(frames))
        if plain and len(_LAYOUTS) < 4096:
            _LAYOUTS[lay] = c
    return c


def _fused_operands(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                    gate_layout, ss_layout, affine_dtype, y_dtype, y_scale):
    n, ss = B * L * D, _rows(ss_layout, B, L) * D
    return _operands((("y", y, n, y_dtype), ("residual_out", residual_out, n, RN_DTYPE_BF16),
                      ("x", x, n, RN_DTYPE_BF16), ("residual", residual, n, RN_DTYPE_BF16),
                      ("gate", gate, _rows(gate_layout, B, L) * D, RN_DTYPE_BF16),
                      ("weight", weight, D, affine_dtype), ("bias", bias, D, affine_dtype),
                      ("scale", scale, ss, RN_DTYPE_BF16), ("shift", shift, ss, RN_DTYPE_BF16),
                      ("y_scale", y_scale, B * L, RN_DTYPE_F32)))


def _nss_operands(y, x, weight, bias, scale, shift, B, L, D, ss_layout, affine_dtype, y_dtype,
                  y_scale):
    n, ss = B * L * D, _rows(ss_layout, B, L) * D
    return _operands((("y", y, n, y_dtype), ("x", x, n, RN_DTYPE_BF16),
                      ("weight", weight, D, affine_dtype), ("bias", bias, D, affine_dtype),
                      ("scale", scale, ss, RN_DTYPE_BF16), ("shift", shift, ss, RN_DTYPE_BF16),
                      ("y_scale", y_scale, B * L, RN_DTYPE_F32)))


def _args_fused(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D, flags,
                gate_layout, ss_layout, eps, stream, affine_dtype, y_dtype, y_scale):
    """Checked C arguments of resnorm_fused_fwd_ex."""
    B, L, D, affine_dtype, y_dtype = int(B), int(L), int(D), int(affine_dtype), int(y_dtype)
    dev, p = _fused_operands(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L,
                             D, gate_layout, ss_layout, affine_dtype, y_dtype, y_scale)
    ext = rn_ext(affine_dtype, y_dtype, p[9])
    return (_lib.resnorm_fused_fwd_ex,
            (*p[:9], B, L, D, int(flags), _layout(gate_layout), _layout(ss_layout), float(eps),
             ctypes.byref(ext), _stream(stream, dev)), ext)


def _args_nss(y, x, weight, bias, scale, shift, B, L, D, flags, ss_layout, eps, stream,
              affine_dtype, y_dtype, y_scale):
    """Checked C arguments of norm_scale_shift_fwd_ex."""
    B, L, D, affine_dtype, y_dtype = int(B), int(L), int(D), int(affine_dtype), int(y_dtype)
    dev, p = _nss_operands(y, x, weight, bias, scale, shift, B, L, D, ss_layout, affine_dtype,
                           y_dtype, y_scale)
    ext = rn_ext(affine_dtype, y_dtype, p[6])
    return (_lib.norm_scale_shift_fwd_ex,
            (*p[:6], B, L, D, int(flags), _layout(ss_layout), float(eps), ctypes.byref(ext),
             _stream(stream, dev)), ext)


def resnorm_fused_fwd(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                      flags, gate_layout=(RN_BCAST, 0), ss_layout=(RN_BCAST, 0), eps=1e-6,
                      stream=None) -> None:
    """Enqueue the fused op (C entry point of the same name); raises RnError."""
    B, L, D = int(B), int(L), int(D)
    dev, p = _fused_operands(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L,
                             D, gate_layout, ss_layout, RN_DTYPE_BF16, RN_DTYPE_BF16, None)
    st = _lib.resnorm_fused_fwd(*p[:9], B, L, D, int(flags), _layout(gate_layout),
                                _layout(ss_layout), float(eps), _stream(stream, dev))
    if st != RN_OK:
        raise RnError(st, last_error())


def norm_scale_shift_fwd(y, x, weight, bias, scale, shift, B, L, D, flags,
                         ss_layout=(RN_BCAST, 0), eps=1e-6, stream=None) -> None:
    """Enqueue the norm-only op (C entry point of the same name); raises RnError."""
    B, L, D = int(B), int(L), int(D)
    dev, p = _nss_operands(y, x, weight, bias, scale, shift, B, L, D, ss_layout, RN_DTYPE_BF16,
                           RN_DTYPE_BF16, None)
    st = _lib.norm_scale_shift_fwd(*p[:6], B, L, D, int(flags), _layout(ss_layout), float(eps),
                                   _stream(stream, dev))
    if st != RN_OK:
        raise RnError(st, last_error())


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
