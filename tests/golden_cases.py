"""Reader of tests/golden/worked_rows.txt: hand-worked rows of the operation,
each value a small dyadic number given in decimal, stored as bf16 bits (or as
binary32 values and FP8 codes where the case says so)."""
import os

import numpy as np

from util import bf16_of_exact

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "golden", "worked_rows.txt")
LAYOUTS = {"bcast": 0, "row": 1, "frame": 2}
TENSORS = ("x", "residual", "gate", "weight", "bias", "scale", "shift",
           "expect.residual_out", "expect.y", "expect.y_scale")


def _bf16(vals):
    return np.array([bf16_of_exact(float(v)) for v in vals], dtype=np.uint16)


def _f32(vals):
    out = []
    for v in vals:
        if "/" in v:                       # a quotient, rounded once to binary32
            num, den = v.split("/")
            out.append(np.float32(float(num) / float(den)))
        else:
            f = np.float32(v)
            assert float(f) == float(v), "%s is not a binary32 value" % v
            out.append(f)
    return np.array(out, dtype=np.float32)


def _finish(case):
    """Convert the raw value lists once every key of the case is known:
    binary32 weight/bias when `affine: f32`, binary32 or FP8 expected y when
    `out: f32` / `out: fp8`, bf16 bits otherwise."""
    case.setdefault("affine", "bf16")
    case.setdefault("out", "bf16")
    for key in TENSORS:
        if key not in case:
            continue
        vals = case[key]
        if key in ("weight", "bias") and case["affine"] == "f32":
            case[key] = _f32(vals)
        elif key == "expect.y" and case["out"] == "f32":
            case[key] = _f32(vals)
        elif key == "expect.y" and case["out"] == "fp8":
            case[key] = np.array([int(v, 16) for v in vals], dtype=np.uint8)
        elif key == "expect.y_scale":
            case[key] = _f32(vals)
        else:
            case[key] = _bf16(vals)


def load_cases(path=FIXTURE):
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("[") and line.endswith("]"):
            cur = {"name": line[1:-1]}
            cases.append(cur)
            continue
        key, val = (s.strip() for s in line.split(":", 1))
        assert cur is not None and key not in cur, (key, line)
        if key in TENSORS:
            cur[key] = val.split()
        elif key.startswith("layout."):
            parts = val.split()
            cur[key] = (LAYOUTS[parts[0]], int(parts[1]) if len(parts) > 1 else 0)
        elif key in ("B", "L", "D"):
            cur[key] = int(val)
        elif key == "eps":
            cur[key] = float(val)
        else:
            cur[key] = val
    for c in cases:
        _finish(c)
    return cases


Y_DTYPES = {"bf16": 0, "f32": 1, "fp8": 2}       # the oracle's Y_BF16, Y_F32, Y_FP8


def run_oracle(o, c):
    """The oracle on one case: (y, residual_out or None, y_scale or None)."""
    common = dict(B=c["B"], L=c["L"], D=c["D"], is_rms=c["norm"] == "rms",
                  ss_layout=c["layout.ss"], eps=c["eps"], affine_f32=c["affine"] == "f32",
                  y_dtype=Y_DTYPES[c["out"]])
    if c["op"] == "fused":
        out = o.fused(c["x"], c["residual"], c["gate"], c.get("weight"), c.get("bias"), c["scale"],
                      c["shift"], gate_layout=c["layout.gate"], **common)
        y, ro = out[0], out[1]
    else:
        out = o.nss(c["x"], c.get("weight"), c.get("bias"), c["scale"], c["shift"], **common)
        y, ro = out[0], None
    ys = out[-1] if c["out"] == "fp8" else None
    return y, ro, ys
