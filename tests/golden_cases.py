"""Reader of tests/golden/worked_rows.txt: hand-worked rows of the operation,
each value a small dyadic number given in decimal and stored as bf16 bits."""
import os

import numpy as np

from util import bf16_of_exact

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "golden", "worked_rows.txt")
LAYOUTS = {"bcast": 0, "row": 1, "frame": 2}
TENSORS = ("x", "residual", "gate", "weight", "bias", "scale", "shift",
           "expect.residual_out", "expect.y")


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
            vals = [float(v) for v in val.split()]
            cur[key] = np.array([bf16_of_exact(v) for v in vals], dtype=np.uint16)
        elif key.startswith("layout."):
            parts = val.split()
            cur[key] = (LAYOUTS[parts[0]], int(parts[1]) if len(parts) > 1 else 0)
        elif key in ("B", "L", "D"):
            cur[key] = int(val)
        elif key == "eps":
            cur[key] = float(val)
        else:
            cur[key] = val
    return cases
