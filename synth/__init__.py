"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the CPU oracle.

This module only draws numbers (see ``synth.c`` for the generator's
definition); it contains none of the normalisation arithmetic.  The workloads
below are the shapes the pages measure -- WAN2.2 T2V-A14B at 720p and 193
frames gives 49 latent frames x 3600 tokens = sequence 176400 at model width
5120 (sglang PR #36349, "Microbenchmark"); L=16 and L=90000 at D=5120 and a
D=10240 case are the pages' accuracy/speed matrix (sglang PR #33144,
"Accuracy Tests" and "Speed Tests and Profiling").  Synthetic Gaussian /
uniform activations stand in for real model activations; no dataset is used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

SEED = 42  # the pages' end-to-end seed (sglang PR #36349, "Command")

NORMAL, UNIFORM = 0, 1
BCAST, ROW, FRAME = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (plain C, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                        "-ffp-contract=off", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_int64, ctypes.c_double, ctypes.c_double]
        lib.synth_fill.restype = None
        lib.synth_row_stressed.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                           ctypes.c_double]
        lib.synth_row_stressed.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class TensorSpec:
    """One input tensor of a workload: its generator stream and distribution."""
    tensor_id: int
    dist: int
    a: float
    b: float


# Tensor ids inside a workload's key space.
X, RES, GATE, WEIGHT, BIAS, SCALE, SHIFT = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class Workload:
    """A problem instance: op, flags, shape, layouts and input distributions."""
    name: str
    wid: int
    op: str                      # "fused" or "nss"
    is_rms: bool
    B: int
    L: int
    D: int
    gate_layout: tuple | None    # (kind, frames) or None when there is no gate
    ss_layout: tuple             # (kind, frames)
    has_weight: bool = False
    has_bias: bool = False
    eps: float = 1e-6
    stress: tuple | None = None  # (probability, factor) for x and residual rows
    dists: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return self.B * self.L

    def mod_rows(self, layout) -> int:
        kind, frames = layout
        return {BCAST: 1, ROW: self.R, FRAME: self.B * frames}[kind]

    def algorithmic_bytes(self) -> int:
        """Every operand read once plus every output written once (bf16)."""
        n = 0
        per_row = 2 * self.D
        n += self.R * per_row            # x
        n += self.R * per_row            # y
        if self.op == "fused":
            n += 2 * self.R * per_row    # residual in, residual out
            if self.gate_layout is not None:
                n += self.mod_rows(self.gate_layout) * per_row
        n += 2 * self.mod_rows(self.ss_layout) * per_row
        if self.has_weight:
            n += per_row
        if self.has_bias:
            n += per_row
        return n


def _std_dists(**over):
    d = {X: TensorSpec(X, NORMAL, 0.0, 1.0), RES: TensorSpec(RES, NORMAL, 0.0, 1.0),
         GATE: TensorSpec(GATE, UNIFORM, 0.0, 1.0), WEIGHT: TensorSpec(WEIGHT, NORMAL, 1.0, 0.05),
         BIAS: TensorSpec(BIAS, NORMAL, 0.0, 0.1), SCALE: TensorSpec(SCALE, NORMAL, 0.0, 0.1),
         SHIFT: TensorSpec(SHIFT, NORMAL, 0.0, 0.1)}
    d.update(over)
    return d


WORKLOADS = {w.name: w for w in [
    Workload("fused_ln_b1_l16_d5120", 1, "fused", False, 1, 16, 5120, (BCAST, 0), (BCAST, 0),
             dists=_std_dists()),
    Workload("fused_ln_b1_l90000_d5120", 2, "fused", False, 1, 90000, 5120, (BCAST, 0), (BCAST, 0),
             stress=(0.01, 50.0), dists=_std_dists()),
    Workload("fused_rms_w_b2_l16_d10240", 3, "fused", True, 2, 16, 10240, (BCAST, 0), (ROW, 0),
             has_weight=True, dists=_std_dists()),
    Workload("fused_rms_w_b1_l90000_d10240", 4, "fused", True, 1, 90000, 10240, (BCAST, 0), (ROW, 0),
             has_weight=True, dists=_std_dists()),
    Workload("nss_ln_b1_l176400_d5120", 5, "nss", False, 1, 176400, 5120, None, (BCAST, 0),
             dists=_std_dists()),
    Workload("fused_ln_frame_b1_f49_l176400_d5120", 6, "fused", False, 1, 176400, 5120,
             (FRAME, 49), (FRAME, 49), dists=_std_dists()),
    # the rest of the speed matrix (sglang PR #33144, "Speed Tests and
    # Profiling": B1-L16, B2-L16 and B1-L90000 at D 5120 for both ops)
    Workload("fused_ln_b2_l16_d5120", 7, "fused", False, 2, 16, 5120, (BCAST, 0), (BCAST, 0),
             dists=_std_dists()),
    Workload("nss_ln_b1_l16_d5120", 8, "nss", False, 1, 16, 5120, None, (BCAST, 0),
             dists=_std_dists()),
    Workload("nss_ln_b2_l16_d5120", 9, "nss", False, 2, 16, 5120, None, (BCAST, 0),
             dists=_std_dists()),
    Workload("nss_ln_b1_l90000_d5120", 10, "nss", False, 1, 90000, 5120, None, (BCAST, 0),
             dists=_std_dists()),
]}


def fill(spec: TensorSpec, wid: int, n: int, idx0: int = 0, row_len: int = 0,
         stress: tuple | None = None, threads: int | None = None,
         seed: int = SEED) -> np.ndarray:
    """Elements idx0 .. idx0+n-1 of one tensor stream as bf16 bits (uint16)."""
    lib = _load()
    out = np.empty(n, dtype=np.uint16)
    sp, sm = stress if stress else (0.0, 1.0)
    threads = threads or default_threads()
    chunk = max(1 << 20, (n + threads - 1) // threads)

    def work(j0):
        j1 = min(n, j0 + chunk)
        lib.synth_fill(out.ctypes.data + 2 * j0, j1 - j0, idx0 + j0, seed, wid, spec.tensor_id,
                       spec.dist, spec.a, spec.b, row_len, sp, sm)

    starts = list(range(0, n, chunk))
    if len(starts) <= 1:
        for j0 in starts:
            work(j0)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, starts))
    return out


def row_stressed(wl: Workload, row: int, seed: int = SEED) -> bool:
    if not wl.stress:
        return False
    return bool(_load().synth_row_stressed(seed, wl.wid, row, wl.stress[0]))


def make_inputs(wl: Workload, threads: int | None = None, seed: int = SEED) -> dict:
    """All inputs of a workload as uint16 bf16-bit arrays.

    Activations are [R, D]; modulation tensors are [rows_of_layout, D];
    weight/bias are [D].  Missing operands are absent from the dict.
    """
    R, D = wl.R, wl.D
    d = wl.dists
    out = {}
    out["x"] = fill(d[X], wl.wid, R * D, row_len=D, stress=wl.stress, threads=threads,
                    seed=seed).reshape(R, D)
    if wl.op == "fused":
        out["residual"] = fill(d[RES], wl.wid, R * D, row_len=D, stress=wl.stress,
                               threads=threads, seed=seed).reshape(R, D)
        if wl.gate_layout is not None:
            g = wl.mod_rows(wl.gate_layout)
            out["gate"] = fill(d[GATE], wl.wid, g * D, threads=threads, seed=seed).reshape(g, D)
    m = wl.mod_rows(wl.ss_layout)
    out["scale"] = fill(d[SCALE], wl.wid, m * D, threads=threads, seed=seed).reshape(m, D)
    out["shift"] = fill(d[SHIFT], wl.wid, m * D, threads=threads, seed=seed).reshape(m, D)
    if wl.has_weight:
        out["weight"] = fill(d[WEIGHT], wl.wid, D, threads=threads, seed=seed)
    if wl.has_bias:
        out["bias"] = fill(d[BIAS], wl.wid, D, threads=threads, seed=seed)
    return out


def random_bf16(shape, seed: int, tensor: int, dist: int = NORMAL, a: float = 0.0,
                b: float = 1.0, workload: int = 1000) -> np.ndarray:
    """A small seeded tensor for ad-hoc test cases (same generator, own key)."""
    n = int(np.prod(shape)) if len(shape) else 1
    return fill(TensorSpec(tensor, dist, a, b), workload, n, seed=seed, threads=1).reshape(shape)

