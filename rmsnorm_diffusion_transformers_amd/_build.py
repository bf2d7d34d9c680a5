"""Build the gfx950 HIP libraries in-tree with hipcc.

librnorm.so: every translation unit under csrc/, compiled for gfx950 only, in
parallel, then linked into one shared library next to this file.
libtrafficref.so: the measurement reference under csrc/ref/ (a kernel with
the fused op's memory traffic and none of its arithmetic, which the
benchmark times beside the fused kernel); not part of the operation.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librnorm.so")
REF_LIB = os.path.join(HERE, "libtrafficref.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def ref_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "ref", "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(jobs: int | None = None) -> str:
    """Compile and link librnorm.so and libtrafficref.so; returns librnorm.so's
    path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs, refs = sources(), ref_sources()
    jobs = jobs or max(1, min(len(srcs) + len(refs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + refs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], REF_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
