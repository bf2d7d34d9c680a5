"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/, each built here with the sanitizers and
run as a child process:
  * oracle_check.c: every oracle entry point on exactly sized heap buffers
    (all layouts, affine and output types, degenerate rows, invalid
    arguments, the elementwise helpers);
  * abi_check.cpp: the host side of the C ABI (validation, launch planning,
    the per-thread memo of the last validated call) with stand-ins for the two
    HIP runtime functions it calls, so successful calls are exercised without
    a GPU: a grid of valid problems, rejected calls, and a seeded fuzz of
    300,000 argument sets.
A sanitizer report makes the driver exit non-zero (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "rmsnorm_diffusion_transformers_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_check"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
          "-o", str(exe), os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "synth", "synth.c"), os.path.join(HERE, "oracle_check.c"), "-lm"])
    r = _run([str(exe)], env=ENV, timeout=600)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    # host-only compilation (no device code in these units); the sanitizers
    # apply to the host side only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(CSRC, "rn_api.hip"), os.path.join(CSRC, "rn_dispatch.hip"),
                os.path.join(HERE, "abi_check.cpp")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        _run([HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", *san,
              "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", str(obj)])
        objs.append(str(obj))
    exe = tmp_path / "abi_check"
    # linked without the HIP runtime: the driver defines the two functions the
    # host code calls
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", str(exe), *objs])
    r = _run([str(exe)], env=ENV, timeout=600)
    assert " 0 failures" in r.stdout
