"""The C ABI used without PyTorch: a C++ host program (hipcc, host code only)
allocates device memory with hipMalloc, creates its own stream, calls
resnorm_fused_fwd and norm_scale_shift_fwd through include/resnorm.h, and
writes the results to files that are compared with the oracle here."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_outputs, log, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROGRAM = r"""
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include "resnorm.h"

#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { \
  fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e), __LINE__); return 10; } } while (0)

static int load(const char* dir, const char* name, uint16_t* dst, size_t n) {
  char path[1024]; snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "rb"); if (!f) return 1;
  size_t got = fread(dst, 2, n, f); fclose(f); return got == n ? 0 : 1;
}
static int save(const char* dir, const char* name, const uint16_t* src, size_t n) {
  char path[1024]; snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "wb"); if (!f) return 1;
  size_t put = fwrite(src, 2, n, f); fclose(f); return put == n ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const char* dir = argv[1];
  const int64_t B = 1, L = atoll(argv[2]), D = atoll(argv[3]);
  const uint32_t flags = (uint32_t)atoi(argv[4]);
  const size_t n = (size_t)(B * L * D);
  uint16_t* h = (uint16_t*)malloc(n * 2);
  uint16_t* hrow = (uint16_t*)malloc((size_t)D * 2);
  void *x, *r, *g, *sc, *sh, *y, *ro, *yn;
  CK(hipMalloc(&x, n * 2)); CK(hipMalloc(&r, n * 2)); CK(hipMalloc(&y, n * 2));
  CK(hipMalloc(&ro, n * 2)); CK(hipMalloc(&yn, n * 2));
  CK(hipMalloc(&g, D * 2)); CK(hipMalloc(&sc, D * 2)); CK(hipMalloc(&sh, D * 2));
  if (load(dir, "x", h, n)) return 3;
  CK(hipMemcpy(x, h, n * 2, hipMemcpyHostToDevice));
  if (load(dir, "residual", h, n)) return 3;
  CK(hipMemcpy(r, h, n * 2, hipMemcpyHostToDevice));
  if (load(dir, "gate", hrow, D)) return 3;
  CK(hipMemcpy(g, hrow, D * 2, hipMemcpyHostToDevice));
  if (load(dir, "scale", hrow, D)) return 3;
  CK(hipMemcpy(sc, hrow, D * 2, hipMemcpyHostToDevice));
  if (load(dir, "shift", hrow, D)) return 3;
  CK(hipMemcpy(sh, hrow, D * 2, hipMemcpyHostToDevice));
  hipStream_t s;
  CK(hipStreamCreate(&s));
  rn_layout bc = {RN_BCAST, 0};
  rn_status st = resnorm_fused_fwd(y, ro, x, r, g, NULL, NULL, sc, sh, B, L, D, flags | RN_GATE,
                                   bc, bc, 1e-6f, (void*)s);
  if (st != RN_OK) { fprintf(stderr, "fused: %s\n", rn_last_error()); return 4; }
  st = norm_scale_shift_fwd(yn, x, NULL, NULL, sc, sh, B, L, D, flags, bc, 1e-6f, (void*)s);
  if (st != RN_OK) { fprintf(stderr, "nss: %s\n", rn_last_error()); return 4; }
  /* a refused call enqueues nothing and reports why */
  if (norm_scale_shift_fwd(yn, x, NULL, NULL, sc, sh, B, L, D + 4, flags, bc, 1e-6f, (void*)s) != RN_EINVAL)
    return 5;
  printf("refused as expected: %s\n", rn_last_error());
  CK(hipStreamSynchronize(s));
  CK(hipMemcpy(h, y, n * 2, hipMemcpyDeviceToHost));
  if (save(dir, "y", h, n)) return 6;
  CK(hipMemcpy(h, ro, n * 2, hipMemcpyDeviceToHost));
  if (save(dir, "residual_out", h, n)) return 6;
  CK(hipMemcpy(h, yn, n * 2, hipMemcpyDeviceToHost));
  if (save(dir, "y_nss", h, n)) return 6;
  CK(hipStreamDestroy(s));
  printf("%s\n", rn_version());
  return 0;
}
"""


@pytest.mark.parametrize("rms", [False, True])
def test_c_program_through_the_abi(tmp_path, rms):
    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    L, D = 96, 2560
    flags = rn.RN_RMS if rms else 0
    inp = {"x": synth.random_bf16((L, D), 61, 1), "residual": synth.random_bf16((L, D), 61, 2),
           "gate": synth.random_bf16((1, D), 61, 3, dist=synth.UNIFORM, a=0.0, b=1.0),
           "scale": synth.random_bf16((1, D), 61, 6, a=0.0, b=0.1),
           "shift": synth.random_bf16((1, D), 61, 7, a=0.0, b=0.1)}
    for k, v in inp.items():
        v.tofile(str(tmp_path / (k + ".bin")))
    src = tmp_path / "client.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "client"
    libdir = os.path.dirname(rn.LIB_PATH)
    log("compiling the C++ client (host code only)")
    subprocess.run([HIPCC, "-O2", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-lrnorm", "-Wl,-rpath," + libdir], check=True)
    log("running it: L=%d D=%d rms=%s" % (L, D, rms))
    out = subprocess.run([str(exe), str(tmp_path), str(L), str(D), str(flags)],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    assert "refused as expected" in out.stdout and "gfx950" in out.stdout
    read = lambda name: np.fromfile(str(tmp_path / (name + ".bin")), dtype=np.uint16).reshape(L, D)  # noqa: E731
    orc = oracle.Oracle()
    y_ref, ro_ref, _ = orc.fused(inp["x"], inp["residual"], inp["gate"], None, None, inp["scale"],
                                 inp["shift"], 1, L, D, rms)
    compare_outputs(read("y"), y_ref, read("residual_out"), ro_ref, "C client fused")
    yn_ref, _ = orc.nss(inp["x"], None, None, inp["scale"], inp["shift"], 1, L, D, rms)
    compare_outputs(read("y_nss"), yn_ref, what="C client norm-only")
