"""bench.py's host-side helpers (no GPU): the kernel-source digest that ties
the committed rocprof counter summary to the code it was measured on, and
the lookup of that summary."""
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _copy_sources(tmp_path):
    for p in bench.KERNEL_SOURCES:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)


def _digest_at(monkeypatch, root):
    monkeypatch.setattr(bench, "ROOT", str(root))
    return bench.kernel_digest()


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    base = _digest_at(monkeypatch, tmp_path)
    kernel = tmp_path / bench.KERNEL_SOURCES[0]
    text = kernel.read_text()
    # comments and blank lines only: same digest
    kernel.write_text("// a new comment line\n\n" + text.replace("// Position of one activation row",
                                                                  "/* moved */ // Position of an activation row"))
    assert _digest_at(monkeypatch, tmp_path) == base
    # a code change: new digest
    kernel.write_text(text.replace("constexpr int kPolicyStream = 2;", "constexpr int kPolicyStream = 3;"))
    assert "constexpr int kPolicyStream = 2;" in text
    assert _digest_at(monkeypatch, tmp_path) != base
    # so does a change in the shape table header
    kernel.write_text(text)
    args = tmp_path / bench.KERNEL_SOURCES[1]
    args.write_text(args.read_text().replace("constexpr int kPaceStores = 2;", "constexpr int kPaceStores = 3;"))
    assert _digest_at(monkeypatch, tmp_path) != base


def test_committed_traffic_matches_current_sources():
    """The committed counter summary was taken on the current kernel code, and
    its HBM bytes are within 0.5 % of the algorithmic bytes."""
    for wl in ("fused_ln_frame_b1_f49_l176400_d5120", "nss_ln_b1_l176400_d5120"):
        t = bench.measured_traffic(wl)
        assert t is not None, wl
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("workload "):
                tok = line.split()
                kv = dict(zip(tok[::2], tok[1::2]))
                assert kv["kernel_digest"] == bench.kernel_digest()
                hbm, alg = int(kv["hbm_bytes_per_launch"]), int(kv["algorithmic_bytes"])
                assert abs(hbm / alg - 1) < 0.005, line


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says why,
    before anything touches a device."""
    import subprocess
    import sys
    out = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "exactly one GPU" in out.stderr and "--gpus 2" in out.stderr
    assert out.stdout == ""


def test_traffic_reference_library_refuses_what_it_does_not_take():
    """The measurement reference (libtrafficref.so) loads without a GPU and
    refuses, before any launch, the arguments it does not take; an empty
    problem is a no-op."""
    import ctypes
    lib = ctypes.CDLL(bench.REF_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.rn_traffic_ref
    f.argtypes = [P] * 7 + [I64] * 4 + [P]
    f.restype = ctypes.c_int
    p = [4096 * (i + 1) for i in range(7)]
    assert f(*p, 1, 16, 4096, 1, None) == 1          # D other than 5120
    assert f(*p, 1, 16, 5120, 3, None) == 1          # L not a multiple of frames
    assert f(*p, 1, 16, 5120, 0, None) == 1          # no frames
    assert f(*p, -1, 16, 5120, 1, None) == 1
    assert f(*p, 1, 1 << 31, 5120, 1, None) == 1     # more than 2^31 - 1 rows
    assert f(*([None] * 7), 1, 16, 5120, 1, None) == 1
    assert f(*([None] * 7), 0, 16, 5120, 1, None) == 0   # empty: nothing launched
    g = lib.rn_traffic_ref_nss
    g.argtypes = [P] * 4 + [I64] * 3 + [P]
    g.restype = ctypes.c_int
    assert g(*p[:4], 1, 16, 2048, None) == 1
    assert g(*p[:4], 1, 1 << 31, 5120, None) == 1
    assert g(*p[:4], 1, -16, 5120, None) == 1
    assert g(*([None] * 4), 1, 16, 5120, None) == 1
    assert g(*([None] * 4), 1, 0, 5120, None) == 0
