"""The shared input generator: determinism, counter-based addressing,
distributions and the stressed-row recipe."""
import numpy as np

import synth
from util import bf16_to_f64


def test_counter_based_and_deterministic():
    spec = synth.TensorSpec(synth.X, synth.NORMAL, 0.0, 1.0)
    a = synth.fill(spec, 7, 100000, threads=4)
    b = synth.fill(spec, 7, 100000, threads=1)
    assert np.array_equal(a, b)
    c = synth.fill(spec, 7, 1000, idx0=5000, threads=1)
    assert np.array_equal(a[5000:6000], c)
    d = synth.fill(spec, 8, 1000, threads=1)
    assert not np.array_equal(a[:1000], d)


def test_distributions():
    n = 1 << 20
    x = bf16_to_f64(synth.fill(synth.TensorSpec(1, synth.NORMAL, 0.0, 1.0), 3, n))
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    s = bf16_to_f64(synth.fill(synth.TensorSpec(6, synth.NORMAL, 0.0, 0.1), 3, n))
    assert abs(s.std() - 0.1) < 1e-3
    w = bf16_to_f64(synth.fill(synth.TensorSpec(4, synth.NORMAL, 1.0, 0.05), 3, n))
    assert abs(w.mean() - 1) < 2e-3 and abs(w.std() - 0.05) < 1e-3
    g = bf16_to_f64(synth.fill(synth.TensorSpec(3, synth.UNIFORM, 0.0, 1.0), 3, n))
    assert g.min() >= 0 and g.max() <= 1 and abs(g.mean() - 0.5) < 5e-3
    for arr in (x, s, w, g):
        assert np.all(np.isfinite(arr))


def test_no_negative_zero():
    bits = synth.fill(synth.TensorSpec(3, synth.UNIFORM, -1e-30, 1e-30), 3, 1 << 16)
    assert not np.any(bits == 0x8000)


def test_stressed_rows_recipe():
    wl = synth.WORKLOADS["fused_ln_b1_l90000_d5120"]
    rows = 20000
    flags = np.array([synth.row_stressed(wl, r) for r in range(rows)])
    assert 0.008 < flags.mean() < 0.012
    D = 64
    spec = synth.TensorSpec(synth.X, synth.NORMAL, 0.0, 1.0)
    plain = bf16_to_f64(synth.fill(spec, wl.wid, rows * D, row_len=D))
    stressed = bf16_to_f64(synth.fill(spec, wl.wid, rows * D, row_len=D, stress=wl.stress))
    ratio = np.abs(stressed).reshape(rows, D).mean(1) / np.abs(plain).reshape(rows, D).mean(1)
    assert np.allclose(ratio[flags], 50, rtol=0.02)
    assert np.allclose(ratio[~flags], 1)


def test_workload_table_matches_pages_shapes():
    w = synth.WORKLOADS
    c5 = w["fused_ln_frame_b1_f49_l176400_d5120"]
    assert c5.L == 49 * 3600 and c5.D == 5120 and c5.gate_layout == (synth.FRAME, 49)
    assert c5.algorithmic_bytes() == 7226849280
    assert w["nss_ln_b1_l176400_d5120"].algorithmic_bytes() == 3612692480
    assert w["fused_ln_b1_l90000_d5120"].algorithmic_bytes() == 3686430720
    assert w["fused_rms_w_b1_l90000_d10240"].algorithmic_bytes() == 11059240960
    assert w["fused_ln_b1_l16_d5120"].algorithmic_bytes() == 686080
    assert w["fused_rms_w_b2_l16_d10240"].algorithmic_bytes() == 3973120
    # the rest of the pages' speed matrix at D 5120
    assert w["fused_ln_b2_l16_d5120"].algorithmic_bytes() == 32 * 4 * 10240 + 3 * 10240
    assert w["nss_ln_b1_l16_d5120"].algorithmic_bytes() == 16 * 2 * 10240 + 2 * 10240
    assert w["nss_ln_b2_l16_d5120"].algorithmic_bytes() == 32 * 2 * 10240 + 2 * 10240
    assert w["nss_ln_b1_l90000_d5120"].algorithmic_bytes() == 90000 * 2 * 10240 + 2 * 10240
    assert len({x.wid for x in w.values()}) == len(w)     # one generator key space each
