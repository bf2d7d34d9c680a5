"""The C-ABI library on the CPU (no GPU here): it loads, exports every entry
point include/resnorm.h declares, and rejects every invalid argument on the
host with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "resnorm.h")


@pytest.fixture(scope="module")
def rn():
    import rmsnorm_diffusion_transformers_amd as rn
    return rn


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                                 r"([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("resnorm_fused_fwd", "norm_scale_shift_fwd", "rn_last_error",
              "rn_describe_launch", "rn_describe_launch_ex", "rn_version"):
        assert n in names, names


def test_library_exports_every_declared_symbol(rn):
    lib = ctypes.CDLL(rn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), "librnorm.so does not export %s" % name


def test_version(rn):
    assert "gfx950" in rn.version()


# Fake, 16-byte aligned, non-overlapping "device" addresses: validation never
# dereferences them and every call below fails before any device work.
A = 1 << 40
STRIDE = 1 << 32


def addr(i):
    return A + i * STRIDE


def fused(rn, **kw):
    args = dict(y=addr(0), residual_out=addr(1), x=addr(2), residual=addr(3), gate=addr(4),
                weight=None, bias=None, scale=addr(7), shift=addr(8), B=1, L=16, D=5120,
                flags=rn.RN_GATE, gate_layout=(rn.RN_BCAST, 0), ss_layout=(rn.RN_BCAST, 0),
                eps=1e-6)
    args.update(kw)
    st = rn._lib.resnorm_fused_fwd(args["y"], args["residual_out"], args["x"], args["residual"],
                                   args["gate"], args["weight"], args["bias"], args["scale"],
                                   args["shift"], args["B"], args["L"], args["D"], args["flags"],
                                   rn._layout(args["gate_layout"]), rn._layout(args["ss_layout"]),
                                   args["eps"], None)
    return st, rn.last_error()


def nss(rn, **kw):
    args = dict(y=addr(0), x=addr(2), weight=None, bias=None, scale=addr(7), shift=addr(8), B=1,
                L=16, D=5120, flags=0, ss_layout=(rn.RN_BCAST, 0), eps=1e-6)
    args.update(kw)
    st = rn._lib.norm_scale_shift_fwd(args["y"], args["x"], args["weight"], args["bias"],
                                      args["scale"], args["shift"], args["B"], args["L"],
                                      args["D"], args["flags"], rn._layout(args["ss_layout"]),
                                      args["eps"], None)
    return st, rn.last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(y=None), 1, "y is NULL"),
    (dict(x=None), 1, "x is NULL"),
    (dict(residual=None), 1, "residual is NULL"),
    (dict(residual_out=None), 1, "residual_out is NULL"),
    (dict(scale=None), 1, "scale is NULL"),
    (dict(shift=None), 1, "shift is NULL"),
    (dict(gate=None), 1, "RN_GATE set but gate is NULL"),
    (dict(flags=0), 1, "gate given but RN_GATE not set"),
    (dict(weight=addr(5)), 1, "weight given"),
    (dict(flags=2 | 4), 1, "RN_WEIGHT set but weight is NULL"),
    (dict(flags=2 | 8, bias=addr(6)), 1, "RN_BIAS requires RN_WEIGHT"),
    (dict(flags=2 | 4 | 8, weight=addr(5)), 1, "RN_BIAS set but bias is NULL"),
    (dict(flags=2 | 64), 1, "unknown flag"),
    (dict(D=5121), 1, "multiple of 8"),
    (dict(D=0), 1, "multiple of 8"),
    (dict(D=4), 1, "multiple of 8"),
    (dict(D=16392), 2, "RN_D_MAX"),
    (dict(B=-1), 1, "negative"),
    (dict(L=-5), 1, "negative"),
    (dict(B=1 << 20, L=1 << 12), 2, "2^31"),
    (dict(B=1, L=1 << 31), 2, "2^31"),
    (dict(eps=-1e-6), 1, "eps"),
    (dict(eps=float("nan")), 1, "eps"),
    (dict(eps=float("inf")), 1, "eps"),
    (dict(x=addr(2) + 8), 1, "x is not 16-byte aligned"),
    (dict(gate=addr(4) + 2), 1, "gate is not 16-byte aligned"),
    (dict(gate_layout=(7, 0)), 1, "gate layout kind"),
    (dict(ss_layout=(-1, 0)), 1, "scale/shift layout kind"),
    (dict(ss_layout=(2, 0)), 1, "frames >= 1"),
    (dict(ss_layout=(2, 5)), 1, "L % frames"),
    (dict(gate_layout=(2, 3)), 1, "L % frames"),
    (dict(y=addr(2) + 16), 1, "y overlaps x"),
    (dict(y=addr(3)), 1, "y overlaps residual"),
    (dict(residual_out=addr(2)), 1, "residual_out overlaps x"),
    (dict(residual_out=addr(0)), 1, "overlaps"),
    (dict(y=addr(7)), 1, "y overlaps scale"),
    (dict(residual_out=addr(3) + 32), 1, "residual_out overlaps residual"),
])
def test_fused_rejects(rn, kw, status, msg):
    st, err = fused(rn, **kw)
    assert st == status, (st, err)
    assert msg in err, err


@pytest.mark.parametrize("kw,status,msg", [
    (dict(flags=2), 1, "RN_GATE is only valid"),
    (dict(y=None), 1, "y is NULL"),
    (dict(D=12), 1, "multiple of 8"),
    (dict(D=32768), 2, "RN_D_MAX"),
    (dict(flags=4), 1, "RN_WEIGHT set but weight is NULL"),
    (dict(ss_layout=(2, 3)), 1, "L % frames"),
    (dict(y=addr(8)), 1, "y overlaps shift"),
])
def test_nss_rejects(rn, kw, status, msg):
    st, err = nss(rn, **kw)
    assert st == status, (st, err)
    assert msg in err, err


def test_empty_problem_is_ok_without_launch(rn):
    assert fused(rn, B=0)[0] == 0
    assert fused(rn, L=0)[0] == 0
    assert nss(rn, B=3, L=0)[0] == 0
    # an empty problem is still validated
    assert fused(rn, B=0, D=7)[0] == 1


def test_status_mapping_in_binding(rn):
    with pytest.raises(rn.RnError) as e:
        rn.resnorm_fused_fwd(addr(0), addr(1), addr(2), addr(3), None, None, None, addr(7),
                             addr(8), 1, 16, 100, 0, stream=0)
    assert e.value.status == rn.RN_EINVAL and "multiple of 8" in str(e.value)


def plan_of(rn, R, D):
    i = rn.describe_launch(1, R, D, 0, False)
    return i["waves_per_row"], i["vec_per_lane"]


def test_describe_launch(rn):
    """The planner: for large problems the smallest waves-per-row that covers
    D within the register budget (vectors per lane x row operands <= 52); for
    a few hundred rows, rows split over 2-10 waves; ten waves when per-row
    modulation adds HBM streams."""
    info = rn.describe_launch(1, 176400, 5120, rn.RN_GATE, True)
    assert (info["waves_per_row"], info["vec_per_lane"]) == (1, 10)
    assert info["block_threads"] == 256 and info["rows_per_block"] == 4
    assert info["grid_blocks"] == 176400 // 4
    c3 = rn.describe_launch(1, 90000, 10240, rn.RN_GATE | rn.RN_RMS | rn.RN_WEIGHT, True,
                            (rn.RN_BCAST, 0), (rn.RN_ROW, 0))
    assert (c3["waves_per_row"], c3["vec_per_lane"], c3["rows_per_block"]) == (10, 2, 1)
    assert c3["grid_blocks"] == 90000 and c3["block_threads"] == 640
    c3b = rn.describe_launch(1, 90000, 10240, rn.RN_GATE | rn.RN_RMS | rn.RN_WEIGHT)
    assert (c3b["waves_per_row"], c3b["vec_per_lane"], c3b["rows_per_block"]) == (4, 5, 1)
    c5 = rn.describe_launch(1, 176400, 5120, rn.RN_GATE, True, (rn.RN_FRAME, 49), (rn.RN_FRAME, 49))
    c1 = rn.describe_launch(1, 16, 5120, rn.RN_GATE, True)
    assert (c1["waves_per_row"], c1["vec_per_lane"]) == (10, 1)
    assert (c5["waves_per_row"], c5["vec_per_lane"]) == (1, 10)
    small_row = rn.describe_launch(1, 8, 1024, rn.RN_GATE, True, (rn.RN_ROW, 0), (rn.RN_ROW, 0))
    assert small_row["waves_per_row"] == 1
    nss = rn.describe_launch(1, 176400, 5120, 0, False)
    assert (nss["waves_per_row"], nss["vec_per_lane"]) == (1, 10)
    assert rn.describe_launch(1, 3, 8, 0, False)["vec_per_lane"] == 1
    assert rn.describe_launch(1, 3, 1000, 0, False)["vec_per_lane"] == 2
    big = rn.describe_launch(1, 3000, 16384, 0, False)
    assert (big["waves_per_row"], big["vec_per_lane"]) == (4, 8)
    mid = rn.describe_launch(1, 3000, 8192, rn.RN_GATE | rn.RN_WEIGHT | rn.RN_BIAS, True)
    assert (mid["waves_per_row"], mid["vec_per_lane"]) == (4, 4)
    # a few rows are latency-bound: ten one-vector waves for D in (4096, 5120]
    tiny = rn.describe_launch(1, 16, 5120, rn.RN_GATE, True)
    assert (tiny["waves_per_row"], tiny["vec_per_lane"], tiny["grid_blocks"]) == (10, 1, 16)
    assert plan_of(rn, 3, 16384) == (4, 8)
    assert rn.describe_launch(1, 128, 5120, 0, False)["waves_per_row"] == 10
    # a few hundred rows: rows split so that each wave holds 2-5 vectors per lane
    plan = lambda R, D: plan_of(rn, R, D)  # noqa: E731
    assert plan(129, 5120) == (4, 3)
    assert plan(256, 2048) == (4, 2) and plan(256, 10240) == (4, 5)
    assert plan(257, 3072) == (2, 3) and plan(768, 3072) == (2, 3)
    assert plan(512, 2048) == (2, 3) and plan(513, 2048) == (1, 4)
    assert plan(768, 5120) == (4, 3) and plan(769, 5120) == (2, 5)
    assert plan(1536, 4096) == (2, 4) and plan(1537, 4096) == (1, 8)
    assert plan(1536, 2048) == (1, 4) and plan(1000, 2040) == (1, 4)
    assert plan(100, 2040) == (1, 4)
    assert plan(16, 2552) == (4, 2)
    # the fused op keeps one wave per row from 513 to 1024 rows where it fits
    fplan = lambda R, D: tuple(rn.describe_launch(1, R, D, rn.RN_GATE, True)[k]  # noqa: E731
                               for k in ("waves_per_row", "vec_per_lane"))
    assert fplan(512, 5120) == (4, 3) and fplan(513, 5120) == (1, 10)
    assert fplan(1024, 5120) == (1, 10) and fplan(1025, 5120) == (2, 5)
    assert fplan(768, 6144) == (4, 3)
    # the fused op with one wave per row keeps weight/bias in LDS, so only its
    # 5 row operands count: one wave per row up to D = 5120 for every affine
    # type; with two or more waves per row weight/bias take registers
    # (binary32 counting twice)
    wb = rn.RN_GATE | rn.RN_WEIGHT | rn.RN_BIAS
    for D, want in ((5120, (1, 10)), (3072, (1, 6)), (2048, (1, 4))):
        for adt in (rn.RN_DTYPE_BF16, rn.RN_DTYPE_F32):
            i = rn.describe_launch(1, 176400, D, wb, True, affine_dtype=adt)
            assert (i["waves_per_row"], i["vec_per_lane"]) == want, (D, adt)
    a32 = rn.describe_launch(1, 110250, 8192, wb, True, affine_dtype=rn.RN_DTYPE_F32)
    assert (a32["waves_per_row"], a32["vec_per_lane"]) == (4, 4)     # 9 x 8 > 52 at W = 2
    a16 = rn.describe_launch(1, 110250, 8192, wb, True)
    assert (a16["waves_per_row"], a16["vec_per_lane"]) == (4, 4)     # 7 x 8 > 52 at W = 2
    # and from 513 to 1024 rows (the fused op's one-wave band)
    assert rn.describe_launch(1, 1024, 5120, wb, True,
                              affine_dtype=rn.RN_DTYPE_F32)["waves_per_row"] == 1
    with pytest.raises(rn.RnError):
        rn.describe_launch(1, 16, 5120, 0, False, affine_dtype=7)
    assert rn.describe_launch(2, 5, 8, 0, False)["grid_blocks"] == 3
    for D in range(8, 16385, 8):
        for fused, flags, gl, sl in ((False, 0, (0, 0), (0, 0)), (True, 14, (1, 0), (1, 0))):
            i = rn.describe_launch(1, 1, D, flags, fused, gl, sl)
            assert 64 * i["waves_per_row"] * i["vec_per_lane"] * 8 >= D
            assert i["block_threads"] == 64 * i["waves_per_block"] <= 1024
    with pytest.raises(rn.RnError):
        rn.describe_launch(1, 3, 20000, 0, False)


def test_describe_launch_norm_affine_budget(rn):
    """The norm-only op with weight keeps weight and bias live with the whole
    row, so it gets a tighter register budget (VPT x operands <= 48): with
    bf16 weight + bias or a binary32 weight (5 operand vectors per VPT) it
    leaves one wave x 10 vectors for two x 5 at D 4608-5120 and two x 10 for
    four x 5 at D 8704-10240; the fused op keeps its shapes."""
    ROW = (rn.RN_ROW, 0)
    WB = rn.RN_WEIGHT | rn.RN_BIAS
    def plan(D, flags, fused=False, adt=rn.RN_DTYPE_BF16, sl=ROW):
        i = rn.describe_launch(1, 176400, D, flags, fused, (rn.RN_BCAST, 0), sl, affine_dtype=adt)
        return i["waves_per_row"], i["vec_per_lane"], i["rows_per_wave"]
    assert plan(5120, WB) == (2, 5, 1)
    assert plan(5120, rn.RN_WEIGHT, adt=rn.RN_DTYPE_F32) == (2, 5, 1)
    assert plan(4096, WB) == (1, 8, 1)                     # 5 x 8 = 40: one wave still fits
    assert plan(10240, WB) == (4, 5, 1)
    assert plan(10240, rn.RN_WEIGHT, adt=rn.RN_DTYPE_F32) == (4, 5, 1)
    assert plan(5120, rn.RN_WEIGHT) == (1, 10, 1)         # 4 operand vectors: 40
    assert plan(5120, 0) == (1, 10, 1)
    # fused, broadcast scale/shift: 5 x 10 = 50 <= 52
    assert plan(5120, rn.RN_WEIGHT, fused=True, sl=(rn.RN_BCAST, 0)) == (1, 10, 1)


def test_describe_launch_norm_only_eight_vectors(rn):
    """Large norm-only problems without affine take 8 vectors per lane where
    the first fit would be 6 (2 or 4 waves per row); the fused op, the
    norm-only op with weight and small problems keep their shapes."""
    def plan(R, D, flags=0, fused=False):
        i = rn.describe_launch(1, R, D, flags, fused)
        return i["waves_per_row"], i["vec_per_lane"]
    assert plan(147000, 6144) == (2, 8)
    assert plan(160000, 5632) == (2, 8)
    assert plan(73500, 12288) == (4, 8)
    assert plan(80000, 10752) == (4, 8)
    assert plan(147000, 6144, rn.RN_GATE, True) == (2, 6)
    i = rn.describe_launch(1, 147000, 6144, rn.RN_WEIGHT, False, (rn.RN_BCAST, 0), (rn.RN_ROW, 0))
    assert (i["waves_per_row"], i["vec_per_lane"]) == (2, 6)   # with weight (per-row scale/shift)
    assert plan(512, 6144) != (2, 8)
    assert plan(176400, 5120) == (1, 10)


def test_describe_launch_pow2_fused(rn):
    """The fused op with rows a multiple of 8 KB apart (D % 4096 == 0) takes
    at least two waves per row (two waves x 4 vectors at D = 4096, with or
    without affine); the norm-only op and other widths are unchanged."""
    def plan(R, D, flags, fused, adt=rn.RN_DTYPE_BF16):
        i = rn.describe_launch(1, R, D, flags, fused, affine_dtype=adt)
        return i["waves_per_row"], i["vec_per_lane"]
    G, WB = rn.RN_GATE, rn.RN_WEIGHT | rn.RN_BIAS
    assert plan(220500, 4096, G, True) == (2, 4)
    assert plan(220500, 4096, G | WB, True, rn.RN_DTYPE_F32) == (2, 4)
    assert plan(220500, 4096, 0, True) == (2, 4)
    assert plan(800, 4096, G, True) == (2, 4)            # the one-wave band too
    assert plan(220500, 4096, 0, False) == (1, 8)        # norm-only: unchanged
    assert plan(441000, 2048, G, True) == (1, 4)         # 4 KB rows: one wave
    assert plan(176400, 5120, G, True) == (1, 10)        # the headline
    for D in range(4096, 16385, 4096):
        for R in (64, 700, 3000, 100000):
            assert plan(R, D, G, True)[0] >= 2, (R, D)


def test_describe_launch_multi_row(rn):
    """The norm-only op with weight from 12 Mi elements: one wave streams 4
    consecutive rows through weight, bias, scale and shift loaded once, on
    the first multi-row shape that covers D (at most 5 vectors per lane),
    when every aligned group of 4 rows shares its scale/shift row."""
    W, WB = rn.RN_WEIGHT, rn.RN_WEIGHT | rn.RN_BIAS
    def k_of(B, L, D, flags, fused=False, sl=(rn.RN_BCAST, 0), **kw):
        i = rn.describe_launch(B, L, D, flags, fused, (rn.RN_BCAST, 0), sl, **kw)
        return i["waves_per_row"], i["vec_per_lane"], i["rows_per_wave"]
    i = rn.describe_launch(1, 176400, 5120, WB, False, affine_dtype=rn.RN_DTYPE_F32)
    assert (i["waves_per_row"], i["vec_per_lane"], i["rows_per_wave"]) == (2, 5, 4)
    assert i["rows_per_block"] == 8 and i["block_threads"] == 256
    assert i["grid_blocks"] == 176400 // 8
    assert k_of(1, 176400, 5120, W) == (2, 5, 4)
    assert k_of(1, 441000, 2048, WB) == (1, 4, 4)
    assert k_of(1, 294000, 3072, WB) == (2, 3, 4)
    assert k_of(1, 110250, 8192, WB) == (4, 4, 4)
    assert k_of(1, 90000, 10240, W) == (4, 5, 4)
    assert k_of(1, 90000, 10248, W)[2] == 1          # no multi-row shape covers it
    assert k_of(1, 786432, 16, W) == (1, 1, 4)
    assert k_of(1, 786431, 16, W)[2] == 1
    # not for the fused op, nor without weight, nor below 12 Mi elements
    assert k_of(1, 176400, 5120, WB, True)[2] == 1
    assert k_of(1, 176400, 5120, 0) == (1, 10, 1)
    assert k_of(1, 2457, 5120, W)[2] == 1 and k_of(1, 2458, 5120, W)[2] == 4
    assert k_of(2, 1229, 5120, W)[2] == 4 and k_of(3, 819, 5120, W)[2] == 1
    # scale/shift rows shared by every aligned group of 4 rows
    frame = lambda F: (rn.RN_FRAME, F)  # noqa: E731
    assert k_of(1, 176400, 5120, W, sl=frame(49))[2] == 4      # 3600 tokens per frame
    assert k_of(1, 176400, 5120, W, sl=frame(16))[2] == 1      # 11025 tokens per frame
    assert k_of(2, 8196, 5120, W, sl=frame(1))[2] == 4          # per batch, L % 4 == 0
    assert k_of(2, 8194, 5120, W, sl=frame(1))[2] == 1          # per batch, L % 4 == 2
    assert k_of(1, 176400, 5120, W, sl=(rn.RN_ROW, 0))[2] == 1
    with pytest.raises(rn.RnError, match="frames >= 1"):
        k_of(1, 176400, 5120, W, sl=frame(0))                    # refused, as a launch would be
    with pytest.raises(rn.RnError, match="L % frames == 0"):
        k_of(1, 176400, 5120, W, sl=frame(17))
    for D in range(8, 10241, 8):
        i = rn.describe_launch(1, -(-(12 << 20) // D), D, WB, False)
        assert i["rows_per_wave"] == 4 and i["vec_per_lane"] <= 5
        assert 64 * i["waves_per_row"] * i["vec_per_lane"] * 8 >= D
        assert i["rows_per_block"] == 4 * i["waves_per_block"] // i["waves_per_row"]


def test_multi_row_groups_share_modulation_rows(rn):
    """Whenever the planner gives a problem four rows per wave, every aligned
    group of four rows maps to one scale/shift row (the index each row takes
    from its layout: broadcast 0, per row r, per frame b * F + l // (L / F));
    and a norm-only problem with weight of at least 12 Mi elements whose width
    a multi-row shape covers gets one whenever its groups share their rows --
    except per-frame layouts whose frame length is not a multiple of 4, which
    the planner refuses from the layout alone (their groups can still share
    rows by chance, e.g. with one batch)."""
    import numpy as np
    rng = np.random.default_rng(11)
    BC, ROW, FR = rn.RN_BCAST, rn.RN_ROW, rn.RN_FRAME
    checked = 0
    for _ in range(400):
        B = int(rng.integers(1, 5))
        F = int(rng.choice([1, 2, 3, 5, 7, 49]))
        tpf = int(rng.integers(1, 4000))
        L = F * tpf
        D = int(rng.integers(1, 1281)) * 8
        kind = int(rng.integers(0, 3))
        lay = (kind, F if kind == FR else 0)
        flags = rn.RN_WEIGHT | (rn.RN_BIAS if rng.random() < 0.5 else 0)
        if B * L >= 2 ** 31:
            continue
        i = rn.describe_launch(B, L, D, flags, False, (BC, 0), lay)
        R = B * L
        r = np.arange(R)
        b, l = r // L, r % L
        srow = {BC: np.zeros(R, np.int64), ROW: r, FR: b * F + l // tpf}[kind]
        n = (R // 4) * 4
        groups_share = bool(np.all(srow[:n].reshape(-1, 4) == srow[:n].reshape(-1, 4)[:, :1])) \
            and (R % 4 == 0 or bool(np.all(srow[n:] == srow[n])))
        if i["rows_per_wave"] == 4:
            assert groups_share, (B, L, D, lay)
            checked += 1
        elif R * D >= 12 << 20 and D <= 10240 and kind != ROW:
            assert not groups_share or kind == FR and tpf % 4 != 0, (B, L, D, lay)
    assert checked > 50


def test_layout_inference(rn):
    import torch
    B, L, D = 2, 12, 16
    f = lambda *s: torch.empty(*s)
    assert rn.infer_layout(f(D), B, L, D) == (rn.RN_BCAST, 0)
    assert rn.infer_layout(f(1, D), B, L, D) == (rn.RN_BCAST, 0)
    assert rn.infer_layout(f(1, 1, D), B, L, D) == (rn.RN_BCAST, 0)
    assert rn.infer_layout(f(B, L, D), B, L, D) == (rn.RN_ROW, 0)
    assert rn.infer_layout(f(B, 3, 1, D), B, L, D) == (rn.RN_FRAME, 3)
    assert rn.infer_layout(f(B, D), B, L, D) == (rn.RN_FRAME, 1)
    assert rn.infer_layout(f(B, 1, D), B, L, D) == (rn.RN_FRAME, 1)
    with pytest.raises(ValueError):
        rn.infer_layout(f(3, D), B, L, D)


def test_no_cpu_path(rn):
    import torch
    x = torch.zeros(1, 2, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="no CPU path"):
        rn.norm_scale_shift(x, None, None, torch.zeros(8, dtype=torch.bfloat16),
                            torch.zeros(8, dtype=torch.bfloat16), "layer", 1e-6, stream=0)


def test_binding_checks_tensor_sizes_and_devices(rn):
    """The tensor wrappers refuse tensors smaller than the sizes and layouts
    make the kernel touch, and operands on different devices, before any
    library call (CPU tensors: the checks run first, no GPU needed)."""
    import torch
    bf = dict(dtype=torch.bfloat16)
    x = torch.zeros(2 * 3 * 8, **bf)
    small = torch.zeros(2 * 3 * 8 - 1, **bf)
    row = torch.zeros(8, **bf)
    with pytest.raises(ValueError, match="y has 47 elements"):
        rn.norm_scale_shift_fwd(small, x, None, None, row, row, 2, 3, 8, 0, stream=0)
    with pytest.raises(ValueError, match="scale has 8 elements; the sizes and layout need 48"):
        rn.norm_scale_shift_fwd(x, x, None, None, row, row, 2, 3, 8, 0, (rn.RN_ROW, 0), stream=0)
    with pytest.raises(ValueError, match="gate has 8 elements; the sizes and layout need 48"):
        rn.resnorm_fused_fwd(x, x.clone(), x, x.clone(), row, None, None, row, row, 2, 3, 8,
                             rn.RN_GATE, (rn.RN_FRAME, 3), (rn.RN_BCAST, 0), stream=0)
    with pytest.raises(ValueError, match="y_scale has 5 elements"):
        rn.norm_scale_shift_fwd_ex(torch.zeros(48, dtype=torch.float8_e4m3fn), x, None, None, row,
                                   row, 2, 3, 8, 0, y_dtype=rn.RN_DTYPE_FP8_E4M3,
                                   y_scale=torch.zeros(5), stream=0)
    with pytest.raises(ValueError, match="weight has 4 elements"):
        rn.norm_scale_shift_fwd_ex(x, x, torch.zeros(4), None, row, row, 2, 3, 8, rn.RN_WEIGHT,
                                   affine_dtype=rn.RN_DTYPE_F32, stream=0)
    with pytest.raises(ValueError, match="is on meta but other operands are on cpu"):
        rn.norm_scale_shift_fwd(x, x, None, None, row, torch.zeros(8, device="meta", **bf), 2, 3,
                                8, 0, stream=0)
    # int addresses are the C ABI's business: passed through unchecked
    assert rn._check_tensors((("y", 1234, 10 ** 9),)) is None


def test_inputs_may_share_memory(rn):
    # scale and shift (read-only) may be the same buffer; an empty problem has
    # no extents at all
    st, err = nss(rn, B=0, shift=addr(7))
    assert st == 0, err
    st, err = fused(rn, B=0, shift=addr(7), gate=addr(7))
    assert st == 0, err


def fused_ex(rn, affine_dtype=0, y_dtype=0, y_scale=None, **kw):
    args = dict(y=addr(0), residual_out=addr(1), x=addr(2), residual=addr(3), gate=addr(4),
                weight=None, bias=None, scale=addr(7), shift=addr(8), B=1, L=16, D=5120,
                flags=rn.RN_GATE, gate_layout=(rn.RN_BCAST, 0), ss_layout=(rn.RN_BCAST, 0),
                eps=1e-6)
    args.update(kw)
    ext = rn.rn_ext(affine_dtype, y_dtype, y_scale)
    st = rn._lib.resnorm_fused_fwd_ex(args["y"], args["residual_out"], args["x"],
                                      args["residual"], args["gate"], args["weight"],
                                      args["bias"], args["scale"], args["shift"], args["B"],
                                      args["L"], args["D"], args["flags"],
                                      rn._layout(args["gate_layout"]),
                                      rn._layout(args["ss_layout"]), args["eps"],
                                      ctypes.byref(ext), None)
    return st, rn.last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(affine_dtype=2), 1, "affine_dtype"),
    (dict(affine_dtype=-1), 1, "affine_dtype"),
    (dict(y_dtype=3), 1, "y_dtype"),
    (dict(y_dtype=2), 1, "needs y_scale"),
    (dict(y_dtype=1, y_scale=addr(9)), 1, "y_scale given"),
    (dict(y_dtype=2, y_scale=addr(9) + 2), 1, "y_scale is not 4-byte aligned"),
    (dict(y_dtype=2, y_scale=addr(2)), 1, "y_scale overlaps x"),
    (dict(y_dtype=1, y=addr(2)), 1, "y overlaps x"),      # binary32 y cannot alias bf16 x
    (dict(y_dtype=1, y=addr(1) - 5120 * 2 * 16), 1, "overlaps"),  # 2x wider y runs into residual_out
])
def test_fused_ex_rejects(rn, kw, status, msg):
    st, err = fused_ex(rn, **kw)
    assert st == status, (st, err)
    assert msg in err, err


def test_ex_empty_problem_and_null_ext(rn):
    assert fused_ex(rn, B=0, y_dtype=2, y_scale=addr(9))[0] == 0
    assert fused_ex(rn, B=0, affine_dtype=1, flags=rn.RN_GATE | rn.RN_WEIGHT, weight=addr(5))[0] == 0
    st = rn._lib.norm_scale_shift_fwd_ex(addr(0), addr(2), None, None, addr(7), addr(8), 0, 4,
                                         64, 0, rn._layout((0, 0)), 1e-6, None, None)
    assert st == 0, rn.last_error()


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "resnorm.h"

int main(void) {
  rn_launch_info info;
  rn_layout bc = {RN_BCAST, 0}, fr = {RN_FRAME, 49};
  if (strstr(rn_version(), "gfx950") == NULL) return 1;
  if (rn_describe_launch(1, 176400, 5120, RN_GATE, 1, fr, fr, &info) != RN_OK) return 2;
  printf("%d %d %d %lld\n", info.waves_per_row, info.vec_per_lane, info.rows_per_block,
         (long long)info.grid_blocks);
  /* error paths fail on the host, before any device work */
  if (resnorm_fused_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 16, 5120,
                        RN_GATE, bc, bc, 1e-6f, NULL) != RN_EINVAL) return 3;
  printf("%s\n", rn_last_error());
  if (norm_scale_shift_fwd((void*)16, (const void*)4096, NULL, NULL, (const void*)8192,
                           (const void*)12288, 1, 16, 20000, 0, bc, 1e-6f, NULL) != RN_EUNSUPPORTED)
    return 4;
  rn_ext ext = {RN_DTYPE_BF16, RN_DTYPE_FP8_E4M3, NULL};
  if (norm_scale_shift_fwd_ex((void*)16, (const void*)(1 << 20), NULL, NULL, (const void*)(2 << 20),
                              (const void*)(3 << 20), 1, 16, 5120, 0, bc, 1e-6f, &ext, NULL)
      != RN_EINVAL) return 5;
  printf("%s\n", rn_last_error());
  return 0;
}
"""


def test_header_is_plain_c_and_links(rn, tmp_path):
    """A C11 program (gcc, -Wall -Wextra -Werror) includes the header, links
    the library and runs its host-only calls: version, the launch planner,
    and three argument errors that must be reported without any device work."""
    import subprocess
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    inc = os.path.join(ROOT, "include")
    libdir = os.path.dirname(rn.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", inc, str(src), "-o",
                    str(exe), "-L", libdir, "-lrnorm", "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    lines = out.stdout.splitlines()
    assert lines[0] == "1 10 4 44100"
    assert "NULL" in lines[1]
    assert "y_scale" in lines[2]


def test_last_error_is_per_thread(rn):
    """rn_last_error() is thread-local: threads that fail with different
    errors at the same time each read back their own message (ctypes releases
    the GIL around the calls, so the C calls do interleave)."""
    import threading
    cases = [(dict(D=12), "multiple of 8"), (dict(D=20000), "RN_D_MAX"), (dict(eps=-1.0), "eps"),
             (dict(flags=1 << 9), "unknown flag"), (dict(B=-1), "negative shape"),
             (dict(y=addr(0) + 4), "16-byte aligned")]
    errors = []
    start = threading.Barrier(len(cases))

    def worker(kw, want):
        start.wait()
        for _ in range(2000):
            st, msg = nss(rn, **kw)
            if st == 0 or want not in msg:
                errors.append((kw, st, msg))
                return

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_describe_launch_properties(rn):
    """Seeded random problems over the whole valid input space: every plan
    covers D, counts enough workgroups for every row, keeps workgroups within
    1024 threads, and gives several rows per wave only to the norm-only op
    with weight on problems of at least 12 Mi elements; invalid sizes are
    refused with an error, never planned."""
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(3000):
        fused = bool(rng.random() < 0.5)
        flags = int(rng.integers(0, 16))
        if not fused:
            flags &= ~rn.RN_GATE
        if flags & rn.RN_BIAS:
            flags |= rn.RN_WEIGHT
        B = int(rng.integers(0, 5))
        L = int(rng.choice([1, 3, 16, 600, 3600, 90000, 176400]))
        D = int(rng.integers(1, rn.RN_D_MAX // 8 + 1)) * 8
        lay = lambda: [(rn.RN_BCAST, 0), (rn.RN_ROW, 0), (rn.RN_FRAME, 1), (rn.RN_FRAME, 3)][int(rng.integers(0, 4))]  # noqa: E731
        gl, sl = lay(), lay()
        adt = rn.RN_DTYPE_F32 if rng.random() < 0.5 else rn.RN_DTYPE_BF16
        bad = [lay for lay in ((gl if fused and flags & rn.RN_GATE else None), sl)
               if lay is not None and lay[0] == rn.RN_FRAME and L % lay[1]]
        if bad:
            with pytest.raises(rn.RnError, match="L % frames == 0"):
                rn.describe_launch(B, L, D, flags, fused, gl, sl, affine_dtype=adt)
            continue
        i = rn.describe_launch(B, L, D, flags, fused, gl, sl, affine_dtype=adt)
        R = B * L
        assert 64 * i["waves_per_row"] * i["vec_per_lane"] * 8 >= D
        assert i["block_threads"] == 64 * i["waves_per_block"] <= 1024
        assert i["rows_per_block"] == i["rows_per_wave"] * i["waves_per_block"] // i["waves_per_row"]
        assert i["grid_blocks"] * i["rows_per_block"] >= R
        assert i["grid_blocks"] == -(-R // i["rows_per_block"])
        assert i["rows_per_wave"] in (1, 4)
        if i["rows_per_wave"] == 4:
            assert not fused and flags & rn.RN_WEIGHT and R * D >= 12 << 20
    for bad in ((1, 16, 7, 0), (1, 16, 0, 0), (1, 16, rn.RN_D_MAX + 8, 0), (-1, 16, 64, 0),
                (1, 16, 64, rn.RN_BIAS), (1, 16, 64, 1 << 7)):
        with pytest.raises(rn.RnError):
            rn.describe_launch(*bad, False)


def test_missing_library_fails_loudly(tmp_path):
    """Without the built HIP library the binding refuses to import (no CPU
    fallback exists): a copy of the package without librnorm.so raises
    ImportError naming the missing library and how to build it."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "rmsnorm_diffusion_transformers_amd", "__init__.py")
    pkg = tmp_path / "rmsnorm_diffusion_transformers_amd"
    pkg.mkdir()
    shutil.copy(src, pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import rmsnorm_diffusion_transformers_amd\n"
            "except ImportError as e:\n    print('IMPORTERROR', e)\n"
            "else:\n    print('IMPORTED')\n") % str(tmp_path)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert "IMPORTERROR" in out.stdout, out.stdout + out.stderr
    assert "librnorm.so is not built" in out.stdout and "build()" in out.stdout


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch must not map a second HIP or HSA
    runtime next to torch's own copies (two runtimes in one process can leave
    one of them without a device)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import rmsnorm_diffusion_transformers_amd\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l or 'libhsa-runtime64' in l})\n"
            "print('\\n'.join(libs))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    libs = out.stdout.split()
    assert len([l for l in libs if "libamdhip64" in l]) == 1, libs
    assert len([l for l in libs if "libhsa-runtime64" in l]) == 1, libs


def test_norm_only_two_rows_per_workgroup(rn):
    """Large norm-only problems without affine run the one-wave shapes of 8 or
    10 vectors per lane with 2 rows per workgroup; narrower rows, smaller
    problems, the fused op and the norm-only op with weight keep their
    shapes."""
    i = rn.describe_launch(1, 176400, 5120, 0, False)
    assert (i["waves_per_row"], i["vec_per_lane"], i["rows_per_block"], i["block_threads"]) == (1, 10, 2, 128)
    assert i["grid_blocks"] == 176400 // 2
    i = rn.describe_launch(1, 220500, 4096, 0, False)
    assert (i["waves_per_row"], i["vec_per_lane"], i["rows_per_block"]) == (1, 8, 2)
    for D in range(3592, 5121, 8):
        i = rn.describe_launch(1, -(-(12 << 20) // D), D, rn.RN_RMS, False)
        assert (i["waves_per_row"], i["rows_per_block"]) == (1, 2), D
    for D in (2048, 3072):
        i = rn.describe_launch(1, 903168000 // D, D, 0, False)
        assert (i["waves_per_row"], i["rows_per_block"]) == (1, 4), D
    # below 12 Mi elements, with weight, or fused: four rows per workgroup
    assert rn.describe_launch(1, 2000, 5120, 0, False)["rows_per_block"] == 4
    assert rn.describe_launch(1, 176400, 5120, rn.RN_GATE, True)["rows_per_block"] == 4
    assert rn.describe_launch(1, 176400, 5120, rn.RN_WEIGHT, False)["rows_per_wave"] == 4


def test_layout_structs_are_cached_only_for_plain_int_pairs(rn):
    """The binding reuses one rn_layout per (kind, frames) pair of plain ints
    (ctypes passes it by value); any other sequence is converted afresh."""
    import numpy as np
    a, b = rn._layout((rn.RN_FRAME, 49)), rn._layout((rn.RN_FRAME, 49))
    assert a is b and (a.kind, a.frames) == (rn.RN_FRAME, 49)
    c = rn._layout((np.int64(rn.RN_FRAME), 49))
    assert c is not a and (c.kind, c.frames) == (rn.RN_FRAME, 49)
    d = rn._layout([rn.RN_ROW, 0])
    assert (d.kind, d.frames) == (rn.RN_ROW, 0)
    assert rn._layout(a) is a


def test_stream_choice(rn, monkeypatch):
    """An explicit stream wins (a raw handle as is, a torch stream by its
    handle); without one the binding asks torch for the current stream of
    the operands' device (the current device when no tensor was given),
    through torch's raw-handle query or, where torch has none, a Stream
    object."""
    import types

    import torch
    assert rn._stream(1234) == 1234
    assert rn._stream(types.SimpleNamespace(cuda_stream=77)) == 77
    asked = []
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 3)
    monkeypatch.setattr(rn, "_RAW_STREAM", lambda dev: asked.append(("raw", dev)) or 1000 + dev)
    assert rn._stream(None, 1) == 1001 and rn._stream(None) == 1003
    monkeypatch.setattr(rn, "_RAW_STREAM", False)
    monkeypatch.setattr(torch.cuda, "current_stream",
                        lambda dev=None: asked.append(("obj", dev)) or types.SimpleNamespace(cuda_stream=5))
    assert rn._stream(None, 2) == 5
    assert asked == [("raw", 1), ("raw", 3), ("obj", 2)]
