"""Audit of the gfx950 assembly of the hot kernels (built here, on the CPU).

The pages audit the prior-art kernel's ISA for 128-bit-only global traffic,
no scratch, and the count of cross-lane steps (sglang PR #33144, "Speed Tests
and Profiling").  The same invariants for this library's kernels, from the
assembly hipcc writes for them:
  * every global access is a 128-bit buffer load/store (no global_/flat_ or
    narrower accesses; the FP8 output's 8-byte stores are the one exception,
    in the FP8 kernels only);
  * no scratch (private segment 0, no VGPR spills) and no LDS for one wave
    per row;
  * the wave reductions are DPP steps plus permlane16/permlane32 swaps: the
    mean and the variance on the common path, and on the paths for rows
    whose binary32 sums overflow, a NaN-propagating maximum and a rescaled
    sum each for the mean and for the variance;
  * the instruction counts per row match the design: 10 vectors per lane of
    each of x, residual, gate, and scale/shift (twice: the per-row and the
    shared-row paths), 20 stores, 80 bf16 packs;
  * the fused op with weight and one wave per row stages weight and bias in
    LDS with buffer loads that write LDS directly, reads them back with
    128-bit LDS reads, and keeps the headline kernel's register count.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rmsnorm_diffusion_transformers_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asm(tu, tmp_path):
    out = tmp_path / (tu + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", CSRC,
                    "--cuda-device-only", "-S", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-o", str(out), os.path.join(CSRC, tu)],
                   check=True, capture_output=True)
    return out.read_text()


def _kernel(asm, symbol):
    """(instructions, metadata) of one kernel: the code from its label to
    s_endpgm, and its kernel descriptor plus its entry in the code-object
    metadata."""
    m = re.search(r"^%s:[^\n]*\n(.*?)s_endpgm" % re.escape(symbol), asm, re.S | re.M)
    assert m, symbol
    body = m.group(1)
    desc = re.search(r"\.amdhsa_kernel %s\n(.*?)\.end_amdhsa_kernel" % re.escape(symbol), asm, re.S)
    entries = asm.split("amdhsa.kernels:")[1].split("\n  - ")
    entry = [e for e in entries if re.search(r"\.name:\s+%s\n" % re.escape(symbol), e)]
    return body, (desc.group(1) if desc else "") + "\n" + (entry[0] if entry else "")


def _count(body, mnemonic):
    return len(re.findall(r"^\s+%s\b" % re.escape(mnemonic), body, re.M))


def _meta_int(meta, key):
    m = re.search(r"\.%s:?\s+(\d+)" % key, meta)
    return int(m.group(1)) if m else None


@pytest.fixture(scope="module")
def fused_asm(tmp_path_factory):
    return _asm("rn_inst_fused_ln_gate_bf16.hip", tmp_path_factory.mktemp("asm"))


HEADLINE = "_ZN2rn10row_kernelINS_2OpILb0ELb1ELb1ELi0ELi0EEELi7EEEvNS_7RowArgsE"


def test_headline_kernel_memory_traffic_is_128bit(fused_asm):
    body, meta = _kernel(fused_asm, HEADLINE)
    assert not re.search(r"^\s+(global|flat|scratch)_", body, re.M)
    assert not re.search(r"^\s+buffer_(load|store)_(dword|dwordx2|dwordx3|short|byte|ubyte|ushort|sbyte|sshort)\b", body, re.M)
    # x, residual, gate 10 vectors each; scale/shift 20 on each of the
    # per-row and shared-row paths
    assert _count(body, "buffer_load_dwordx4") == 70
    assert _count(body, "buffer_store_dwordx4") == 20    # residual_out, y
    assert _count(body, "v_cvt_pk_bf16_f32") == 80


def test_headline_kernel_reductions_and_resources(fused_asm):
    body, meta = _kernel(fused_asm, HEADLINE)
    assert _count(body, "v_add_f32_dpp") == 16           # (2 common + 2 overflow) sums x 4 steps
    assert _count(body, "v_mov_b32_dpp") == 8            # 2 overflow-path maxima x 4 steps
    assert _count(body, "v_permlane16_swap_b32_e32") == 6
    assert _count(body, "v_permlane32_swap_b32_e32") == 6
    assert _count(body, "s_barrier") == 0                # one wave per row: no barrier
    assert not re.search(r"^\s+ds_", body, re.M)         # no LDS
    assert _meta_int(meta, "amdhsa_private_segment_fixed_size") == 0
    assert _meta_int(meta, "amdhsa_group_segment_fixed_size") == 0
    assert _meta_int(meta, "vgpr_spill_count") == 0
    assert _meta_int(meta, "sgpr_spill_count") == 0
    assert _meta_int(meta, "vgpr_count") <= 256          # two waves per SIMD
    assert _meta_int(meta, "amdhsa_float_denorm_mode_32") == 3   # fp32 denormals kept


def test_fp8_kernel_stores(tmp_path):
    asm = _asm("rn_inst_nss_ln_fp8.hip", tmp_path)
    sym = "_ZN2rn10row_kernelINS_2OpILb0ELb0ELb0ELi0ELi2EEELi7EEEvNS_7RowArgsE"
    body, meta = _kernel(asm, sym)
    assert _count(body, "buffer_store_dwordx2") == 10    # 8 FP8 bytes per lane per vector
    assert _count(body, "v_cvt_pk_fp8_f32") == 40
    assert _count(body, "v_mov_b32_dpp") == 12           # |t| maximum + 2 overflow-path maxima
    assert _count(body, "v_add_f32_dpp") == 16           # mean and variance, + their overflow paths
    assert _count(body, "v_permlane32_swap_b32_e32") == 7
    assert _count(body, "global_store_dword") == 1       # the per-row scale
    assert _meta_int(meta, "amdhsa_private_segment_fixed_size") == 0
    assert not re.search(r"^\s+(flat|scratch)_", body, re.M)


@pytest.mark.parametrize("aff,lds_loads,lds_reads,lds_bytes", [
    (4, 10, 40, 40960),    # binary32 weight + bias: 40 1-KB blocks over 4 waves
    (2, 5, 20, 20480),     # bf16 weight + bias
    (1, 3, 10, 10240),     # bf16 weight: 10 blocks, 3 rounds over 4 waves
])
def test_fused_affine_stages_weight_in_lds(fused_asm, aff, lds_loads, lds_reads, lds_bytes):
    sym = "_ZN2rn10row_kernelINS_2OpILb0ELb1ELb1ELi%dELi0EEELi7EEEvNS_7RowArgsE" % aff
    body, meta = _kernel(fused_asm, sym)
    fills = re.findall(r"^\s+buffer_load_dwordx4 .*\blds\b", body, re.M)
    assert len(fills) == lds_loads
    # the row's own loads are those of the headline kernel
    assert _count(body, "buffer_load_dwordx4") - len(fills) == 70
    assert _count(body, "ds_read_b128") == lds_reads
    assert not re.search(r"^\s+ds_(?!read_b128)", body, re.M)   # nothing else touches LDS
    assert _count(body, "s_barrier") == 1
    # The fills complete before the barrier: the last wait ahead of it allows
    # at most the 50 loads issued after the fills (gate, scale/shift, x,
    # residual; 10 vectors each) to be outstanding, and no fill follows it.
    lines = body.splitlines()
    bar = next(i for i, ln in enumerate(lines) if re.match(r"\s+s_barrier\b", ln))
    wait = next(i for i in range(bar - 1, -1, -1)
                if re.match(r"\s+s_waitcnt\b.*\bvmcnt\(", lines[i]))
    assert int(re.search(r"vmcnt\((\d+)\)", lines[wait]).group(1)) <= 50
    assert not any(re.search(r"buffer_load.*\blds\b", ln) for ln in lines[wait:bar])
    assert _count(body, "buffer_store_dwordx4") == 20
    assert _meta_int(meta, "amdhsa_group_segment_fixed_size") == lds_bytes
    assert _meta_int(meta, "amdhsa_private_segment_fixed_size") == 0
    assert _meta_int(meta, "vgpr_count") <= 256 and not _meta_int(meta, "agpr_count")


@pytest.fixture(scope="module")
def nss_asm(tmp_path_factory):
    return _asm("rn_inst_nss_ln_bf16.hip", tmp_path_factory.mktemp("asm_nss"))


@pytest.mark.parametrize("shape,w,vpt", [(31, 2, 5), (27, 1, 4)])
def test_multi_row_kernel_loads_shared_rows_once(nss_asm, shape, w, vpt):
    """The norm-only op with binary32 weight + bias on a multi-row shape (4
    consecutive rows per wave): the x loads and the stores of 4 rows, the
    weight, bias, scale and shift loads once (scale/shift on both cache-policy
    paths), 4 rows of bf16 packs; barriers only with several waves per row."""
    sym = "_ZN2rn10row_kernelINS_2OpILb0ELb0ELb0ELi4ELi0EEELi%dEEEvNS_7RowArgsE" % shape
    body, meta = _kernel(nss_asm, sym)
    k = 4
    assert _count(body, "buffer_load_dwordx4") == k * vpt + 2 * 2 * vpt + 2 * 2 * vpt
    assert _count(body, "buffer_store_dwordx4") == k * vpt
    assert _count(body, "v_cvt_pk_bf16_f32") == k * vpt * 4
    assert (_count(body, "s_barrier") > 0) == (w > 1)
    assert _meta_int(meta, "amdhsa_private_segment_fixed_size") == 0
    assert _meta_int(meta, "vgpr_count") <= 256 and not _meta_int(meta, "agpr_count")


@pytest.fixture(scope="module")
def nss_rms_asm(tmp_path_factory):
    return _asm("rn_inst_nss_rms_bf16.hip", tmp_path_factory.mktemp("asm_nss_rms"))


@pytest.mark.parametrize("shape,w,rpb,vpt", [(29, 2, 2, 3), (30, 2, 2, 4), (31, 2, 2, 5),
                                             (32, 4, 1, 3), (33, 4, 1, 4), (34, 4, 1, 5)])
@pytest.mark.parametrize("aff", [1, 4])
def test_multi_row_rms_partials_alternate_copies(nss_rms_asm, shape, w, rpb, vpt, aff):
    """RMSNorm has one barrier per row, so on the multi-row shapes with several
    waves per row consecutive rows must write their cross-wave partials to
    different LDS copies (a wave that moves on to the next row must not
    overwrite a partial a slower wave of the row has yet to read): the first
    LDS write of each of the 4 rows alternates between two offsets, and the
    workgroup's LDS holds two copies of the sum-of-squares and maximum
    partials."""
    sym = "_ZN2rn10row_kernelINS_2OpILb1ELb0ELb0ELi%dELi0EEELi%dEEEvNS_7RowArgsE" % (aff, shape)
    body, meta = _kernel(nss_rms_asm, sym)
    lines = body.splitlines()
    stores = [i for i, ln in enumerate(lines) if re.match(r"\s+buffer_store_dwordx4\b", ln)]
    assert len(stores) == 4 * vpt
    ends = [stores[vpt * k + vpt - 1] for k in range(4)]
    starts = [0] + [e + 1 for e in ends[:-1]]
    offs = []
    for a, b in zip(starts, ends):
        first = next(ln for ln in lines[a:b] if re.match(r"\s+ds_write_b32\b", ln))
        m = re.search(r"offset:(\d+)", first)
        offs.append(int(m.group(1)) if m else 0)
    assert all(offs[k] != offs[k + 1] for k in range(3)), offs
    assert offs[0] == offs[2] and offs[1] == offs[3], offs
    nred = w * rpb
    assert _meta_int(meta, "amdhsa_group_segment_fixed_size") == 2 * 2 * nred * 4


@pytest.mark.parametrize("shape,w,rpb,vpt", [(29, 2, 2, 3), (31, 2, 2, 5), (32, 4, 1, 3), (34, 4, 1, 5)])
@pytest.mark.parametrize("aff", [2, 4])
def test_multi_row_layernorm_partials_alternate_copies(nss_asm, shape, w, rpb, vpt, aff):
    """The LayerNorm multi-row kernels with several waves per row: the first
    LDS write of each of the 4 rows (its partial sum) alternates between two
    copies, and the workgroup holds two copies of each of the three partial
    arrays (sum, sum of squares, and the maximum of the overflow path)."""
    sym = "_ZN2rn10row_kernelINS_2OpILb0ELb0ELb0ELi%dELi0EEELi%dEEEvNS_7RowArgsE" % (aff, shape)
    body, meta = _kernel(nss_asm, sym)
    lines = body.splitlines()
    stores = [i for i, ln in enumerate(lines) if re.match(r"\s+buffer_store_dwordx4\b", ln)]
    assert len(stores) == 4 * vpt
    ends = [stores[vpt * k + vpt - 1] for k in range(4)]
    starts = [0] + [e + 1 for e in ends[:-1]]
    offs = []
    for a, b in zip(starts, ends):
        first = next(ln for ln in lines[a:b] if re.match(r"\s+ds_write_b32\b", ln))
        m = re.search(r"offset:(\d+)", first)
        offs.append(int(m.group(1)) if m else 0)
    assert all(offs[k] != offs[k + 1] for k in range(3)), offs
    assert offs[0] == offs[2] and offs[1] == offs[3], offs
    assert _meta_int(meta, "amdhsa_group_segment_fixed_size") == 2 * 3 * w * rpb * 4
