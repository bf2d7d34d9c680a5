"""Benchmark of the fused residual + gate + LayerNorm + scale/shift path on one MI355X.

Workload (one step = one launch of the fused op over the whole batch): WAN2.2
T2V-A14B at 720p / 193 frames -- 49 latent frames x 3600 tokens = sequence
176400, model width 5120, LayerNorm without affine, gated residual, with the
4D per-frame gate / scale / shift layout (B=1, F=49): the shape of sglang
PR #36349, "Microbenchmark", with synthetic N(0,1) activations.  Inputs are
resident in HBM before the timed region.

Metric: algorithmic HBM bytes (every operand read once + every output written
once) / time, in GB/s (1e9 B/s), against the 8 TB/s HBM3E peak.

Placement: by default the streamed tensors (x, residual and any per-row
operands; y and residual_out) live in one HBM arena at offsets chosen by
measurement (rmsnorm_diffusion_transformers_amd.hbm: inputs in one 32 GiB
granule, each output in its own granule of another class).  The rate with
torch's own back-to-back allocations on the fresh device is measured first
and reported beside it (placement.default_allocation); --placement default
times that layout throughout.

Beside the headline the line carries: companions (the norm-only op at the
same shape with broadcast scale/shift, and the other large workloads: fused
LayerNorm at L 90000 with 1 % of rows scaled by 50, fused RMSNorm + weight
with per-row scale/shift at L 90000, D 10240); variants of
the op at the same shape (broadcast modulation with and without binary32
weight+bias, FP8 and binary32 outputs, per-batch modulation); a DiT-forward
mix of the three calls WAN2.2 makes per forward (41 norm-only + 40 fused with
affine + 40 fused without, broadcast modulation, as in sglang PR #36349,
"Microbenchmark") against the pages' per-forward total; a plain-copy
reference; and the CPU oracle baseline.

Prints ONE JSON line.  Options: --gpus N (only 1: this path is measured on one
GPU), --steps K, --warmup W, --placement planned|default, --calibrate (time a
plain elementwise copy, used to scale rocprof byte counters), --no-cpu-baseline,
--no-extras, --no-companion, --workload NAME, --placement-map (the granule class
map of the headline kernel), --placement-thirds (its rate against the outputs'
place in one large allocation at 512 MiB steps), --placement-counters (three
placements, 40 warm + 40 measured launches each, for rocprofv3 counter runs),
--placement-widths (torch's allocations against a planned placement at row
widths 2048-10240); each of the placement modes prints one JSON line of its own.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "fused_ln_frame_b1_f49_l176400_d5120"
# Reported beside the headline: the norm-only op at the same shape, and the
# other large workloads (fused LayerNorm at L 90000 with 1 % of rows scaled
# by 50; fused RMSNorm + weight with per-row scale/shift at D 10240).
COMPANIONS = ["nss_ln_b1_l176400_d5120", "fused_ln_b1_l90000_d5120",
              "fused_rms_w_b1_l90000_d10240", "nss_ln_b1_l90000_d5120"]
KERNEL_SOURCES = ["rmsnorm_diffusion_transformers_amd/csrc/rn_row_kernel.hpp",
                  "rmsnorm_diffusion_transformers_amd/csrc/rn_args.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_digest() -> str:
    """Digest of the kernel sources' code: comments and blank lines are left
    out (the sources hold no string literal with a comment marker), so an
    edit to a comment keeps the counters taken on the same code valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprof counters, if they were taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [ln.split() for ln in f if ln.startswith("workload ")]
    except OSError:
        return None
    for toks in lines:
        rec = dict(zip(toks[0::2], toks[1::2]))
        if rec.get("workload") == workload and rec.get("kernel_digest") == kernel_digest():
            return int(rec["hbm_bytes_per_launch"])
    return None


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def upload(inp, dev):
    import numpy as np
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
            for k, v in inp.items()}


# Wall time the GPU is kept busy with the timed call itself before its warmup
# steps.  Measured on MI355X: after a second without kernels (input
# generation, host-to-device copies) the chip sits at idle clocks, and the
# first ~15-30 launches of these kernels run 3-5 % slower until its clocks
# and fabric have ramped (the fused headline's launches 1.256 -> 1.19 ms over
# the first 20 ms; the norm-only op's 0.648 -> 0.601 ms).  A fixed number of
# warmup launches covers that only for long runs; the settle phase covers it
# whatever the step counts, and it changes nothing in the timed region.
SETTLE_S = 0.1


_settle_count = [0]


def settle_launches():
    """Calls made by the last settle()."""
    return _settle_count[0]


def settle(fn, seconds=SETTLE_S):
    """Run fn() back to back, in batches that double up to 64 calls, until
    `seconds` of wall time have passed; returns the number of calls."""
    import torch
    n, batch, t0 = 0, 1, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        n += batch
        batch = min(2 * batch, 64)
        torch.cuda.synchronize()
    _settle_count[0] = n
    return n


def time_calls(fn, steps, warmup, settle_s=SETTLE_S):
    """Average ms per call of fn() over `steps` calls after a settle phase
    (settle()) and `warmup` calls, timed with events on the current stream
    (the stream the kernels run on)."""
    import torch
    stream = torch.cuda.current_stream()
    if settle_s > 0:
        settle(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - w0


def launch_stats(fn, steps):
    """Per-launch durations (ms) of `steps` calls, each between its own pair of
    events on the current stream: median, min, max.  Run after the timed
    region, so that the extra events do not perturb it."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": round(ts[len(ts) // 2], 5), "min": round(ts[0], 5), "max": round(ts[-1], 5),
            "n": len(ts)}


def streamed_keys(wl):
    """The inputs with one row per activation row (each read once per launch)."""
    keys = ["x"]
    if wl.op == "fused":
        keys.append("residual")
        if wl.gate_layout is not None and wl.gate_layout[0] == 1:
            keys.append("gate")
    if wl.ss_layout[0] == 1:
        keys += ["scale", "shift"]
    return keys


def host_bf16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def plan_workload(rn, wl, inp, arena, dev, extra_out=()):
    """Measured placement of the workload's streamed inputs and its outputs in
    the arena (rmsnorm_diffusion_transformers_amd.hbm.place_streams); the
    extra outputs, given as (shape, dtype), share y's granule."""
    import torch

    from rmsnorm_diffusion_transformers_amd import hbm
    keys = streamed_keys(wl)
    small = upload({k: v for k, v in inp.items() if k not in keys}, dev)
    shape = inp["x"].shape
    bf = torch.bfloat16
    y_spec = [(shape, bf), *extra_out] if extra_out else (shape, bf)
    outputs = [y_spec] + ([(shape, bf)] if wl.op == "fused" else [])
    stream = torch.cuda.current_stream()

    def make_launch(ins, outs):
        d = dict(small, **dict(zip(keys, ins)))
        y = outs[0][0] if extra_out else outs[0]
        ro = outs[1] if wl.op == "fused" else None
        return lambda: launch_workload(rn, wl, d, y, ro, stream)

    t0 = time.time()
    _, _, pl = hbm.place_streams(arena, [(inp[k].shape, bf) for k in keys], outputs, make_launch,
                                 stream=stream)
    info = pl.describe()
    info["search_s"] = round(time.time() - t0, 2)
    log("%s: placement inputs @ granule %d, outputs @ %s (%d candidates %.4f..%.4f ms, chosen %.4f ms, "
        "%.1f s)" % (wl.name, pl.read_granule, list(pl.write_granules), pl.candidates,
                     info["ms_first_pass_best"], info["ms_first_pass_worst"], pl.ms, info["search_s"]))
    return pl, info


def device_tensors(wl, inp, dev, arena=None, placement=None, extra_out=()):
    """(operands, y, residual_out, extra outputs) on the device: torch's own
    allocations, or views of the arena at the planned offsets with the inputs
    copied in.  extra_out lists (shape, dtype) of outputs placed after y."""
    import torch
    fused = wl.op == "fused"
    if placement is None:
        d = upload(inp, dev)
        y = torch.empty_like(d["x"])
        ro = torch.empty_like(d["x"]) if fused else None
        extra = [torch.empty(shape, dtype=dt, device=dev) for shape, dt in extra_out]
        return d, y, ro, extra
    keys = streamed_keys(wl)
    d = upload({k: v for k, v in inp.items() if k not in keys}, dev)
    for k, off in zip(keys, placement.read_offsets):
        t = arena.view(off, inp[k].shape, torch.bfloat16)
        t.copy_(host_bf16(inp[k]))
        d[k] = t
    w0 = placement.write_offsets[0]
    y_offs = w0 if isinstance(w0, list) else [w0]
    y = arena.view(y_offs[0], inp["x"].shape, torch.bfloat16)
    extra = [arena.view(o, shape, dt) for o, (shape, dt) in zip(y_offs[1:], extra_out)]
    ro = arena.view(placement.write_offsets[1], inp["x"].shape, torch.bfloat16) if fused else None
    torch.cuda.synchronize()
    return d, y, ro, extra


def make_inputs(wl):
    import synth
    t0 = time.time()
    inp = synth.make_inputs(wl, threads=threads())
    log("%s: inputs generated in %.1f s" % (wl.name, time.time() - t0))
    return inp


def time_workload(rn, wl, steps, warmup, dev, keep=False, stats=False, inp=None, arena=None,
                  placement=None, extra_out=()):
    import torch

    if inp is None:
        inp = make_inputs(wl)
    d, y, ro, extra = device_tensors(wl, inp, dev, arena, placement, extra_out)
    del inp
    stream = torch.cuda.current_stream()
    call = lambda: launch_workload(rn, wl, d, y, ro, stream)  # noqa: E731
    ms, wall = time_calls(call, steps, warmup)
    per_launch = launch_stats(call, steps) if stats else None
    if keep:
        return ms, wall, per_launch, (d, y, ro, extra)
    del d, y, ro, extra
    torch.cuda.empty_cache()
    return ms, wall, per_launch


def extras(rn, dev_tensors, steps, warmup, variants=True):
    """Variants of the op and the DiT-forward mix at the headline shape, on the
    headline's resident x / residual (B 1, L 176400, D 5120) and its outputs
    (y, residual_out, and the binary32 and FP8 y placed beside y; without
    `variants`, only the mix, and those two are not needed)."""
    import numpy as np
    import torch

    import synth
    d, y, ro, extra = dev_tensors
    y32, y8 = extra if variants else (None, None)
    x, res = d["x"], d["residual"]
    R, D = x.shape
    dev = x.device
    wl = synth.WORKLOADS[HEADLINE]
    bc = {k: synth.fill(wl.dists[t], 99, D).reshape(1, D) for k, t in
          (("gate", synth.GATE), ("scale", synth.SCALE), ("shift", synth.SHIFT))}
    bc = upload(bc, dev)
    rng = np.random.default_rng(99)
    w32 = torch.from_numpy((1.0 + 0.05 * rng.standard_normal(D)).astype(np.float32)).to(dev)
    b32 = torch.from_numpy((0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev)
    G, W, Bi = rn.RN_GATE, rn.RN_WEIGHT, rn.RN_BIAS
    F32, FP8 = rn.RN_DTYPE_F32, rn.RN_DTYPE_FP8_E4M3
    BC, FR = (rn.RN_BCAST, 0), (rn.RN_FRAME, 49)
    ys = torch.empty((R,), dtype=torch.float32, device=dev)

    def fused_bcast():
        rn.resnorm_fused_fwd(y, ro, x, res, bc["gate"], None, None, bc["scale"], bc["shift"],
                             1, R, D, G, BC, BC, 1e-6)

    def fused_affine():
        rn.resnorm_fused_fwd_ex(y, ro, x, res, bc["gate"], w32, b32, bc["scale"], bc["shift"],
                                1, R, D, G | W | Bi, BC, BC, 1e-6, F32)

    def nss_bcast():
        rn.norm_scale_shift_fwd(y, x, None, None, bc["scale"], bc["shift"], 1, R, D, 0, BC, 1e-6)

    w16, b16 = w32.to(torch.bfloat16), b32.to(torch.bfloat16)

    def nss_affine():
        rn.norm_scale_shift_fwd_ex(y, x, w32, b32, bc["scale"], bc["shift"], 1, R, D, W | Bi, BC,
                                   1e-6, F32)

    def nss_affine_bf16():
        rn.norm_scale_shift_fwd(y, x, w16, b16, bc["scale"], bc["shift"], 1, R, D, W | Bi, BC,
                                1e-6)

    def frame_fp8():
        rn.resnorm_fused_fwd_ex(y8, ro, x, res, d["gate"], None, None, d["scale"], d["shift"],
                                1, R, D, G, FR, FR, 1e-6, y_dtype=FP8, y_scale=ys)

    def frame_f32():
        rn.resnorm_fused_fwd_ex(y32, ro, x, res, d["gate"], None, None, d["scale"], d["shift"],
                                1, R, D, G, FR, FR, 1e-6, y_dtype=F32)

    pb = {k: v.expand(4, D).contiguous() for k, v in bc.items()}   # (4, D): per batch

    def per_batch():
        rn.resnorm_fused_fwd(y, ro, x, res, pb["gate"], None, None, pb["scale"], pb["shift"],
                             4, R // 4, D, G, (rn.RN_FRAME, 1), (rn.RN_FRAME, 1), 1e-6)

    act = R * D * 2
    row = D * 2
    cases = [
        ("fused_ln_bcast", "fused LN, gate/scale/shift (1,C)", fused_bcast, 4 * act + 3 * row),
        ("fused_ln_bcast_affine_fp32", "fused LN + fp32 weight/bias, (1,C) modulation",
         fused_affine, 4 * act + 3 * row + 2 * 4 * D),
        ("fused_ln_frame_fp8_out", "headline op, FP8 E4M3 y + per-row scale", frame_fp8,
         3 * act + R * D + 4 * R + 3 * 49 * row),
        ("fused_ln_frame_fp32_out", "headline op, binary32 y", frame_f32,
         3 * act + 2 * act + 3 * 49 * row),
        ("fused_ln_per_batch_b4", "fused LN, B 4 x L 44100, (B,1,C) modulation", per_batch,
         4 * act + 3 * 4 * row),
        ("nss_ln_bcast_affine_fp32", "norm-only LN + fp32 weight/bias, (1,C) modulation",
         nss_affine, 2 * act + 2 * row + 2 * 4 * D),
        ("nss_ln_bcast_affine_bf16", "norm-only LN + bf16 weight/bias, (1,C) modulation",
         nss_affine_bf16, 2 * act + 4 * row),
    ]
    out = []
    launches = 0   # row-kernel launches made here
    for name, what, fn, nbytes in (cases if variants else []):
        ms, _ = time_calls(fn, steps, warmup)
        launches += settle_launches() + steps + warmup
        gbs = nbytes / (ms * 1e-3) / 1e9
        log("%s: %.4f ms/launch, %.1f GB/s" % (name, ms, gbs))
        out.append({"variant": name, "what": what, "ms_per_launch": round(ms, 5),
                    "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})

    # DiT forward: per block norm1 (norm-only), self-attention norm (fused,
    # affine), cross-attention norm (fused, no affine); norm_out at the end.
    def forward():
        for _ in range(40):
            nss_bcast()
            fused_affine()
            fused_bcast()
        nss_bcast()

    # right after the variants, warm; on its own, after a settle phase
    fwd_ms, _ = time_calls(forward, 3, 1, settle_s=0 if variants else SETTLE_S)
    launches += 121 * ((0 if variants else settle_launches()) + 1 + 3)
    log("DiT forward mix: %.2f ms per forward (121 calls)" % fwd_ms)
    mix = {"ms_per_forward": round(fwd_ms, 3),
           "calls": {"norm_scale_shift (no affine)": 41, "fused, fp32 affine": 40,
                     "fused, no affine": 40},
           "shape": "B 1, L 176400, D 5120, broadcast (1,C) gate/scale/shift, LayerNorm",
           "pages_prior_art_ms_per_forward_context": [171.6, 174.8],
           "row_kernel_launches": launches}
    del ys, bc, pb, w32, b32, w16, b16
    return out, mix


def flags_of(rn, wl):
    f = (rn.RN_RMS if wl.is_rms else 0) | (rn.RN_WEIGHT if wl.has_weight else 0) | \
        (rn.RN_BIAS if wl.has_bias else 0)
    if wl.op == "fused" and wl.gate_layout is not None:
        f |= rn.RN_GATE
    return f


def prepare_workload(rn, wl, d, y, ro, stream):
    """launch_workload's call, checked once (rn.prepare)."""
    flags = flags_of(rn, wl)
    if wl.op == "fused":
        return rn.prepare(rn.resnorm_fused_fwd, y, ro, d["x"], d["residual"], d.get("gate"),
                          d.get("weight"), d.get("bias"), d["scale"], d["shift"], wl.B, wl.L,
                          wl.D, flags, wl.gate_layout or (0, 0), wl.ss_layout, wl.eps, stream)
    return rn.prepare(rn.norm_scale_shift_fwd, y, d["x"], d.get("weight"), d.get("bias"),
                      d["scale"], d["shift"], wl.B, wl.L, wl.D, flags, wl.ss_layout, wl.eps,
                      stream)


def launch_workload(rn, wl, d, y, ro, stream):
    """One pass of the workload through the C entry points."""
    flags = flags_of(rn, wl)
    if wl.op == "fused":
        rn.resnorm_fused_fwd(y, ro, d["x"], d["residual"], d.get("gate"), d.get("weight"),
                             d.get("bias"), d["scale"], d["shift"], wl.B, wl.L, wl.D, flags,
                             wl.gate_layout or (0, 0), wl.ss_layout, wl.eps, stream)
    else:
        rn.norm_scale_shift_fwd(y, d["x"], d.get("weight"), d.get("bias"), d["scale"],
                                d["shift"], wl.B, wl.L, wl.D, flags, wl.ss_layout, wl.eps, stream)


REF_LIB = os.path.join(ROOT, "rmsnorm_diffusion_transformers_amd", "libtrafficref.so")
# workloads with a traffic reference (libtrafficref.so: the kernel's memory
# traffic at D 5120 without its arithmetic)
REF_WORKLOADS = (HEADLINE, "nss_ln_b1_l176400_d5120")
_ref_lib = []


def _traffic_ref_lib():
    import ctypes
    if not _ref_lib:
        if not os.path.exists(REF_LIB):
            raise RuntimeError("libtrafficref.so is not built (expected at %s); build it with "
                               "__graft_entry__.build()" % REF_LIB)
        lib = ctypes.CDLL(REF_LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.rn_traffic_ref.argtypes = [P] * 7 + [I64] * 4 + [P]
        lib.rn_traffic_ref.restype = ctypes.c_int
        lib.rn_traffic_ref_nss.argtypes = [P] * 4 + [I64] * 3 + [P]
        lib.rn_traffic_ref_nss.restype = ctypes.c_int
        _ref_lib.append(lib)
    return _ref_lib[0]


def traffic_reference_call(wl, d, y, ro, stream):
    """A launcher of the measurement reference on the workload's own tensors:
    for the fused op with per-frame gate/scale/shift, rn_traffic_ref; for the
    norm-only op with broadcast scale/shift, rn_traffic_ref_nss (D 5120)."""
    lib = _traffic_ref_lib()
    n = wl.B * wl.L * wl.D
    if wl.op == "fused":
        frames = wl.gate_layout[1]
        assert wl.gate_layout == wl.ss_layout == (2, frames) and not wl.has_weight
        m = wl.B * frames * wl.D
        ops = ((y, n), (ro, n), (d["x"], n), (d["residual"], n), (d["gate"], m), (d["scale"], m),
               (d["shift"], m))
        fn = lib.rn_traffic_ref
        tail = (wl.B, wl.L, wl.D, frames, stream.cuda_stream)
    else:
        assert wl.ss_layout == (0, 0) and not wl.has_weight
        ops = ((y, n), (d["x"], n), (d["scale"], wl.D), (d["shift"], wl.D))
        fn = lib.rn_traffic_ref_nss
        tail = (wl.B, wl.L, wl.D, stream.cuda_stream)
    for t, need in ops:
        assert t.is_cuda and t.is_contiguous() and t.element_size() == 2 and t.numel() >= need
    args = tuple(t.data_ptr() for t, _ in ops) + tail

    def call():
        st = fn(*args)
        if st != 0:
            raise RuntimeError("%s returned %d" % (fn.__name__, st))
    return call


def traffic_reference_entry(wl, ref, ref_torch, gbs, torch_alloc, placement_kind):
    """The bench line's record of a traffic reference: its rate on the
    workload's placement and on torch's allocations, and the kernel's rate
    over it on each."""
    if wl.op == "fused":
        what = ("rn_traffic_ref (libtrafficref.so): residual_out = x ^ residual, y = residual_out ^ "
                "gate ^ scale ^ shift, the fused kernel's loads and stores")
    else:
        what = ("rn_traffic_ref_nss (libtrafficref.so): y = x ^ scale ^ shift, the norm-only "
                "kernel's loads, stores and occupancy")
    tr = {"kernel": what, "bytes_per_launch": wl.algorithmic_bytes(), "placement": placement_kind,
          **(ref or {}), "torch_allocation": ref_torch}
    if ref:
        tr["kernel_over_reference"] = round(gbs / ref["GB/s"], 4)
    if ref_torch and torch_alloc:
        tr["kernel_over_reference_torch_allocation"] = round(torch_alloc["GB/s"] / ref_torch["GB/s"], 4)
    return tr


def traffic_reference_rate(wl, d, y, ro, steps, warmup):
    """The reference timed like the workload (settle, warmup, steps) on the
    same tensors: {ms_per_launch, GB/s, frac} over the workload's algorithmic
    bytes (the reference moves the same bytes)."""
    import torch
    ms, _ = time_calls(traffic_reference_call(wl, d, y, ro, torch.cuda.current_stream()), steps,
                       warmup)
    g = wl.algorithmic_bytes() / (ms * 1e-3) / 1e9
    return {"ms_per_launch": round(ms, 5), "GB/s": round(g, 1), "frac": round(g / HBM_PEAK_GBS, 4)}


SMALL = ("fused_ln_b1_l16_d5120", "fused_ln_b2_l16_d5120", "nss_ln_b1_l16_d5120",
         "nss_ln_b2_l16_d5120", "fused_rms_w_b2_l16_d10240")


def small_batch_latency(rn, dev, names=SMALL):
    """The L = 16 workloads (the pages' speed matrix at B 1 and 2, D 5120, and
    the RMS case at D 10240) are launch- and latency-bound (their bytes fit
    in cache): per-call time of back-to-back launches on the stream through
    the checked binding and through a prepared call (rn.prepare: the checks
    done once), and with 100 launches captured in one HIP graph and replayed
    (wall time / 100)."""
    import torch

    import synth
    out = []
    for name in names:
        wl = synth.WORKLOADS[name]
        d = upload(synth.make_inputs(wl, threads=1), dev)
        y = torch.empty_like(d["x"])
        ro = torch.empty_like(d["x"]) if wl.op == "fused" else None
        stream = torch.cuda.current_stream()
        eager_ms, _ = time_calls(lambda: launch_workload(rn, wl, d, y, ro, stream), 200, 20)
        prepared = prepare_workload(rn, wl, d, y, ro, stream)
        prep_ms, _ = time_calls(prepared, 200, 20)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            launch_workload(rn, wl, d, y, ro, torch.cuda.current_stream())
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(100):
                launch_workload(rn, wl, d, y, ro, torch.cuda.current_stream())
        graph_ms, _ = time_calls(g.replay, 20, 3)
        out.append({"workload": name, "us_per_call_stream": round(eager_ms * 1e3, 2),
                    "us_per_call_prepared": round(prep_ms * 1e3, 2),
                    "us_per_call_graph": round(graph_ms * 1e3 / 100, 2),
                    "algorithmic_bytes": wl.algorithmic_bytes()})
        log("%s: %.2f us/call on the stream (%.2f prepared), %.2f us/call in a graph" % (
            name, eager_ms * 1e3, prep_ms * 1e3, graph_ms * 1e3 / 100))
        del g, d, y, ro
    # the floor: a one-element torch.neg, 100 launches captured and replayed the same way
    a = torch.zeros(1, device=dev)
    b = torch.empty_like(a)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.neg(a, out=b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(100):
            torch.neg(a, out=b)
    floor_ms, _ = time_calls(g.replay, 20, 3)
    out.append({"workload": "launch floor: one-element torch.neg", "us_per_call_graph": round(floor_ms * 1e3 / 100, 2)})
    log("launch floor (one-element torch.neg in a graph): %.2f us/call" % (floor_ms * 1e3 / 100))
    del g, a, b
    return out


def copy_reference(steps, warmup, dev):
    """A plain elementwise copy (torch.neg on bf16: reads N bytes, writes N
    bytes) on a tensor of the headline's activation size: the rocprof counter
    calibration kernel, and a practical read+write bandwidth reference on the
    same GPU in the same run."""
    import torch
    n = 176400 * 5120
    x = torch.randn(n, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    for _ in range(warmup):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        torch.neg(x, out=y)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    del x, y
    torch.cuda.empty_cache()
    return {"kernel": "torch.neg bf16 (1 read + 1 write stream)", "bytes_per_launch": 4 * n,
            "ms_per_launch": round(ms, 5), "GB/s": round(4 * n / ms / 1e6, 1),
            "frac": round(4 * n / ms / 1e6 / HBM_PEAK_GBS, 4)}


def placement_map(rn, dev, granules=7):
    """Rate of the headline kernel for every assignment of x, residual, y and
    residual_out to distinct granules of an HBM arena (the first `granules`
    of it), a fixed reference placement timed every 40 assignments for drift;
    then the granule classes inferred from which output pairs are slow, and
    the rates grouped by class pattern.  Prints one JSON line."""
    import itertools
    import statistics

    import torch

    import synth
    from rmsnorm_diffusion_transformers_amd import hbm
    wl = synth.WORKLOADS[HEADLINE]
    R, D = wl.R, wl.D
    inp = make_inputs(wl)
    arena = hbm.HbmArena(dev)
    n = min(granules, arena.granules)
    nb = R * D * 2
    slot = lambda g: arena.view(g * hbm.GRANULE + hbm.SLOT_START, (R, D), torch.bfloat16)  # noqa: E731
    views = [slot(g) for g in range(n)]
    small = upload({k: inp[k] for k in ("gate", "scale", "shift")}, dev)
    for v in views:
        v.copy_(host_bf16(inp["x"]))
    stream = torch.cuda.current_stream()

    def rate(x, r, y, o, steps=16):
        call = lambda: launch_workload(rn, wl, dict(small, x=x, residual=r), y, o, stream)  # noqa: E731
        ms, _ = time_calls(call, steps, 3, settle_s=0)   # back to back with the other trials
        return wl.algorithmic_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS

    ref_place = (0, 0, 1, 2)
    ref_views = (views[0], arena.view(hbm.SLOT_START + hbm.round_up(nb), (R, D), torch.bfloat16),
                 views[1], views[2])
    ref_views[1].copy_(host_bf16(inp["residual"]))
    rows, refs = [], []
    t0 = time.time()
    for k, (gx, gr, gy, go) in enumerate(itertools.permutations(range(n), 4)):
        if k % 40 == 0:
            refs.append(rate(*ref_views))
        rows.append(((gx, gr, gy, go), rate(views[gx], views[gr], views[gy], views[go])))
    log("placement map: %d assignments in %.0f s" % (len(rows), time.time() - t0))
    # output pairs: mean rate over assignments with {y, o} = {i, j}
    pair = {}
    for (gx, gr, gy, go), f in rows:
        pair.setdefault(tuple(sorted((gy, go))), []).append(f)
    pair = {k: statistics.mean(v) for k, v in pair.items()}
    lo, hi = min(pair.values()), max(pair.values())
    cut = (lo + hi) / 2
    cls = list(range(n))

    def find(a):
        while cls[a] != a:
            a = cls[a]
        return a
    for (i, j), f in pair.items():
        if f < cut:
            cls[find(i)] = find(j)
    labels = {}
    names = [labels.setdefault(find(g), "ABCDEFGH"[len(labels)]) for g in range(n)]
    groups = {}
    for (gx, gr, gy, go), f in rows:
        groups.setdefault("".join(names[g] for g in (gx, gr, gy, go)), []).append(f)
    patterns = sorted(((statistics.mean(v), k, len(v), min(v), max(v)) for k, v in groups.items()),
                      reverse=True)
    rows.sort(key=lambda t: t[1])
    out = {"workload": wl.name, "granule_gib": hbm.GRANULE >> 30, "granules": n,
           "assignments": len(rows), "reference_frac": [round(min(refs), 4), round(max(refs), 4)],
           "output_pair_cut": round(cut, 4), "granule_class": names,
           "patterns_x_r_y_o": [{"pattern": k, "n": c, "mean": round(m, 4), "min": round(a, 4),
                                 "max": round(b, 4)} for m, k, c, a, b in patterns],
           "slowest": [[list(p), round(f, 4)] for p, f in rows[:5]],
           "fastest": [[list(p), round(f, 4)] for p, f in rows[-5:]]}
    arena.release()
    print(json.dumps(out), flush=True)


def _headline_on(rn, dev):
    """(inputs, small device operands, launch factory) of the headline workload:
    the factory takes (x, residual, y, residual_out) views."""
    import torch

    import synth
    wl = synth.WORKLOADS[HEADLINE]
    inp = make_inputs(wl)
    small = upload({k: inp[k] for k in ("gate", "scale", "shift")}, dev)
    stream = torch.cuda.current_stream()

    def make(x, r, y, o):
        return lambda: launch_workload(rn, wl, dict(small, x=x, residual=r), y, o, stream)
    return wl, inp, make


def placement_thirds(rn, dev, step_gib=0.5):
    """The headline kernel's rate against where its outputs sit in one large
    allocation: x and residual at its start; an adjacent output pair
    (residual_out at P, y at P + 2 GiB) swept over the allocation; then y
    swept over it with residual_out fixed at 40 GiB and at 100.5 GiB.  Steps
    of `step_gib`; 10 launches after 2 for each point.  Prints one JSON line."""
    import torch

    from rmsnorm_diffusion_transformers_amd import hbm
    GiB = 1 << 30
    wl, inp, make = _headline_on(rn, dev)
    R, D = wl.R, wl.D

    def frac(call):
        ms, _ = time_calls(call, 10, 2, settle_s=0)
        return round(wl.algorithmic_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    arena = hbm.HbmArena(dev)
    N = arena.nbytes
    view = lambda off: arena.view(int(off), (R, D), torch.bfloat16)  # noqa: E731
    x, r = view(0), view(2 * GiB)
    x.copy_(host_bf16(inp["x"]))
    r.copy_(host_bf16(inp["residual"]))
    del inp
    settle(make(x, r, view(4 * GiB), view(6 * GiB)), 0.2)
    step = int(step_gib * GiB)
    out = {"workload": wl.name, "allocation_gib": N / GiB, "step_gib": step_gib,
           "device_memory_gib": round(torch.cuda.get_device_properties(dev).total_memory / GiB, 3)}
    adj, P = [], 4 * GiB
    while P + 4 * GiB <= N:
        adj.append([P / GiB, frac(make(x, r, view(P + 2 * GiB), view(P)))])
        P += step
    out["adjacent_pair"] = adj
    for anchor in (40 * GiB, 100 * GiB + GiB // 2):
        if anchor + 2 * GiB > N:
            continue
        sw, P = [], 4 * GiB
        while P + 2 * GiB <= N:
            if abs(P - anchor) >= 2 * GiB:
                sw.append([P / GiB, frac(make(x, r, view(P), view(anchor)))])
            P += step
        out["y_sweep_residual_out_at_%g" % (anchor / GiB)] = sw
    log("placement thirds: %d + sweep points" % len(adj))
    del x, r
    arena.release()
    print(json.dumps(out), flush=True)


def placement_counters(rn, dev, n=40):
    """The headline kernel on three placements, 2n launches each, in this
    order: torch's back-to-back allocations; one large allocation with both
    outputs in its first third (residual_out at 40 GiB, y at 60 GiB); the
    same with the outputs in two thirds (y at 150 GiB).  Each placement's
    first n launches bring the GPU out of its idle clocks and its last n are
    the measured ones, so a counter trace of this command splits by
    row-kernel dispatch index (measured: n..2n-1, 3n..4n-1, 5n..6n-1).
    Without a profiler the printed line gives each placement's rate from its
    measured launches."""
    import torch

    from rmsnorm_diffusion_transformers_amd import hbm
    GiB = 1 << 30
    wl, inp, make = _headline_on(rn, dev)
    R, D = wl.R, wl.D
    res = {}

    def run(name, call):
        # n launches to bring the GPU out of its idle clocks, then n timed
        # (a fixed count, so a counter trace splits by dispatch index)
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(n):
            call()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / n
        res[name] = round(wl.algorithmic_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        log("placement counters: %s %.4f ms" % (name, ms))

    x, r = upload({"x": inp["x"]}, dev)["x"], upload({"r": inp["residual"]}, dev)["r"]
    y, o = torch.empty_like(x), torch.empty_like(x)
    run("torch_allocations", make(x, r, y, o))
    del x, r, y, o
    torch.cuda.empty_cache()
    arena = hbm.HbmArena(dev)
    view = lambda off: arena.view(int(off), (R, D), torch.bfloat16)  # noqa: E731
    x, r = view(0), view(2 * GiB)
    x.copy_(host_bf16(inp["x"]))
    r.copy_(host_bf16(inp["residual"]))
    run("outputs_in_one_third", make(x, r, view(60 * GiB), view(40 * GiB)))
    run("outputs_in_two_thirds", make(x, r, view(150 * GiB), view(40 * GiB)))
    del x, r
    arena.release()
    print(json.dumps({"workload": wl.name, "launches_each": n, "frac": res}), flush=True)


def placement_arena_sizes(rn, dev, sizes=(3, 4, 5, 6, None), rounds=2):
    """The headline's planned rate against the arena's size: for each number
    of 32 GiB granules (None: all free HBM but 24 GiB), `rounds` fresh
    arenas, each planned (rmsnorm_diffusion_transformers_amd.hbm) and timed
    at its placement (40 launches after 10).  Prints one JSON line."""
    import torch

    import synth
    from rmsnorm_diffusion_transformers_amd import hbm
    wl = synth.WORKLOADS[HEADLINE]
    inp = make_inputs(wl)
    nb = wl.algorithmic_bytes()
    ms, _, _ = time_workload(rn, wl, 40, 10, dev, inp=inp)
    out = {"workload": wl.name, "torch_allocation_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "arenas": []}
    for rnd in range(rounds):
        for g in sizes:
            arena = hbm.HbmArena(dev, granules=g)
            pl, info = plan_workload(rn, wl, inp, arena, dev)
            ms, _, _ = time_workload(rn, wl, 40, 10, dev, inp=inp, arena=arena, placement=pl)
            out["arenas"].append({"round": rnd, "granules": arena.granules, "gib": arena.nbytes >> 30,
                                  "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "candidates": pl.candidates, "read_granule": pl.read_granule,
                                  "write_granules": list(pl.write_granules),
                                  "ms_first_pass_best": info["ms_first_pass_best"],
                                  "ms_first_pass_worst": info["ms_first_pass_worst"]})
            log("arena of %d granules: %.4f" % (arena.granules, out["arenas"][-1]["frac"]))
            arena.release()
            del arena
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def placement_widths(rn, dev, widths=(2048, 3072, 4096, 5120, 6144, 8192, 10240)):
    """Fused LayerNorm (broadcast gate/scale/shift) and the norm-only op at
    several row widths, 176400 x 5120 elements each: torch's own allocations
    first, then one planned placement per problem (hbm.place_streams).  Prints
    one JSON line."""
    import numpy as np
    import torch

    from rmsnorm_diffusion_transformers_amd import hbm
    total = 176400 * 5120
    stream = torch.cuda.current_stream()
    bf = torch.bfloat16
    rng = np.random.default_rng(5)

    def mods(D):
        g = torch.from_numpy(rng.uniform(0, 1, (1, D)).astype(np.float32)).to(dev).to(bf)
        sc = torch.from_numpy((0.1 * rng.standard_normal((1, D))).astype(np.float32)).to(dev).to(bf)
        sh = torch.from_numpy((0.1 * rng.standard_normal((1, D))).astype(np.float32)).to(dev).to(bf)
        return g, sc, sh

    def fused(L, D, g, sc, sh):
        return lambda x, r, y, o: (lambda: rn.resnorm_fused_fwd(
            y, o, x, r, g, None, None, sc, sh, 1, L, D, rn.RN_GATE, (0, 0), (0, 0), 1e-6, stream))

    def nss(L, D, sc, sh):
        return lambda x, y: (lambda: rn.norm_scale_shift_fwd(
            y, x, None, None, sc, sh, 1, L, D, 0, (0, 0), 1e-6, stream))

    def frac(nbytes, call):
        ms, _ = time_calls(call, 40, 8, settle_s=0.05)
        return round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    rows = {}
    for D in widths:
        L = total // D
        g, sc, sh = mods(D)
        x = torch.randn(L, D, device=dev).to(bf)
        r = torch.randn(L, D, device=dev).to(bf)
        y, o = torch.empty_like(x), torch.empty_like(x)
        fi = rn.describe_launch(1, L, D, rn.RN_GATE, True)
        ni = rn.describe_launch(1, L, D, 0, False)
        rows[D] = {"rows": L, "fused_shape": [fi["waves_per_row"], fi["vec_per_lane"], fi["rows_per_block"]],
                   "nss_shape": [ni["waves_per_row"], ni["vec_per_lane"], ni["rows_per_block"]],
                   "fused_torch": frac(4 * L * D * 2, fused(L, D, g, sc, sh)(x, r, y, o)),
                   "nss_torch": frac(2 * L * D * 2, nss(L, D, sc, sh)(x, y))}
        del x, r, y, o
        torch.cuda.empty_cache()
    arena = hbm.HbmArena(dev)
    for D in widths:
        L = total // D
        g, sc, sh = mods(D)
        act = ((L, D), bf)
        mk = fused(L, D, g, sc, sh)
        (x, r), (y, o), _ = hbm.place_streams(arena, [act, act], [act, act],
                                              lambda i, w: mk(i[0], i[1], w[0], w[1]), stream=stream)
        x.normal_()
        r.normal_()
        rows[D]["fused_planned"] = frac(4 * L * D * 2, mk(x, r, y, o))
        mkn = nss(L, D, sc, sh)
        (xn,), (yn,), _ = hbm.place_streams(arena, [act], [act], lambda i, w: mkn(i[0], w[0]), stream=stream)
        xn.normal_()
        rows[D]["nss_planned"] = frac(2 * L * D * 2, mkn(xn, yn))
        log("D %d: %s" % (D, rows[D]))
    arena.release()
    print(json.dumps({"elements": total, "widths": rows}), flush=True)


def calibrate(steps, warmup, dev):
    print(json.dumps(copy_reference(steps, warmup, dev)), flush=True)


def cpu_baseline(wl):
    """The oracle (as it is) on this host's cores: every row of the workload on
    all threads (up to 16), and the first 16384 rows on one thread.  Input
    generation is not timed.  Returns the record for the JSON line."""
    import oracle
    n = threads()
    rows = wl.R
    t0 = time.time()
    inp = _first_rows(wl, rows, n)
    log("cpu baseline: inputs for %d rows in %.1f s" % (rows, time.time() - t0))
    o = oracle.Oracle()
    per_row = wl.algorithmic_bytes() / wl.R
    t0 = time.perf_counter()
    o.run_workload(wl, inp, row0=0, nrows=rows, threads=n)
    dt = time.perf_counter() - t0
    log("cpu baseline: %d rows on %d threads in %.2f s" % (rows, n, dt))
    rows1 = min(16384, wl.R)
    t1 = time.perf_counter()
    o.run_workload(wl, inp, row0=0, nrows=rows1, threads=1)
    dt1 = time.perf_counter() - t1
    log("cpu baseline: %d rows on 1 thread in %.2f s" % (rows1, dt1))
    return {"value": round(rows * per_row / dt / 1e9, 3), "unit": "GB/s", "cores": n,
            "kind": "oracle", "rows_per_s": round(rows / dt, 1),
            "sample": "all %d rows of %s (every operand), oracle threads=%d, %.2f s wall; "
                      "input generation not timed" % (rows, wl.name, n, dt),
            "single_thread": {"value": round(rows1 * per_row / dt1 / 1e9, 3), "unit": "GB/s",
                              "rows_per_s": round(rows1 / dt1, 1),
                              "sample": "first %d rows, 1 thread, %.2f s wall" % (rows1, dt1)}}


def _first_rows(wl, rows, n):
    """Inputs of the first `rows` activation rows (modulation tensors whole)."""
    import synth
    d = wl.dists
    out = {"x": synth.fill(d[synth.X], wl.wid, rows * wl.D, row_len=wl.D, stress=wl.stress,
                           threads=n).reshape(rows, wl.D)}
    if wl.op == "fused":
        out["residual"] = synth.fill(d[synth.RES], wl.wid, rows * wl.D, row_len=wl.D,
                                     stress=wl.stress, threads=n).reshape(rows, wl.D)
        if wl.gate_layout is not None:
            g = wl.mod_rows(wl.gate_layout)
            out["gate"] = synth.fill(d[synth.GATE], wl.wid, g * wl.D, threads=n).reshape(g, wl.D)
    m = wl.mod_rows(wl.ss_layout)
    out["scale"] = synth.fill(d[synth.SCALE], wl.wid, m * wl.D, threads=n).reshape(m, wl.D)
    out["shift"] = synth.fill(d[synth.SHIFT], wl.wid, m * wl.D, threads=n).reshape(m, wl.D)
    if wl.has_weight:
        out["weight"] = synth.fill(d[synth.WEIGHT], wl.wid, wl.D, threads=n)
    if wl.has_bias:
        out["bias"] = synth.fill(d[synth.BIAS], wl.wid, wl.D, threads=n)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--placement", choices=("planned", "default"), default="planned",
                    help="planned: streamed tensors in an HBM arena at measured offsets; "
                         "default: torch's own allocations")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--placement-map", action="store_true",
                    help="time the headline kernel on every assignment of its four streamed "
                         "tensors to distinct HBM granules and print the class map")
    ap.add_argument("--placement-thirds", action="store_true",
                    help="the headline kernel's rate against where its outputs sit in one large "
                         "allocation, at 512 MiB steps")
    ap.add_argument("--placement-counters", action="store_true",
                    help="the headline kernel on three placements, 40 warm + 40 measured "
                         "launches each, for rocprofv3 counter runs")
    ap.add_argument("--small-batch", action="store_true",
                    help="only the L = 16 latency measurements (small_batch_latency), one JSON line")
    ap.add_argument("--placement-arena-sizes", action="store_true",
                    help="the headline's planned rate against the HBM arena's size")
    ap.add_argument("--placement-widths", action="store_true",
                    help="torch's allocations against a planned placement for the fused and "
                         "norm-only ops at several row widths")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-companion", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the traffic reference (the fused op's memory traffic without its "
                         "arithmetic, timed on the headline's tensors)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures this path on exactly one GPU; --gpus %d is not supported. "
              "Rows are independent, so several GPUs would each run the one-GPU kernel on a "
              "contiguous range of rows with no communication." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.calibrate:
        calibrate(args.steps, args.warmup, dev)
        return

    import rmsnorm_diffusion_transformers_amd as rn
    import synth
    from rmsnorm_diffusion_transformers_amd import hbm
    if args.placement_map:
        placement_map(rn, dev)
        return
    if args.placement_widths:
        placement_widths(rn, dev)
        return
    if args.placement_arena_sizes:
        placement_arena_sizes(rn, dev)
        return
    if args.small_batch:
        print(json.dumps({"small_batch_latency": small_batch_latency(rn, dev)}), flush=True)
        return
    if args.placement_thirds:
        placement_thirds(rn, dev)
        return
    if args.placement_counters:
        placement_counters(rn, dev)
        return
    wl = synth.WORKLOADS[args.workload]
    want_extras = not args.no_extras and args.workload == HEADLINE
    companions_wanted = not args.no_companion and args.workload == HEADLINE
    nbytes = wl.algorithmic_bytes()
    inp = make_inputs(wl)
    extra_out = [((wl.R, wl.D), torch.float32), ((wl.R, wl.D), torch.float8_e4m3fn)] if want_extras else []
    want_ref = not args.no_reference and args.workload == HEADLINE
    ref_missing = want_ref and not os.path.exists(REF_LIB)
    if ref_missing:
        # a measurement aid, not the operation: the line says it is missing
        log("libtrafficref.so is not built (%s); the traffic references are skipped" % REF_LIB)
        want_ref = False
    ref_torch, ref_planned = {}, None
    mix_torch, variants_torch = None, []

    # Row-kernel launches before the timed workloads (the torch-allocation
    # passes and the placement trials), so that a kernel trace can be split.
    prelude = 0
    placement = {"kind": "default"}
    arena = None
    plans = {}
    comp_inputs = {}
    torch_alloc = {}
    if companions_wanted:
        for name in COMPANIONS:
            comp_inputs[name] = make_inputs(synth.WORKLOADS[name])
    if args.placement == "planned":
        # what torch's own back-to-back allocations give, for every large
        # workload, measured first (each workload's tensors freed after it)
        for name, winp in [(wl.name, inp)] + list(comp_inputs.items()):
            w = synth.WORKLOADS[name]
            with_ref = want_ref and name in REF_WORKLOADS
            with_mix = name == wl.name and want_extras
            if with_ref or with_mix:
                dms, _, _, kept = time_workload(rn, w, args.steps, args.warmup, dev, keep=True,
                                                inp=winp, extra_out=extra_out if with_mix else ())
            else:
                dms, _, _ = time_workload(rn, w, args.steps, args.warmup, dev, inp=winp)
            prelude += settle_launches() + args.steps + args.warmup
            if with_ref:
                ref_torch[name] = traffic_reference_rate(w, kept[0], kept[1], kept[2], args.steps,
                                                         args.warmup)
                log("%s traffic reference, torch allocations: %.4f ms/launch, %.1f GB/s"
                    % (name, ref_torch[name]["ms_per_launch"], ref_torch[name]["GB/s"]))
            if with_mix:
                # the variants and the mix on the same torch allocations
                variants_torch, mix_torch = extras(rn, kept, args.steps, args.warmup)
                prelude += mix_torch["row_kernel_launches"]
                log("DiT forward mix, torch allocations: %.2f ms" % mix_torch["ms_per_forward"])
            if with_ref or with_mix:
                del kept
                torch.cuda.empty_cache()
            dg = w.algorithmic_bytes() / (dms * 1e-3) / 1e9
            log("%s, torch allocations: %.4f ms/launch, %.1f GB/s" % (name, dms, dg))
            torch_alloc[name] = {"ms_per_launch": round(dms, 5), "GB/s": round(dg, 1),
                                 "frac": round(dg / HBM_PEAK_GBS, 4)}
        placement["default_allocation"] = torch_alloc[wl.name]
        try:
            arena = hbm.HbmArena(dev)
            if arena.granules < 3:
                raise RuntimeError("only %d granules of free HBM" % arena.granules)
        except RuntimeError as e:
            log("no HBM arena (%s); torch allocations are used" % e)
            placement["note"] = str(e)
            arena = None
            torch.cuda.empty_cache()
    if arena is not None:
        placement["arena_granules"] = arena.granules
        try:
            pl, info = plan_workload(rn, wl, inp, arena, dev, extra_out)
            plans[wl.name] = pl
            placement["kind"] = "planned"
            placement.update(info)
            prelude += hbm.launches(pl.candidates)
        except ValueError as e:
            log("%s: no placement (%s); torch allocations are used" % (wl.name, e))
            placement["note"] = str(e)
        for name, cinp in comp_inputs.items():
            try:
                plans[name], _ = plan_workload(rn, synth.WORKLOADS[name], cinp, arena, dev)
                prelude += hbm.launches(plans[name].candidates)
            except ValueError as e:
                log("%s: no placement (%s); torch allocations are used" % (name, e))
    log("row-kernel launches before the timed workloads: %d" % prelude)

    pl = plans.get(wl.name)
    ms, wall, per_launch, kept = time_workload(rn, wl, args.steps, args.warmup, dev, keep=True,
                                               stats=True, inp=inp, arena=arena, placement=pl,
                                               extra_out=extra_out)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("%s: %.4f ms/launch, %.1f GB/s (%.1f%% of %g)" % (wl.name, ms, gbs, 100 * gbs / HBM_PEAK_GBS,
                                                          HBM_PEAK_GBS))
    copy_placed = None
    if pl is not None:
        d, y = kept[0], kept[1]
        cms, _ = time_calls(lambda: torch.neg(d["x"], out=y), args.steps, args.warmup)
        nb = 2 * wl.R * wl.D * 2
        copy_placed = {"kernel": "torch.neg bf16, x -> y at the planned offsets", "bytes_per_launch": nb,
                       "ms_per_launch": round(cms, 5), "GB/s": round(nb / cms / 1e6, 1),
                       "frac": round(nb / cms / 1e6 / HBM_PEAK_GBS, 4)}
        del d, y   # views of the arena: the arena is released below
    if want_ref:
        ref_planned = traffic_reference_rate(wl, kept[0], kept[1], kept[2], args.steps, args.warmup)
        log("traffic reference: %.4f ms/launch, %.1f GB/s" % (ref_planned["ms_per_launch"],
                                                              ref_planned["GB/s"]))
    if want_extras:
        variants, mix = extras(rn, kept, args.steps, args.warmup)
    del kept
    torch.cuda.empty_cache()
    companions = []
    if companions_wanted:
        for name in COMPANIONS:
            wc = synth.WORKLOADS[name]
            cinp = comp_inputs.pop(name, None)
            cref = None
            if want_ref and name in REF_WORKLOADS:
                cms, _, cstats, ckept = time_workload(rn, wc, args.steps, args.warmup, dev, stats=True,
                                                      inp=cinp, arena=arena, placement=plans.get(name),
                                                      keep=True)
                cref = traffic_reference_rate(wc, ckept[0], ckept[1], ckept[2], args.steps, args.warmup)
                log("%s traffic reference: %.4f ms/launch, %.1f GB/s" % (name, cref["ms_per_launch"],
                                                                         cref["GB/s"]))
                del ckept
                torch.cuda.empty_cache()
            else:
                cms, _, cstats = time_workload(rn, wc, args.steps, args.warmup, dev, stats=True,
                                               inp=cinp, arena=arena, placement=plans.get(name))
            del cinp
            cg = wc.algorithmic_bytes() / (cms * 1e-3) / 1e9
            log("%s: %.4f ms/launch, %.1f GB/s" % (wc.name, cms, cg))
            ci = rn.describe_launch(wc.B, wc.L, wc.D, flags_of(rn, wc), wc.op == "fused",
                                    wc.gate_layout or (0, 0), wc.ss_layout)
            entry = {"workload": wc.name, "ms_per_launch": round(cms, 5),
                     "GB/s": round(cg, 1), "frac": round(cg / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": wc.algorithmic_bytes(),
                     "traffic": measured_traffic(wc.name), "launch_ms": cstats,
                     "launch": ci}
            if name in plans:
                entry["placement"] = plans[name].describe()
            if name in torch_alloc:
                entry["torch_allocation"] = torch_alloc[name]
            if cref is not None:
                entry["traffic_reference"] = traffic_reference_entry(
                    wc, cref, ref_torch.get(name), cg, torch_alloc.get(name),
                    "planned" if name in plans else "default")
            companions.append(entry)
    if arena is not None:
        arena.release()
        arena = None
        torch.cuda.empty_cache()
    if pl is not None and want_extras:
        # the same planning in an arena of 3 granules (96 GiB), the size a
        # process holding a model's weights beside it can spare
        try:
            a3 = hbm.HbmArena(dev, granules=3)
            pl3, info3 = plan_workload(rn, wl, inp, a3, dev)
            ms3, _, _ = time_workload(rn, wl, args.steps, args.warmup, dev, inp=inp, arena=a3,
                                      placement=pl3)
            g3 = nbytes / (ms3 * 1e-3) / 1e9
            placement["arena_3_granules"] = {
                "gib": a3.nbytes >> 30, "candidates": pl3.candidates, "search_s": info3["search_s"],
                "ms_per_launch": round(ms3, 5), "GB/s": round(g3, 1), "frac": round(g3 / HBM_PEAK_GBS, 4)}
            log("%s in a 96 GiB arena: %.4f ms/launch, %.1f GB/s" % (wl.name, ms3, g3))
            a3.release()
            del a3
        except (RuntimeError, ValueError) as e:
            placement["arena_3_granules"] = {"note": str(e)}
        torch.cuda.empty_cache()
    del inp
    info = rn.describe_launch(wl.B, wl.L, wl.D, flags_of(rn, wl), wl.op == "fused",
                              wl.gate_layout or (0, 0), wl.ss_layout)
    ref = copy_reference(args.steps, args.warmup, dev)
    log("copy reference: %.1f GB/s" % ref["GB/s"])
    line = {
        "metric": "fused residual-norm HBM GB/s and % of peak, bf16 L=176400 D=5120",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, U(0,1) gate, N(0,0.1) scale/shift)",
        "config": {"workload": wl.name, "op": wl.op, "norm": "rms" if wl.is_rms else "layer",
                   "B": wl.B, "L": wl.L, "D": wl.D, "frames": 49 if wl.gate_layout == (2, 49) else None,
                   "gate_layout": wl.gate_layout, "ss_layout": wl.ss_layout,
                   "algorithmic_bytes": nbytes, "launch": info},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                     "frac_torch_allocation": torch_alloc.get(wl.name, {}).get("frac")},
        # the same kernel and workload on torch's own back-to-back allocations
        # (x, residual, y, residual_out allocated one after the other)
        "torch_allocation": torch_alloc.get(wl.name),
        "placement": placement,
        "wall_s_timed_region": round(wall, 4),
        "launch_ms": per_launch,
        "companions": companions,
        "copy_reference": ref,
    }
    if copy_placed is not None:
        line["copy_reference_placed"] = copy_placed
    if ref_missing:
        line["traffic_reference"] = {"skipped": "libtrafficref.so is not built"}
    if want_ref:
        line["traffic_reference"] = traffic_reference_entry(wl, ref_planned, ref_torch.get(wl.name), gbs,
                                                            torch_alloc.get(wl.name), placement["kind"])
    if want_extras:
        line["variants"] = variants
        if mix_torch is not None:
            mix["torch_allocation_ms_per_forward"] = mix_torch["ms_per_forward"]
        on_torch = {v["variant"]: v for v in variants_torch}
        for v in variants:
            t = on_torch.get(v["variant"])
            if t is not None:
                v["torch_allocation"] = {k: t[k] for k in ("ms_per_launch", "GB/s", "frac")}
        line["dit_forward_mix"] = mix
        line["small_batch_latency"] = small_batch_latency(rn, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
