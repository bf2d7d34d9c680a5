"""The HBM arena and the measured placement on the GPU: a planned placement
changes where the operands live, never the results."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import FULL_SIZE_MIN_IDENTICAL, compare_outputs, log, require_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_planned_placement_gives_the_same_bits():
    import torch

    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    from rmsnorm_diffusion_transformers_amd import hbm

    B, L, D, F = 1, 4096, 5120, 4
    log("hbm placement: fused LN per-frame B %d L %d D %d F %d, 3-granule arena" % (B, L, D, F))
    x = synth.random_bf16((L, D), seed=21, tensor=synth.X)
    r = synth.random_bf16((L, D), seed=21, tensor=synth.RES)
    g = synth.random_bf16((F, D), seed=21, tensor=synth.GATE, dist=synth.UNIFORM)
    sc = synth.random_bf16((F, D), seed=21, tensor=synth.SCALE, b=0.1)
    sh = synth.random_bf16((F, D), seed=21, tensor=synth.SHIFT, b=0.1)
    dg, dsc, dsh = to_dev(g), to_dev(sc), to_dev(sh)
    lay = (rn.RN_FRAME, F)
    stream = torch.cuda.current_stream()

    def run(xd, rd, yd, od):
        rn.resnorm_fused_fwd(yd, od, xd, rd, dg, None, None, dsc, dsh, B, L, D, rn.RN_GATE,
                             lay, lay, 1e-6, stream)

    # torch's own allocations
    xd, rd = to_dev(x), to_dev(r)
    yd, od = torch.empty_like(xd), torch.empty_like(xd)
    run(xd, rd, yd, od)
    torch.cuda.synchronize()
    y_ref, ro_ref = to_host(yd), to_host(od)

    arena = hbm.HbmArena(granules=3)
    bf = torch.bfloat16

    def make_launch(ins, outs):
        return lambda: run(ins[0], ins[1], outs[0][0], outs[1])

    # y shares its granule with a binary32 tensor of the same shape (as a
    # second output type would); residual_out gets its own granule
    (xa, ra), (ygroup, oa), pl = hbm.place_streams(
        arena, [((L, D), bf), ((L, D), bf)], [[((L, D), bf), ((L, D), torch.float32)], ((L, D), bf)],
        make_launch, stream=stream)
    ya, y32 = ygroup
    assert pl.candidates == 4 and len(pl.trials) == 7 and pl.read_granule in (0, 1)
    assert len({pl.read_granule, *pl.write_granules}) == 3
    base = arena.buf.data_ptr()
    granule = lambda t: (t.data_ptr() - base) // hbm.GRANULE  # noqa: E731
    assert y32.data_ptr() >= ya.data_ptr() + L * D * 2
    assert granule(y32) == granule(ya) == pl.write_granules[0]
    assert granule(oa) == pl.write_granules[1] and granule(xa) == granule(ra) == pl.read_granule
    xa.copy_(xd)
    ra.copy_(rd)
    ya.fill_(float("nan"))
    oa.fill_(float("nan"))
    run(xa, ra, ya, oa)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(oa), ro_ref)
    assert np.array_equal(to_host(ya), y_ref)
    # and against the oracle on the placed outputs
    y_o, ro_o, _ = oracle.Oracle().fused(x, r, g, None, None, sc, sh, B, L, D, False,
                                         gate_layout=(2, F), ss_layout=(2, F), threads=8)
    compare_outputs(to_host(ya), y_o, to_host(oa), ro_o, what="placed")
    # the arena's heap hands out memory outside every placed tensor; writing
    # it leaves the placed tensors as they were
    placed = [(t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()) for t in (xa, ra, ya, y32, oa)]
    held = []
    for shape, dt in (((D, D), bf), ((3, D), torch.float32), ((1 << 28,), torch.uint8)):
        w = arena.alloc(shape, dt)
        lo, hi = w.data_ptr(), w.data_ptr() + w.numel() * w.element_size()
        assert (lo - base) % hbm.ALIGN == 0 and base <= lo and hi <= base + arena.nbytes
        assert all(hi <= a or lo >= b for a, b in placed + held)
        held.append((lo, hi))
        w.view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ya), y_ref) and np.array_equal(to_host(oa), ro_ref)
    assert torch.equal(xa, xd) and torch.equal(ra, rd)
    del xa, ra, ya, oa, y32, ygroup, w
    arena.release()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["fused_ln_frame_b1_f49_l176400_d5120", "nss_ln_b1_l176400_d5120"])
def test_full_size_workload_on_a_planned_placement(name):
    """Every row of a full-size workload with its streamed tensors at a planned
    placement (as bench.py times it), against the oracle."""
    import os

    import torch

    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn
    from rmsnorm_diffusion_transformers_amd import hbm
    from gpu_util import launch_workload

    threads = max(1, min(16, os.cpu_count() or 1))
    wl = synth.WORKLOADS[name]
    log("workload %s on a planned placement: generating inputs" % name)
    inp = synth.make_inputs(wl, threads=threads)
    fused = wl.op == "fused"
    streamed = ["x", "residual"] if fused else ["x"]
    small = {k: to_dev(v) for k, v in inp.items() if k not in streamed}
    act = ((wl.R, wl.D), torch.bfloat16)
    arena = hbm.HbmArena(granules=3)

    def make_launch(ins, outs):
        d = dict(small, **dict(zip(streamed, ins)))
        return lambda: launch_workload(rn, wl, d, outs[0], outs[1] if fused else None)

    ins, outs, pl = hbm.place_streams(arena, [act] * len(streamed), [act] * (2 if fused else 1),
                                      make_launch)
    log("placement: inputs @ %d, outputs @ %s" % (pl.read_granule, list(pl.write_granules)))
    for k, v in zip(streamed, ins):
        v.copy_(to_dev(inp[k]))
    for o in outs:
        o.fill_(float("nan"))
    make_launch(ins, outs)()
    torch.cuda.synchronize()
    yh = to_host(outs[0])
    roh = to_host(outs[1]) if fused else None
    del ins, outs
    arena.release()
    torch.cuda.empty_cache()
    log("workload %s: oracle on %d rows x %d threads" % (name, wl.R, threads))
    y_ref, ro_ref, _ = oracle.Oracle().run_workload(wl, inp, threads=threads)
    compare_outputs(yh, y_ref, roh, ro_ref, name + " (planned placement)",
                    min_identical=FULL_SIZE_MIN_IDENTICAL)
    log("workload %s on a planned placement: OK" % name)
