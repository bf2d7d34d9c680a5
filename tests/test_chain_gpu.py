"""Chained blocks, as a DiT forward runs them: per block a norm-only call on
the residual stream, a fused call with binary32 weight/bias and a fused call
without affine, each writing the residual stream in place (residual_out ==
residual).  Every residual update is exact in binary32 and rounded once, so
the chained stream must match the oracle's chain bit for bit after every
block; every y is held to the contract's bar."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_outputs, log, require_gpu, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_chained_blocks_keep_the_residual_stream_bit_exact():
    import torch

    require_gpu()
    import rmsnorm_diffusion_transformers_amd as rn

    B, L, D, blocks = 1, 384, 5120, 12
    orc = oracle.Oracle()
    rng = np.random.default_rng(77)
    res = synth.random_bf16((L, D), 77, synth.RES)
    w32 = (1.0 + 0.05 * rng.standard_normal(D)).astype(np.float32)
    b32 = (0.1 * rng.standard_normal(D)).astype(np.float32)
    d_res = to_dev(res)
    d_w, d_b = torch.from_numpy(w32).cuda(), torch.from_numpy(b32).cuda()
    bc = (rn.RN_BCAST, 0)
    for k in range(blocks):
        x1 = synth.random_bf16((L, D), 100 + k, synth.X)
        x2 = synth.random_bf16((L, D), 200 + k, synth.X)
        g1, g2 = (synth.random_bf16((1, D), s + k, synth.GATE, dist=synth.UNIFORM) for s in (300, 400))
        sc = [synth.random_bf16((1, D), s + k, synth.SCALE, b=0.1) for s in (500, 600, 700)]
        sh = [synth.random_bf16((1, D), s + k, synth.SHIFT, b=0.1) for s in (800, 900, 1000)]
        ds = [to_dev(a) for a in sc]
        dh = [to_dev(a) for a in sh]
        # GPU: norm-only on the stream, then two fused calls updating it in place
        y0 = torch.empty_like(d_res)
        rn.norm_scale_shift_fwd(y0, d_res, None, None, ds[0], dh[0], B, L, D, 0, bc, 1e-6)
        y1 = torch.empty_like(d_res)
        rn.resnorm_fused_fwd_ex(y1, d_res, to_dev(x1), d_res, to_dev(g1), d_w, d_b, ds[1], dh[1], B, L, D,
                                rn.RN_GATE | rn.RN_WEIGHT | rn.RN_BIAS, bc, bc, 1e-6, rn.RN_DTYPE_F32)
        y2 = torch.empty_like(d_res)
        rn.resnorm_fused_fwd(y2, d_res, to_dev(x2), d_res, to_dev(g2), None, None, ds[2], dh[2], B, L, D,
                             rn.RN_GATE, bc, bc, 1e-6)
        torch.cuda.synchronize()
        # oracle: the same chain on the host
        y0_o, _ = orc.nss(res, None, None, sc[0], sh[0], B, L, D, False, threads=8)
        y1_o, res, _ = orc.fused(x1, res, g1, w32, b32, sc[1], sh[1], B, L, D, False, threads=8,
                                 affine_f32=True)
        y2_o, res, _ = orc.fused(x2, res, g2, None, None, sc[2], sh[2], B, L, D, False, threads=8)
        compare_outputs(to_host(y0), y0_o, what="block %d norm-only" % k)
        compare_outputs(to_host(y1), y1_o, what="block %d fused + affine" % k)
        compare_outputs(to_host(y2), y2_o, to_host(d_res), res, what="block %d fused" % k)
    log("%d chained blocks: residual stream bit-exact after every block" % blocks)
