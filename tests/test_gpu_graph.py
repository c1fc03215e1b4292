"""The entry points under HIP graph capture: they allocate nothing, set no
memory with runtime calls and keep no state, so a captured sequence replays
like the eager one.  The forward step of a block-wise FP8 linear pair (both
operand quantizations and both GEMMs, "Low Precision RL", section "2.
Unified block-wise FP8 (DeepSeek-style)") and a grouped GEMM with the
dispatch gather are captured once and replayed several times, with other
eager work and a poisoning of every output between replays; each replay
must reproduce the eager results byte for byte."""
import numpy as np
import pytest
import torch

from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16

pytestmark = pytest.mark.gpu


def _bits(shape, seed, sigma=1.0, frac=0.0, mult=1.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def test_forward_step_and_grouped_gemm_replay():
    T, H, I = 1024, 1280, 2560
    x_up, w_up = dev_bf16(_bits((T, H), 70, 1.0, 0.01, 50.0)), dev_bf16(_bits((I, H), 71, 0.02))
    x_dn, w_dn = dev_bf16(_bits((T, I), 72, 1.0, 0.01, 50.0)), dev_bf16(_bits((H, I), 73, 0.02))
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    qxu, sxu, qwu, swu = u8(T, H), f32(H // 128, T), u8(I, H), f32(I // 128, H // 128)
    qxd, sxd, qwd, swd = u8(T, I), f32(I // 128, T), u8(H, I), f32(H // 128, I // 128)
    yu = torch.empty((T, I), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    # grouped: 6 experts (one empty), rows gathered from the quantized x_up
    d = inputs.small_moe(seed=74, tokens=512, hidden=H, experts=6, inter=128, top_k=2)
    r = d["routing"]
    rows, G, N = int(r.offsets[-1]), 6, 256
    offs, a_rows = dev(r.offsets), dev(r.row_token)
    qb = dev(np.random.default_rng(75).integers(0, 120, size=(G, N, H)).astype(np.uint8))
    sb = torch.full((G, N // 128, H // 128), 0.01, dtype=torch.float32, device="cuda")
    yg = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    outs = [qxu, sxu, qwu, swu, yu, qxd, sxd, qwd, swd, yd, yg]

    def step():
        ops.fp8_quant_linear(x_up, T, H, H, qxu, H, sxu, 1, T, w_up, I, H, qwu, H, swu)
        ops.fp8_blockscaled_gemm(T, I, H, qxu, H, sxu, 1, T, qwu, H, swu, H // 128, 1, ops.BSCALE_BLOCK128,
                                 yu, I, ops.OUT_BF16)
        ops.fp8_quant_linear(x_dn, T, I, I, qxd, I, sxd, 1, T, w_dn, H, I, qwd, I, swd)
        ops.fp8_blockscaled_gemm(T, H, I, qxd, I, sxd, 1, T, qwd, I, swd, I // 128, 1, ops.BSCALE_BLOCK128,
                                 yd, H, ops.OUT_BF16)
        ops.fp8_grouped_gemm(rows, N, H, G, offs, a_rows, T, qxu, H, sxu, 1, T, qb, H, N * H, sb,
                             sb.stride(0), sb.stride(1), sb.stride(2), yg, N, ops.OUT_FP32)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5 + rep)     # poison every output (eager fill kernels)
        junk = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")   # other eager work
        g.replay()
        torch.cuda.synchronize()
        del junk
        for k, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), "replay %d: output %d differs" % (rep, k)
