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


def test_backward_step_replay():
    """The backward step of the block-wise FP8 linear layer under capture:
    dY's two groupings from one read (fp8_quant_dual_axis, 1x128 for dgrad
    and 128x1 for wgrad, and its MX form), X in 128x1 groups, the transposed
    copy of the forward's weight codes (fp8_transpose_codes), dgrad and wgrad
    (fp32 out), and the power-of-two operand pair.  Every replay, with the
    outputs poisoned and other eager work between replays, reproduces the
    eager bytes."""
    T, I, O = 1024, 1280, 2560
    dy = dev_bf16(_bits((T, O), 80, 1e-3))
    x = dev_bf16(_bits((T, I), 81, 1.0, 0.01, 50.0))
    w = dev_bf16(_bits((O, I), 82, 0.02))
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    # the forward's weight codes and scales, made once
    qw, sw = u8(O, I), f32(O // 128, I // 128)
    ops.fp8_quant_block2d(w, 1, O, I, I, qw, I, None, 0, sw)
    qdy, sdy, qdyt, sdyt = u8(T, O), f32(O // 128, T), u8(O, T), f32(T // 128, O)
    mq, ms, mqt, mst = u8(T, O), u8(T, O // 32), u8(O, T), u8(O, T // 32)
    qxt, sxt, qwt = u8(I, T), f32(T // 128, I), u8(I, O)
    dx, dw = f32(T, I), f32(O, I)
    lds = 4 * ((I + 511) // 512)
    px, psx, pw, psw = u8(T, I), u8(T, lds), u8(O, I), u8(O // 128, lds)
    outs = [qdy, sdy, qdyt, sdyt, mq, ms, mqt, mst, qxt, sxt, qwt, dx, dw, px, psx, pw, psw]
    # compared: the written part of each output (the power-of-two scale rows
    # are padded to the GEMM's 4-byte words; the quantizer writes ceil(I/128)
    # bytes of each)
    g = (I + 127) // 128
    written = outs[:14] + [psx[:, :g], pw, psw[:, :g]]

    def step():
        ops.fp8_quant_dual_axis(dy, T, O, O, 0, qdy, O, sdy, 1, T, qdyt, T, sdyt, 1, O)
        ops.fp8_quant_dual_axis(dy, T, O, O, 1, mq, O, ms, O // 32, 1, mqt, T, mst, T // 32, 1)
        ops.fp8_quant_rowblock(x, T, I, I, ops.AXIS_COL, qxt, T, sxt, 1, I)
        ops.fp8_transpose_codes(qw, 1, O, I, I, qwt, O)
        ops.fp8_blockscaled_gemm(T, I, O, qdy, O, sdy, 1, T, qwt, O, sw, 1, I // 128, ops.BSCALE_BLOCK128, dx, I,
                                 ops.OUT_FP32)
        ops.fp8_blockscaled_gemm(O, I, T, qdyt, T, sdyt, 1, O, qxt, T, sxt, 1, I, ops.BSCALE_ROW128, dw, I,
                                 ops.OUT_FP32)
        ops.fp8_quant_linear_pow2(x, T, I, I, px, I, psx, lds, w, O, I, pw, I, psw, lds)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in written]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for o in outs:
            o.view(torch.uint8).fill_(0x5C + rep)
        junk = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        graph.replay()
        torch.cuda.synchronize()
        del junk
        for k, (o, e) in enumerate(zip(written, ref)):
            assert torch.equal(o.contiguous().view(torch.uint8), e.contiguous().view(torch.uint8)), \
                "replay %d: output %d differs" % (rep, k)
