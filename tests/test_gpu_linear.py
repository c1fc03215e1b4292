"""The Python conveniences for one block-wise FP8 linear layer ("Low
Precision RL", section "2. Unified block-wise FP8 (DeepSeek-style)": 1x128
activation groups, 128x128 weight blocks, FP32 scales, the same GEMM for
rollout and training): ops.linear_forward and ops.linear_backward order the
C-ABI calls (they compute nothing themselves).  Their outputs must equal,
byte for byte, the explicit sequence of entry points the bench times, and
meet the GEMM tolerance against the oracle on the quantized operands."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev_bf16, host, verify

pytestmark = pytest.mark.gpu


def test_linear_forward_backward_match_the_entry_points():
    rng = np.random.default_rng(31)
    T, I, O = 512, 640, 768
    xb = inputs.normal_bf16(rng, (T, I), 1.0, 0.01, 50.0)
    wb = inputs.normal_bf16(rng, (O, I), 0.02)
    dyb = inputs.normal_bf16(rng, (T, O), 1e-3)
    x, w, dy = dev_bf16(xb), dev_bf16(wb), dev_bf16(dyb)
    y, saved = ops.linear_forward(x, w)
    dx, dw = ops.linear_backward(dy, saved)
    torch.cuda.synchronize()
    # the explicit sequence
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    qx, sx, qw, sw = u8(T, I), f32(I // 128, T), u8(O, I), f32(O // 128, I // 128)
    ops.fp8_quant_linear(x, T, I, I, qx, I, sx, 1, T, w, O, I, qw, I, sw)
    y2 = torch.empty((T, O), dtype=torch.bfloat16, device="cuda")
    ops.fp8_blockscaled_gemm(T, O, I, qx, I, sx, 1, T, qw, I, sw, I // 128, 1, ops.BSCALE_BLOCK128, y2, O,
                             ops.OUT_BF16)
    qdy, sdy, qdyt, sdyt = u8(T, O), f32(O // 128, T), u8(O, T), f32(T // 128, O)
    ops.fp8_quant_dual_axis(dy, T, O, O, 0, qdy, O, sdy, 1, T, qdyt, T, sdyt, 1, O)
    qxt, sxt, qwt = u8(I, T), f32(T // 128, I), u8(I, O)
    ops.fp8_quant_rowblock(x, T, I, I, ops.AXIS_COL, qxt, T, sxt, 1, I)
    ops.fp8_transpose_codes(qw, 1, O, I, I, qwt, O)
    dx2, dw2 = f32(T, I), f32(O, I)
    ops.fp8_blockscaled_gemm(T, I, O, qdy, O, sdy, 1, T, qwt, O, sw, 1, I // 128, ops.BSCALE_BLOCK128, dx2, I,
                             ops.OUT_FP32)
    ops.fp8_blockscaled_gemm(O, I, T, qdyt, T, sdyt, 1, O, qxt, T, sxt, 1, I, ops.BSCALE_ROW128, dw2, I,
                             ops.OUT_FP32)
    torch.cuda.synchronize()
    for a, b in ((y, y2), (dx, dx2), (dw, dw2)):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))
    # dgrad and wgrad against the oracle on the oracle's own operands
    qd_r, sd_r = oracle.quant_1x128(dyb)
    qw_r, sw_r = oracle.quant_128x128(wb)
    qwt_r = np.ascontiguousarray(qw_r.T)
    swt_r = np.ascontiguousarray(sw_r.T)
    verify(qd_r, sd_r, qwt_r, swt_r, host(dx))


def test_moe_forward_matches_the_entry_points():
    """ops.moe_forward on a scaled-down MoE layer (skewed routing with empty
    experts): byte-identical to the chain of entry points it orders (X 1x128,
    gathered gate/up GEMM with SiLU*mul and requantization, grouped down GEMM,
    combine)."""
    d = inputs.small_moe(seed=33, tokens=512, hidden=256, experts=8, inter=128, top_k=2)
    r = d["routing"]
    T, H = d["x"].shape
    G, N2, _ = d["w_gu"].shape
    I = N2 // 2
    rows = int(r.offsets[-1])
    x = dev_bf16(d["x"])
    qgu, sgu, _ = ops.quant_block2d(dev_bf16(d["w_gu"]))
    wd = dev_bf16(d["w_d"])
    qdt = torch.empty((G, H, I), dtype=torch.uint8, device="cuda")
    sdt = torch.empty((G, I // 128, H // 128), dtype=torch.float32, device="cuda")
    ops.fp8_quant_block2d(wd, G, I, H, H, None, 0, qdt, I, sdt)
    offs = torch.from_numpy(r.offsets).cuda()
    a_rows = torch.from_numpy(r.row_token).cuda()
    pos = torch.from_numpy(r.token_rows).cuda()
    wts = torch.from_numpy(r.weights).cuda()
    out = ops.moe_forward(x, qgu, sgu, qdt, sdt, offs, a_rows, pos, wts)
    # the explicit chain
    qx = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sx = torch.empty((H // 128, T), dtype=torch.float32, device="cuda")
    ops.fp8_quant_rowblock(x, T, H, H, ops.AXIS_ROW, qx, H, sx, 1, T)
    qh = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    sh = torch.empty((I // 128, rows), dtype=torch.float32, device="cuda")
    ops.fp8_grouped_gemm_swiglu_quant(rows, I, H, G, offs, a_rows, T, qx, H, sx, 1, T, qgu, H, N2 * H, sgu,
                                      (N2 // 128) * (H // 128), H // 128, 1, qh, I, sh, 1, rows)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    ops.fp8_grouped_gemm(rows, H, I, G, offs, None, rows, qh, I, sh, 1, rows, qdt, I, H * I, sdt,
                         (I // 128) * (H // 128), 1, H // 128, y, H, ops.OUT_BF16)
    out2 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ops.fp8_moe_combine(y, rows, H, H, pos, wts, T, r.token_rows.shape[1], out2, H, ops.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
