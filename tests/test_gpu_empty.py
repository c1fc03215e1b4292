"""Degenerate sizes through the C ABI: zero rows (tokens), an all-empty
grouped problem (every expert group empty), zero routed tokens.  Each call
must return FP8BS_OK, launch nothing that touches memory and leave every
output byte as it was (the buffers passed are real, so a kernel that ran
anyway would show)."""
import numpy as np
import pytest
import torch

from fp8_block_scaled_x128_amd import ops

pytestmark = pytest.mark.gpu

SENT = 0xA5


def _u8(n):
    return torch.full((n,), SENT, dtype=torch.uint8, device="cuda")


def _untouched(*bufs):
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.all(b.view(torch.uint8) == SENT), "an output was written by a call with nothing to do"


def test_quantizers_zero_rows():
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    q, s = _u8(4096), _u8(4096)
    sf = s.view(torch.float32)
    assert ops.fp8_quant_rowblock(x, 0, 256, 256, ops.AXIS_ROW, q, 256, sf, 1, 8) == 0
    assert ops.fp8_quant_rowblock(x, 0, 256, 256, ops.AXIS_COL, q, 16, sf, 2, 1) == 0
    assert ops.fp8_quant_block2d(x, 1, 0, 256, 256, q, 256, q, 16, sf) == 0
    assert ops.fp8_quant_rowwise(x, 0, 256, 256, q, 256, sf) == 0
    assert ops.mxfp8_quant(x, 0, 256, 256, q, 256, s, 8, 1) == 0
    assert ops.fp8_quant_pow2(x, 0, 256, 256, 1, q, 256, s, 4) == 0
    assert ops.fp8_quant_linear(x, 0, 256, 256, q, 256, sf, 1, 8, x, 0, 256, q, 256, sf) == 0
    assert ops.fp8_silu_mul_quant(x, 0, 128, 256, 0, q, 128, sf, 1, 8, None, 0) == 0
    _untouched(q, s)


def test_tensorwise_zero_rows_writes_zero_scale():
    """An empty tensor's single group has amax 0, so its scale is 0 (the
    all-zero-group rule); nothing else is written."""
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    q, s = _u8(4096), torch.full((4,), -1.0, dtype=torch.float32, device="cuda")
    assert ops.fp8_quant_tensorwise(x, 0, 256, 256, q, 256, s) == 0
    torch.cuda.synchronize()
    assert s[0].item() == 0.0 and torch.all(s[1:] == -1.0)
    _untouched(q)


def test_gemms_zero_rows():
    a = torch.zeros((8, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((8, 2), dtype=torch.float32, device="cuda")
    c = _u8(8 * 128 * 4)
    for out in (ops.OUT_BF16, ops.OUT_FP32):
        assert ops.fp8_blockscaled_gemm(0, 128, 256, a, 256, sa, 2, 1, a, 256, sa, 2, 1, ops.BSCALE_BLOCK128,
                                        c, 128, out) == 0
        assert ops.fp8_blockscaled_gemm_pow2(0, 128, 256, a, 256, a, 4, a, 256, a, 4, c, 128, out) == 0
        assert ops.mxfp8_gemm(0, 128, 256, 0, None, None, 0, a, 256, a, 8, a, 256, 0, a, 8, 0, c, 128, out) == 0
    _untouched(c)


@pytest.mark.parametrize("G", [1, 4, 300])
def test_grouped_all_groups_empty(G):
    """total_rows = 0 with G groups whose offsets are all zero: the grouped
    GEMMs (with and without the gather) and both fused gate/up kernels write
    nothing."""
    offs = torch.zeros(G + 1, dtype=torch.int32, device="cuda")
    a_rows = torch.zeros(8, dtype=torch.int32, device="cuda")
    a = torch.zeros((8, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((G * 256, 256), dtype=torch.uint8, device="cuda")
    sa = torch.ones((8, 2), dtype=torch.float32, device="cuda")
    sb = torch.ones((G, 2, 2), dtype=torch.float32, device="cuda")
    eb = torch.full((G * 256, 8), 127, dtype=torch.uint8, device="cuda")
    c, hq, hs = _u8(8 * 256 * 4), _u8(8 * 128), _u8(64)
    for gather, cnt in ((None, 0), (a_rows, 8)):
        for out in (ops.OUT_BF16, ops.OUT_FP32):
            assert ops.fp8_grouped_gemm(0, 256, 256, G, offs, gather, cnt, a, 256, sa, 2, 1, b, 256, 256 * 256,
                                        sb, 4, 2, 1, c, 256, out) == 0
            assert ops.mxfp8_gemm(0, 256, 256, G, offs, gather, cnt, a, 256, eb, 8, b, 256, 256 * 256, eb, 8,
                                  256 * 8, c, 256, out) == 0
        assert ops.fp8_grouped_gemm_swiglu_quant(0, 128, 256, G, offs, gather, cnt, a, 256, sa, 2, 1, b, 256,
                                                 256 * 256, sb, 4, 2, 1, hq, 128, hs.view(torch.float32), 1, 8) == 0
        assert ops.mxfp8_grouped_gemm_swiglu_quant(0, 128, 256, G, offs, gather, cnt, a, 256, eb, 8, b, 256,
                                                   256 * 256, eb, 8, 256 * 8, hq, 128, hs, 4, 1) == 0
    _untouched(c, hq, hs)


def test_combine_zero_tokens():
    y = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(8, dtype=torch.int32, device="cuda")
    w = torch.ones(8, dtype=torch.float32, device="cuda")
    out = _u8(8 * 128 * 4)
    for ot in (ops.OUT_BF16, ops.OUT_FP32):
        assert ops.fp8_moe_combine(y, 8, 128, 128, pos, w, 0, 8, out, 128, ot) == 0
    _untouched(out)
