"""GPU parity of fp8_quant_dual_axis: a tensor's row groups (1x128, or 1x32
MX) and column groups (128x1, or 32x1 MX, written transposed) from one read
of it, the two quantizations of an output gradient dY for the data- and
weight-gradient GEMMs ("Unified FP8: Beyond Mixed Precision...", section
"FP8 Quantization", per-token gradients; "Low Precision RL", section "3.
Unified MXFP8 (Blackwell)").  Codes and scales must be bit-identical to the
oracle's two quantizations, and to the two single-axis entry points."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev_bf16, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed, sigma=1.0, frac=0.01, mult=50.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def _same(a_gpu, b_ref, what):
    a = np.ascontiguousarray(host(a_gpu))
    b = np.ascontiguousarray(b_ref)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.flatnonzero(a != b)
    assert bad.size == 0, "%s: %d mismatches, first at %s: gpu %s ref %s" % (
        what, bad.size, bad[:5], a.reshape(-1)[bad[:5]], b.reshape(-1)[bad[:5]])


def _check(x, mx):
    q, s, qt, st = ops.quant_dual_axis(dev_bf16(x), mx)
    torch.cuda.synchronize()
    if mx:
        qr, sr = oracle.mx_quant_1x32(x)
        qtr, str_ = oracle.mx_quant_32x1_t(x)
    else:
        qr, sr = oracle.quant_1x128(x)
        qtr, str_ = oracle.quant_128x1_t(x)
    _same(q, qr, "row codes")
    _same(s, sr, "row scales")
    _same(qt, qtr, "column codes")
    _same(st, str_, "column scales")


def _specials(x, mx):
    """An all-zero group, a -0 group, a saturating group and a group of bf16
    subnormals along each axis (where the shape has room)."""
    g = 32 if mx else 128
    R, C = x.shape
    if R >= 2 * g and C >= 8:
        x[:g, 0] = 0
        x[g:2 * g, 1] = inputs.to_bf16_bits(np.full(g, 3e38, np.float32))
        x[:g, 2] = inputs.to_bf16_bits((np.arange(g) * 1e-39).astype(np.float32))
        x[:g, 3] = 0x8000
    if C >= 2 * g and R >= 8:
        x[4, :g] = 0
        x[5, g:2 * g] = inputs.to_bf16_bits(np.full(g, -3e38, np.float32))
        x[6, :g] = inputs.to_bf16_bits((np.arange(g) * -1e-39).astype(np.float32))
        x[7, :g] = 0x8000
    return x


@pytest.mark.parametrize("shape", [(512, 384), (272, 72), (16, 8), (400, 520), (4208, 4040), (128, 128)])
def test_dual_fp32_small(shape):
    """Partial 128-row and 128-column tiles, tiles with one 8-column piece,
    and the special groups along both axes."""
    _say("dual fp32", shape)
    _check(_specials(_bits(shape, 11), False), False)


@pytest.mark.parametrize("shape", [(512, 384), (96, 32), (32, 160), (416, 544), (64, 4096)])
def test_dual_mx_small(shape):
    _say("dual mx", shape)
    _check(_specials(_bits(shape, 12), True), True)


def test_dual_division_coverage():
    """Every bf16 significand of x against every bf16 significand of the
    group maximum at several exponent gaps, laid along rows (row groups) and,
    in the transpose, down columns (column groups)."""
    rows = []
    rng = np.random.default_rng(13)
    for gap in (1, 2, 5, 9, 20):
        for ma in range(128):
            amax = np.float32((1 + ma / 128) * 8.0)
            xs = np.array([(1 + m / 128) * 8.0 * 2.0 ** -gap for m in range(128)], np.float32)
            xs *= np.where(np.arange(128) % 2 == 0, 1, -1).astype(np.float32)
            g0 = np.concatenate([[amax], xs[:127]])
            g1 = np.concatenate([[-amax], xs[127:], rng.standard_normal(126).astype(np.float32)])
            rows.append(np.concatenate([g0, g1]).astype(np.float32))
    x = inputs.to_bf16_bits(np.stack(rows))                     # 640 x 256
    _say("dual division coverage", x.shape)
    _check(x, False)
    _check(np.ascontiguousarray(x.T), False)


@pytest.mark.parametrize("mx", [False, True])
def test_dual_qwen3_4b_gradient_full(mx):
    """dY of the Qwen3-4B MLP backward, 4096 tokens x 9728, every code and
    scale of both axes; then byte-identical to the two single-axis calls."""
    dy = inputs.qwen3_4b_mlp_backward(2)["dy"]
    _say("dual full", dy.shape, "mx" if mx else "fp32")
    _check(dy, mx)
    d = dev_bf16(dy)
    q, s, qt, st = ops.quant_dual_axis(d, mx)
    if mx:
        q1, s1 = ops.mx_quant(d)
        qt1, st1 = ops.mx_quant_t(d)
    else:
        q1, s1 = ops.quant_rowblock(d, ops.AXIS_ROW, "m_major")
        qt1, st1 = ops.quant_rowblock(d, ops.AXIS_COL, "m_major")
    torch.cuda.synchronize()
    for a, b in ((q, q1), (s, s1), (qt, qt1), (st, st1)):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_dual_padded_strides():
    """x, q and qt inside wider buffers, scales with custom strides: only the
    described elements are written."""
    R, C = 272, 392
    x = _bits((R, C), 14)
    xb = np.zeros((R, C + 40), np.uint16)
    xb[:, :C] = x
    xd = dev_bf16(xb)
    SENT = 0x5A
    qb = torch.full((R, C + 24), SENT, dtype=torch.uint8, device="cuda")
    qtb = torch.full((C, R + 16), SENT, dtype=torch.uint8, device="cuda")
    ng, ngt = (C + 127) // 128, (R + 127) // 128
    sb = torch.full((R, ng + 3), -1.0, dtype=torch.float32, device="cuda")
    stb = torch.full((C, ngt + 2), -1.0, dtype=torch.float32, device="cuda")
    ops.fp8_quant_dual_axis(xd, R, C, C + 40, 0, qb, C + 24, sb, ng + 3, 1, qtb, R + 16, stb, ngt + 2, 1)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_1x128(x)
    qtr, str_ = oracle.quant_128x1_t(x)
    _same(qb[:, :C], qr, "row codes")
    _same(qtb[:, :R], qtr, "column codes")
    _same(sb[:, :ng], sr, "row scales")
    _same(stb[:, :ngt], str_, "column scales")
    assert torch.all(qb[:, C:] == SENT) and torch.all(qtb[:, R:] == SENT)
    assert torch.all(sb[:, ng:] == -1.0) and torch.all(stb[:, ngt:] == -1.0)


def test_dual_argument_errors_and_empty():
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.full((64 * 256 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    qt = torch.full((64 * 256 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.zeros(4096, dtype=torch.float32, device="cuda")
    st = torch.zeros(4096, dtype=torch.float32, device="cuda")
    call = lambda rows, cols, mx, qq=q, ldqt=64: ops.fp8_quant_dual_axis(
        x, rows, cols, 256, mx, qq, 256, s, 2, 1, qt, ldqt, st, 1, 1, raise_on_error=False)
    assert call(64, 256, 2) == 5                     # FP8BS_ERR_UNSUPPORTED
    assert call(40, 256, 0) == 2                     # rows % 16
    assert call(48, 256, 1) == 2                     # MX rows % 32
    assert call(64, 248, 1) == 2                     # MX cols % 32
    assert call(64, 256, 0, ldqt=60) == 3            # ld_qt < rows
    assert call(64, 256, 0, qq=q[1:]) == 4           # q not 8-byte aligned
    assert call(64, 256, 0, ldqt=68) == 4            # ld_qt % 8
    assert call(0, 256, 0) == 0 and call(64, 0, 1) == 0
    torch.cuda.synchronize()
    assert torch.all(q == 0xA5) and torch.all(qt == 0xA5)


def test_dual_mx_padded_scale_rows():
    """MX scales in padded rows (8 bytes for 5 blocks): the whole first tile
    writes each row's and column's 4 scale bytes as one word, the partial
    second tile byte by byte; the padding bytes stay untouched."""
    R = C = 160
    x = _specials(_bits((R, C), 15), True)
    xd = dev_bf16(x)
    SENT = 0x5A
    q, qt = torch.empty((R, C), dtype=torch.uint8, device="cuda"), torch.empty((C, R), dtype=torch.uint8, device="cuda")
    s = torch.full((R, 8), SENT, dtype=torch.uint8, device="cuda")
    st = torch.full((C, 8), SENT, dtype=torch.uint8, device="cuda")
    ops.fp8_quant_dual_axis(xd, R, C, C, 1, q, C, s, 8, 1, qt, R, st, 8, 1)
    torch.cuda.synchronize()
    qr, sr = oracle.mx_quant_1x32(x)
    qtr, str_ = oracle.mx_quant_32x1_t(x)
    _same(q, qr, "row codes")
    _same(qt, qtr, "column codes")
    _same(s[:, :5], sr, "row scales")
    _same(st[:, :5], str_, "column scales")
    assert torch.all(s[:, 5:] == SENT) and torch.all(st[:, 5:] == SENT)
