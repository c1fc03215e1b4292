"""GPU parity of the quantizers against the CPU oracle: FP8 codes and scales
must be bit-identical ("Unified FP8: Beyond Mixed Precision...", section "FP8
Quantization"; groupings from "Low Precision RL", table "Choose a
precision").  Every call goes through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed, sigma=1.0, frac=0.01, mult=50.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def _assert_same_scales(s_gpu, s_ref):
    a = np.ascontiguousarray(host(s_gpu)).view(np.uint32)
    b = np.ascontiguousarray(s_ref).view(np.uint32)
    assert a.shape == b.shape
    bad = np.flatnonzero(a != b)
    assert bad.size == 0, "scale mismatch at %s: gpu %s ref %s" % (bad[:5], a.reshape(-1)[bad[:5]], b.reshape(-1)[bad[:5]])


def _assert_same_codes(q_gpu, q_ref):
    a = host(q_gpu)
    bad = np.flatnonzero(a != q_ref)
    assert bad.size == 0, "%d code mismatches, first at %s: gpu %s ref %s" % (
        bad.size, bad[:5], a.reshape(-1)[bad[:5]], q_ref.reshape(-1)[bad[:5]])


# ------------------------------------------------------------------- codec
def test_device_codec_table():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = [d for d in dec if not np.isnan(d)]
    grid = dec[:0x7F]
    for c in range(0x7E):
        mid = np.float32((grid[c] + grid[c + 1]) / 2)
        for v in (mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))):
            vals += [v, -v]
    vals += [448.5, 463.99997, 464.0, 465.0, 1e6, 3e38, np.inf, -np.inf, -1e6, 1e-40, -1e-40, 2 ** -10,
             -2 ** -10, 2 ** -11, -2 ** -11, 0.0, -0.0]
    rng = np.random.default_rng(0)
    vals += list(rng.standard_normal(100_000) * np.exp2(rng.uniform(-14, 10, 100_000)))
    v = np.array(vals, np.float32)
    _say("codec probe", v.size)
    out = ops.e4m3_encode(dev(v))
    torch.cuda.synchronize()
    _assert_same_codes(out, oracle.e4m3_encode(v))


# ------------------------------------------------------------ 1x128 groups
@pytest.mark.parametrize("shape,layout", [((256, 512), "m_major"), ((256, 512), "row_major"),
                                          ((7, 264), "m_major"), ((1, 8), "row_major"),
                                          ((300, 1000), "row_major")])
def test_rowblock_small(shape, layout):
    _say("rowblock", shape, layout)
    x = _bits(shape, 1)
    q, s = ops.quant_rowblock(dev_bf16(x), ops.AXIS_ROW, layout)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_1x128(x)
    _assert_same_codes(q, qr)
    _assert_same_scales(s, sr)


def test_rowblock_special_groups():
    x = _bits((6, 256), 2)
    x[0, :128] = 0                                        # zero group
    x[1, :128] = 0x8000                                   # -0 group
    x[2, :128] = inputs.to_bf16_bits(np.linspace(-1e-38, 1e-38, 128).astype(np.float32))   # subnormal S
    x[3, 128:] = inputs.to_bf16_bits(np.linspace(-3e38, 3e38, 128).astype(np.float32))     # huge values
    x[4, :128] = inputs.to_bf16_bits(np.full(128, 448.0, np.float32))
    x[5, 128:] = inputs.to_bf16_bits((np.arange(128) * 1e-20).astype(np.float32))          # S ~ 2^-70
    q, s = ops.quant_rowblock(dev_bf16(x), ops.AXIS_ROW, "row_major")
    torch.cuda.synchronize()
    qr, sr = oracle.quant_1x128(x)
    _assert_same_codes(q, qr)
    _assert_same_scales(s, sr)


def test_rowblock_division_coverage():
    """Every bf16 significand of x against every bf16 significand of amax, at
    several exponent gaps: the device division path must reproduce the IEEE
    division of the oracle bit for bit."""
    rows = []
    rng = np.random.default_rng(3)
    for gap in (1, 2, 5, 9, 20):
        for ma in range(128):
            amax = np.float32((1 + ma / 128) * 8.0)
            xs = np.array([(1 + m / 128) * 8.0 * 2.0 ** -gap for m in range(128)], np.float32)
            xs *= np.where(np.arange(128) % 2 == 0, 1, -1).astype(np.float32)
            g0 = np.concatenate([[amax], xs[:127]])
            g1 = np.concatenate([[-amax], xs[127:], rng.standard_normal(126).astype(np.float32)])
            rows.append(np.concatenate([g0, g1]).astype(np.float32))
    x = inputs.to_bf16_bits(np.stack(rows))
    _say("division coverage", x.shape)
    q, s = ops.quant_rowblock(dev_bf16(x), ops.AXIS_ROW, "row_major")
    torch.cuda.synchronize()
    qr, sr = oracle.quant_1x128(x)
    _assert_same_codes(q, qr)
    _assert_same_scales(s, sr)


def test_rowblock_qwen3_4b_activation_full():
    """Qwen3-4B MLP up-projection input, 4096 x 2560, every code and scale."""
    x = inputs.qwen3_4b_mlp(1, parts=("up",))["x_up"]
    _say("rowblock full", x.shape)
    q, s = ops.quant_rowblock(dev_bf16(x), ops.AXIS_ROW, "m_major")
    torch.cuda.synchronize()
    qr, sr = oracle.quant_1x128(x)
    _assert_same_codes(q, qr)
    _assert_same_scales(s, sr)


def test_rowblock_grid_stride_past_65536_workgroups():
    """A tensor larger than one trip of the row-group grid (65,536
    workgroups x 16 rows of 16 lanes x 4 runs = 4,194,304 runs of 128
    values, about 537M elements): 33,000 x 16,384 (4,224,000 runs) takes the
    grid-stride loop for its last runs, and the streaming-store variant (codes
    above 256 MB).  Every code and scale, both scale layouts, and the MX
    quantizer on the same tensor.  The input is random finite bf16 bit
    patterns (sign, exponent 2^-15..2^9, mantissa uniform): the test is about
    indexing, not value distribution."""
    rows, cols = 33000, 16384
    assert rows * (cols // 128) > 65536 * 16 * 4
    rng = np.random.default_rng(91)
    x = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16) & np.uint16(0x807F)
    x |= (rng.integers(112, 137, size=(rows, cols), dtype=np.uint16) << np.uint16(7)).astype(np.uint16)
    _say("grid-stride rowblock", x.shape)
    xd = dev_bf16(x)
    qr, sr = oracle.quant_1x128(x)
    for layout in ("m_major", "row_major"):
        q, s = ops.quant_rowblock(xd, ops.AXIS_ROW, layout)
        torch.cuda.synchronize()
        _assert_same_codes(q, qr)
        _assert_same_scales(s, sr)
        del q, s
    del qr, sr
    qm, sm = ops.mx_quant(xd)
    torch.cuda.synchronize()
    qr, sr = oracle.mx_quant_1x32(x)
    _assert_same_codes(qm, qr)
    assert np.array_equal(host(sm), sr)


# ------------------------------------------------------------- 128x1 groups
@pytest.mark.parametrize("shape", [(512, 384), (272, 72), (16, 8), (400, 520), (4096, 2560), (4208, 4040)])
def test_colblock_small(shape):
    """128x1 groups down each column, written transposed, with an all-zero
    group, a saturating group and a group of bf16 subnormals.  Grids under
    1024 workgroups take the LDS kernel, (4208, 4040) the register kernel;
    partial 128-row groups and partial 64- and 128-column tiles included."""
    _say("colblock", shape)
    x = _bits(shape, 4)
    if shape[0] >= 256 and shape[1] >= 3:
        x[:128, 0] = 0
        x[128:256, 1] = inputs.to_bf16_bits(np.full(128, 3e38, np.float32))
        x[:128, 2] = inputs.to_bf16_bits((np.arange(128) * 1e-39).astype(np.float32))
    qt, s = ops.quant_rowblock(dev_bf16(x), ops.AXIS_COL, "row_major")
    torch.cuda.synchronize()
    qr, sr = oracle.quant_128x1_t(x)
    _assert_same_codes(qt, qr)
    _assert_same_scales(s, sr)


def test_colblock_qwen3_4b_gradient_full():
    """dY of the Qwen3-4B MLP backward, 4096 tokens x 9728, 128x1 along tokens."""
    dy = inputs.qwen3_4b_mlp_backward(2)["dy"]
    _say("colblock full", dy.shape)
    qt, s = ops.quant_rowblock(dev_bf16(dy), ops.AXIS_COL, "m_major")
    torch.cuda.synchronize()
    qr, sr = oracle.quant_128x1_t(dy)
    _assert_same_codes(qt, qr)
    _assert_same_scales(s, sr)


# ----------------------------------------------------------- 128x128 blocks
@pytest.mark.parametrize("shape", [(512, 512), (272, 200), (16, 8), (3, 384, 256)])
def test_block2d_small(shape):
    _say("block2d", shape)
    w = _bits(shape, 5, 0.02, 0.0, 1.0)
    trans = shape[-2] % 16 == 0
    q, s, qt = ops.quant_block2d(dev_bf16(w), transposed=trans)
    torch.cuda.synchronize()
    ws = w if w.ndim == 3 else w[None]
    qh, sh = host(q).reshape(ws.shape), host(s).reshape(ws.shape[0], -1)
    for b in range(ws.shape[0]):
        qr, sr = oracle.quant_128x128(ws[b])
        assert np.array_equal(qh[b], qr)
        assert np.array_equal(sh[b].view(np.uint32), sr.reshape(-1).view(np.uint32))
        if trans:
            qth = host(qt).reshape(ws.shape[0], ws.shape[2], ws.shape[1])
            assert np.array_equal(qth[b], qr.T)


def test_block2d_qwen3_4b_weight_full():
    w = inputs.qwen3_4b_mlp(1, parts=("up",))["w_up"]
    _say("block2d full", w.shape)
    q, s, qt = ops.quant_block2d(dev_bf16(w), transposed=True)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_128x128(w)
    _assert_same_codes(q, qr)
    _assert_same_scales(s, sr)
    _assert_same_codes(qt, np.ascontiguousarray(qr.T))


@pytest.mark.parametrize("shape", [(272, 200), (3, 384, 256), (768, 2048)])
def test_block2d_transposed_codes_only(shape):
    """q = NULL with q_t given: only the transposed codes and the scales are
    written (a weight stored [in][out], or the data-gradient operand), equal
    to the oracle's; a batch of matrices included."""
    _say("block2d transposed only", shape)
    w = _bits(shape, 6, 0.02, 0.0, 1.0)
    ws = w if w.ndim == 3 else w[None]
    B, R, C = ws.shape
    qt = torch.full((B, C, R), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.empty((B, (R + 127) // 128, (C + 127) // 128), dtype=torch.float32, device="cuda")
    ops.fp8_quant_block2d(dev_bf16(ws), B, R, C, C, None, 0, qt, R, s)
    torch.cuda.synchronize()
    for b in range(B):
        qr, sr = oracle.quant_128x128(ws[b])
        _assert_same_codes(qt[b], np.ascontiguousarray(qr.T))
        _assert_same_scales(s[b], sr)


@pytest.mark.parametrize("shape", [(9728, 2560), (272, 208), (16, 16), (2, 400, 144), (128, 4096)])
def test_transpose_codes(shape):
    """fp8_transpose_codes on codes of the oracle's 128x128 quantization:
    the result equals the transposed codes fp8_quant_block2d writes (and the
    oracle's codes transposed), partial 128-tiles and a batch included; the
    padding of the output rows stays untouched."""
    w = _bits(shape, 8, 0.02, 0.0, 1.0)
    ws = w if w.ndim == 3 else w[None]
    B, R, C = ws.shape
    _say("transpose codes", shape)
    qr = np.stack([oracle.quant_128x128(ws[b])[0] for b in range(B)])
    SENT = 0xA5
    qt = torch.full((B, C, R + 16), SENT, dtype=torch.uint8, device="cuda")
    ops.fp8_transpose_codes(dev(qr), B, R, C, C, qt, R + 16)
    torch.cuda.synchronize()
    for b in range(B):
        _assert_same_codes(qt[b, :, :R], np.ascontiguousarray(qr[b].T))
    assert torch.all(qt[:, :, R:] == SENT)
    if B == 1:
        _, _, qt2 = ops.quant_block2d(dev_bf16(ws[0]), transposed=True)
        torch.cuda.synchronize()
        assert torch.equal(qt2, qt[0, :, :R])


def test_transpose_codes_every_byte_value():
    """The transpose moves bytes: random bytes (every value 0..255, the NaN
    codes 0x7f and 0xff included) through strided views come out transposed
    unchanged."""
    rng = np.random.default_rng(9)
    B, R, C = 2, 528, 400
    q = rng.integers(0, 256, size=(B, R, C + 48), dtype=np.uint8)
    qt = torch.zeros((B, C, R), dtype=torch.uint8, device="cuda")
    qd = dev(q)
    # the matrices start (C + 48) * R bytes apart; fp8_transpose_codes takes
    # batch stride rows * ld_q, which this layout has
    ops.fp8_transpose_codes(qd, B, R, C, C + 48, qt, R)
    torch.cuda.synchronize()
    assert np.array_equal(host(qt), np.ascontiguousarray(np.transpose(q[:, :, :C], (0, 2, 1))))


# ------------------------------------------- both operands in one launch
def _linear_check(x, w, qx, sx, qw, sw):
    qr, sr = oracle.quant_1x128(x)
    _assert_same_codes(qx, qr)
    _assert_same_scales(sx, sr)
    qr, sr = oracle.quant_128x128(w)
    _assert_same_codes(qw, qr)
    _assert_same_scales(sw, sr)


@pytest.mark.parametrize("rows,w_rows,cols", [(300, 200, 1000), (256, 512, 512), (7, 130, 264), (1, 8, 8)])
def test_quant_linear_small(rows, w_rows, cols):
    """X in 1x128 groups and W in 128x128 blocks from one launch: codes and
    scales bit-identical to the oracle (ragged rows, columns and blocks)."""
    _say("quant_linear", rows, w_rows, cols)
    x = _bits((rows, cols), 40 + rows)
    w = _bits((w_rows, cols), 41 + w_rows, 0.02, 0.0, 1.0)
    qx, sx, qw, sw = ops.quant_linear(dev_bf16(x), dev_bf16(w))
    torch.cuda.synchronize()
    _linear_check(x, w, qx, sx, qw, sw)


@pytest.mark.parametrize("part", ["up", "down"])
def test_quant_linear_qwen3_4b_full(part):
    """The MLP step's operand pairs at full size: X_up [4096 x 2560] with
    W_up [9728 x 2560], X_down [4096 x 9728] with W_down [2560 x 9728]."""
    d = inputs.qwen3_4b_mlp(1, parts=(part,))
    x, w = d["x_" + part], d["w_" + part]
    _say("quant_linear full", part, x.shape, w.shape)
    qx, sx, qw, sw = ops.quant_linear(dev_bf16(x), dev_bf16(w))
    torch.cuda.synchronize()
    _linear_check(x, w, qx, sx, qw, sw)


def test_quant_linear_layouts_and_empty_operands():
    """Row-major activation scales, and one operand empty: the results equal
    the separate fp8_quant_rowblock / fp8_quant_block2d calls byte for byte."""
    rows, w_rows, cols = 260, 384, 640
    x = dev_bf16(_bits((rows, cols), 44))
    w = dev_bf16(_bits((w_rows, cols), 45, 0.02, 0.0, 1.0))
    ng = cols // 128
    u8 = lambda *sh: torch.full(sh, 0xAA, dtype=torch.uint8, device="cuda")
    f32 = lambda *sh: torch.full(sh, -1.0, dtype=torch.float32, device="cuda")
    # reference: the two separate calls, row-major activation scales
    qx0, sx0, qw0, sw0 = u8(rows, cols), f32(rows, ng), u8(w_rows, cols), f32(w_rows // 128, ng)
    ops.fp8_quant_rowblock(x, rows, cols, cols, ops.AXIS_ROW, qx0, cols, sx0, ng, 1)
    ops.fp8_quant_block2d(w, 1, w_rows, cols, cols, qw0, cols, None, 0, sw0)
    for rx, rw in ((rows, w_rows), (0, w_rows), (rows, 0)):
        qx, sx, qw, sw = u8(rows, cols), f32(rows, ng), u8(w_rows, cols), f32(w_rows // 128, ng)
        ops.fp8_quant_linear(x, rx, cols, cols, qx, cols, sx, ng, 1, w, rw, cols, qw, cols, sw)
        torch.cuda.synchronize()
        _say("quant_linear rows", rx, "w_rows", rw)
        if rx:
            assert torch.equal(qx, qx0) and torch.equal(sx.view(torch.int32), sx0.view(torch.int32))
        else:   # untouched
            assert bool((qx == 0xAA).all()) and bool((sx == -1.0).all())
        if rw:
            assert torch.equal(qw, qw0) and torch.equal(sw.view(torch.int32), sw0.view(torch.int32))
        else:
            assert bool((qw == 0xAA).all()) and bool((sw == -1.0).all())


# ---------------------------------------------------------------------- MX
@pytest.mark.parametrize("shape", [(64, 256), (5, 96), (300, 2048)])
def test_mx_small(shape):
    _say("mx", shape)
    x = _bits(shape, 6, 1.0, 0.02, 40.0)
    x[0, :32] = 0
    if shape[0] > 2:
        x[1, 32:64] = inputs.to_bf16_bits(np.full(32, 448.0, np.float32))
        x[2, :32] = inputs.to_bf16_bits(np.linspace(-3e-39, 3e-39, 32).astype(np.float32))
    q, s = ops.mx_quant(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.mx_quant_1x32(x)
    _assert_same_codes(q, qr)
    assert np.array_equal(host(s), sr)


def test_mx_moe_activation_full():
    x = inputs.qwen3_30b_a3b_moe(3, weights=False)["x"]
    _say("mx full", x.shape)
    q, s = ops.mx_quant(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.mx_quant_1x32(x)
    _assert_same_codes(q, qr)
    assert np.array_equal(host(s), sr)


def _silu_pairs(g_bits, u_bits):
    """gate|up matrix [rows][256] holding every (g, u) pair of the two bf16
    bit arrays, gate-major, zero-padded to whole rows of 128."""
    n = g_bits.size * u_bits.size
    I = 128
    rows = (n + I - 1) // I
    gate = np.zeros(rows * I, np.uint16)
    up = np.zeros(rows * I, np.uint16)
    gate[:n] = np.tile(g_bits, u_bits.size)
    up[:n] = np.repeat(u_bits, g_bits.size)
    return np.concatenate([gate.reshape(rows, I), up.reshape(rows, I)], axis=1), n


def _silu_device(gu):
    rows, I = gu.shape[0], gu.shape[1] // 2
    q = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    s_ = torch.empty((rows, 1), dtype=torch.float32, device="cuda")
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    ops.fp8_silu_mul_quant(dev_bf16(gu), rows, I, 2 * I, 0, q, I, s_, 1, 1, h, I)
    torch.cuda.synchronize()
    return host(h)


def test_silu_mul_every_bf16_gate_value():
    """h = bf16(silu(g) * u) bit-exact against the oracle's fp64 evaluation for
    every finite bf16 g, with u values that make exact bf16 midpoints common:
    u = 1 + 2^-7 turns g * u into a midpoint whenever g's significand ends in
    a 1 bit, and for large g (sigmoid 1 in fp64) or tiny g (sigmoid 1/2) the
    oracle then rounds the midpoint itself to even."""
    g = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    g = g[np.isfinite((g.astype(np.uint32) << 16).view(np.float32))]
    us = np.array([1.0, -1.0, 1.0078125, -1.0078125, 3.0234375, -3.5, 0.0078125, 1000.0, -2.0 ** -20,
                   2.0 ** 100, 1.5 * 2.0 ** -120, 3.0e38], np.float64)
    gu, n = _silu_pairs(g, oracle.f64_to_bf16(us))
    hg = _silu_device(gu).reshape(-1)[:n]
    hr = oracle.silu_mul(gu).reshape(-1)[:n]
    bad = np.flatnonzero(hg != hr)
    _say("silu h, %d gate values x %d up values: %d mismatches" % (g.size, us.size, bad.size))
    assert bad.size == 0, "h differs from the oracle at g=%s u=%s" % (gu[:, :128].reshape(-1)[bad[:5]],
                                                                     gu[:, 128:].reshape(-1)[bad[:5]])


def test_silu_mul_random_pairs():
    """Bit-exact h on 2^22 random finite (g, u) bf16 pairs drawn over the whole
    exponent range and on 2^20 pairs at GEMM-output magnitudes."""
    rng = np.random.default_rng(11)
    def finite_bits(count):
        b = rng.integers(0, 1 << 16, count * 2).astype(np.uint16)
        b = b[np.isfinite((b.astype(np.uint32) << 16).view(np.float32))]
        return b[:count]
    gb, ub = finite_bits(2048), finite_bits(2048)
    gu, n = _silu_pairs(gb, ub)
    assert np.array_equal(_silu_device(gu).reshape(-1)[:n], oracle.silu_mul(gu).reshape(-1)[:n])
    gn = oracle.f64_to_bf16(rng.standard_normal(1024) * 4.0)
    un = oracle.f64_to_bf16(rng.standard_normal(1024) * 2.0)
    gu, n = _silu_pairs(gn, un)
    assert np.array_equal(_silu_device(gu).reshape(-1)[:n], oracle.silu_mul(gu).reshape(-1)[:n])


# ------------------------------------------------------------ SiLU * up
@pytest.mark.parametrize("mx", [0, 1])
def test_silu_mul_quant(mx):
    rows, I = 1000, 768
    gu = _bits((rows, 2 * I), 7, 2.0, 0.0, 1.0)
    d = dev_bf16(gu)
    q = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    h = torch.empty((rows, I), dtype=torch.bfloat16, device="cuda")
    if mx:
        s = torch.empty((rows, I // 32), dtype=torch.uint8, device="cuda")
        ops.fp8_silu_mul_quant(d, rows, I, 2 * I, 1, q, I, s, I // 32, 1, h, I)
    else:
        s = torch.empty((rows, I // 128), dtype=torch.float32, device="cuda")
        ops.fp8_silu_mul_quant(d, rows, I, 2 * I, 0, q, I, s, I // 128, 1, h, I)
    torch.cuda.synchronize()
    hg = host(h)
    hr = oracle.silu_mul(gu)
    assert np.array_equal(hg, hr), "h differs from the oracle at %s" % (np.argwhere(hg != hr)[:5],)
    # codes and scales against the oracle's quantization of the oracle's h
    if mx:
        qr, sr = oracle.mx_quant_1x32(hr)
        _assert_same_codes(q, qr)
        assert np.array_equal(host(s), sr)
    else:
        qr, sr = oracle.quant_1x128(hr)
        _assert_same_codes(q, qr)
        _assert_same_scales(s, sr)
