"""Caller views with padded leading dimensions and non-default scale strides,
through every quantizer and GEMM entry point of the C ABI.  The logical
region must match the oracle bit for bit, nothing outside it may be read
(padding of the inputs holds NaN patterns, which would poison a group's
maximum or a dot product) and nothing outside it may be written (padding of
the outputs holds sentinel bytes that must survive).  The quantization rule
is that of "Unified FP8: Beyond Mixed Precision...", section "FP8
Quantization", with the groupings of "Low Precision RL", table "Choose a
precision"; the GEMM operands are small integers with power-of-two scales,
so every sum is exact and the oracle's fp64 result is the bit pattern to
match."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC1       # a quiet NaN bf16 pattern in every unread input element
NAN_E4M3 = 0x7F         # the E4M3FN NaN code in every unread operand byte
SENT_U8 = 0xA5          # output bytes outside the logical region
SENT_F32 = -1234.5      # scale cells outside the logical layout


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, 1.0, 0.01, 50.0)


def _padded(a, ld, fill):
    """Device [rows + 1][ld] buffer (one guard row) holding `a` in
    [:rows, :cols] and `fill` everywhere else; returns (buffer, view)."""
    rows, cols = a.shape
    buf = np.full((rows + 1, ld), fill, a.dtype)
    buf[:rows, :cols] = a
    t = dev(buf.view(np.int16) if buf.dtype == np.uint16 else buf)
    return t, t[:rows]


def _out_u8(rows, ld):
    return torch.full((rows + 1, ld), SENT_U8, dtype=torch.uint8, device="cuda")


def _out_f32(n):
    return torch.full((n,), SENT_F32, dtype=torch.float32, device="cuda")


def _check_u8(buf, rows, cols, ref):
    b = host(buf)
    assert np.array_equal(b[:rows, :cols], ref), "codes differ from the oracle"
    assert np.all(b[:rows, cols:] == SENT_U8), "written past the row length"
    assert np.all(b[rows:] == SENT_U8), "written past the last row"


def _check_scales(buf, idx, ref):
    """Scale cells at flat indices `idx` (same shape as ref) equal ref bit
    for bit; every other cell keeps the sentinel."""
    b = host(buf).reshape(-1)
    got = b[idx]
    assert np.array_equal(got.view(np.uint32), np.ascontiguousarray(ref, np.float32).view(np.uint32)), \
        "scales differ from the oracle"
    rest = np.ones(b.size, bool)
    rest[idx.reshape(-1)] = False
    assert np.all(b[rest] == np.float32(SENT_F32)), "a scale cell outside the layout was written"


def _grid(rows, groups, s_row, s_group):
    r, g = np.meshgrid(np.arange(rows), np.arange(groups), indexing="ij")
    return r * s_row + g * s_group


# ------------------------------------------------------------- quantizers
@pytest.mark.parametrize("layout", ["row_major_padded", "m_major_padded"])
def test_rowblock_row_axis_padded(layout):
    rows, cols, ld_x, ld_q = 300, 520, 536, 544
    groups = (cols + 127) // 128
    x = _bits((rows, cols), 11)
    _, xv = _padded(x, ld_x, NAN_BF16)
    q = _out_u8(rows, ld_q)
    s_row, s_group = (8, 1) if layout == "row_major_padded" else (1, rows + 16)
    s = _out_f32((rows - 1) * s_row + (groups - 1) * s_group + 1 + 24)
    _say("rowblock row axis", layout)
    ops.fp8_quant_rowblock(xv, rows, cols, ld_x, ops.AXIS_ROW, q, ld_q, s, s_row, s_group)
    qr, sr = oracle.quant_1x128(x)
    _check_u8(q, rows, cols, qr)
    _check_scales(s, _grid(rows, groups, s_row, s_group), sr)


def test_rowblock_col_axis_padded():
    rows, cols, ld_x, ld_q = 272, 200, 216, 288
    groups = (rows + 127) // 128
    x = _bits((rows, cols), 12)
    _, xv = _padded(x, ld_x, NAN_BF16)
    qt = _out_u8(cols, ld_q)
    s_row, s_group = 4, 1
    s = _out_f32((cols - 1) * s_row + (groups - 1) * s_group + 1 + 24)
    _say("rowblock col axis")
    ops.fp8_quant_rowblock(xv, rows, cols, ld_x, ops.AXIS_COL, qt, ld_q, s, s_row, s_group)
    qr, sr = oracle.quant_128x1_t(x)
    _check_u8(qt, cols, rows, qr)
    _check_scales(s, _grid(cols, groups, s_row, s_group), sr)


def test_block2d_batched_padded_with_transpose():
    batch, rows, cols, ld_w, ld_q, ld_qt = 2, 208, 264, 280, 288, 224
    nbr, nbc = (rows + 127) // 128, (cols + 127) // 128
    ws = [_bits((rows, cols), 13 + b) for b in range(batch)]
    buf = np.full((batch * rows + 1, ld_w), NAN_BF16, np.uint16)
    for b in range(batch):
        buf[b * rows:(b + 1) * rows, :cols] = ws[b]
    w = dev(buf.view(np.int16))
    q = _out_u8(batch * rows, ld_q)
    qt = _out_u8(batch * cols, ld_qt)
    s = _out_f32(batch * nbr * nbc + 16)
    _say("block2d batched padded")
    ops.fp8_quant_block2d(w, batch, rows, cols, ld_w, q, ld_q, qt, ld_qt, s)
    hq, hqt, hs = host(q), host(qt), host(s)
    for b in range(batch):
        qr, sr = oracle.quant_128x128(ws[b])
        assert np.array_equal(hq[b * rows:(b + 1) * rows, :cols], qr)
        assert np.array_equal(hqt[b * cols:(b + 1) * cols, :rows], qr.T)
        assert np.array_equal(hs[b * nbr * nbc:(b + 1) * nbr * nbc].view(np.uint32), sr.reshape(-1).view(np.uint32))
    assert np.all(hq[:, cols:] == SENT_U8) and np.all(hq[batch * rows:] == SENT_U8)
    assert np.all(hqt[:, rows:] == SENT_U8) and np.all(hqt[batch * cols:] == SENT_U8)
    assert np.all(hs[batch * nbr * nbc:] == np.float32(SENT_F32))


def test_quant_linear_padded():
    rows, cols, w_rows, ld_x, ld_qx, ld_w, ld_qw = 130, 384, 200, 400, 416, 392, 400
    groups, nbr = cols // 128, (w_rows + 127) // 128
    x, w = _bits((rows, cols), 15), _bits((w_rows, cols), 16)
    _, xv = _padded(x, ld_x, NAN_BF16)
    _, wv = _padded(w, ld_w, NAN_BF16)
    qx, qw = _out_u8(rows, ld_qx), _out_u8(w_rows, ld_qw)
    s_row, s_group = 1, rows + 14
    sx = _out_f32((rows - 1) * s_row + (groups - 1) * s_group + 1 + 8)
    sw = _out_f32(nbr * groups + 8)
    _say("quant_linear padded")
    ops.fp8_quant_linear(xv, rows, cols, ld_x, qx, ld_qx, sx, s_row, s_group, wv, w_rows, ld_w, qw, ld_qw, sw)
    qxr, sxr = oracle.quant_1x128(x)
    qwr, swr = oracle.quant_128x128(w)
    _check_u8(qx, rows, cols, qxr)
    _check_u8(qw, w_rows, cols, qwr)
    _check_scales(sx, _grid(rows, groups, s_row, s_group), sxr)
    _check_scales(sw, np.arange(nbr * groups).reshape(nbr, groups), swr)


@pytest.mark.parametrize("kind", ["rowwise", "tensorwise"])
def test_rowwise_tensorwise_padded(kind):
    rows, cols, ld_x, ld_q = 100, 256, 272, 288
    x = _bits((rows, cols), 17)
    _, xv = _padded(x, ld_x, NAN_BF16)
    q = _out_u8(rows, ld_q)
    n = rows if kind == "rowwise" else 1
    s = _out_f32(n + 8)
    _say(kind, "padded")
    if kind == "rowwise":
        ops.fp8_quant_rowwise(xv, rows, cols, ld_x, q, ld_q, s)
        qr, sr = oracle.quant_rowwise(x)
    else:
        ops.fp8_quant_tensorwise(xv, rows, cols, ld_x, q, ld_q, s)
        qr, sr = oracle.quant_tensorwise(x)
    _check_u8(q, rows, cols, qr)
    _check_scales(s, np.arange(n), sr)


def _check_bytes(buf, idx, ref):
    b = host(buf).reshape(-1)
    assert np.array_equal(b[idx], np.asarray(ref, np.uint8)), "scale bytes differ from the oracle"
    rest = np.ones(b.size, bool)
    rest[idx.reshape(-1)] = False
    assert np.all(b[rest] == SENT_U8), "a scale byte outside the layout was written"


def test_mx_quant_padded():
    rows, cols, ld_x, ld_q = 64, 160, 176, 176
    groups = cols // 32
    x = _bits((rows, cols), 18)
    _, xv = _padded(x, ld_x, NAN_BF16)
    q = _out_u8(rows, ld_q)
    s_row, s_group = 8, 1
    s = torch.full(((rows - 1) * s_row + groups + 16,), SENT_U8, dtype=torch.uint8, device="cuda")
    _say("mx quant padded")
    ops.mxfp8_quant(xv, rows, cols, ld_x, q, ld_q, s, s_row, s_group)
    qr, sr = oracle.mx_quant_1x32(x)
    _check_u8(q, rows, cols, qr)
    _check_bytes(s, _grid(rows, groups, s_row, s_group), sr)


def test_mx_quant_t_padded():
    rows, cols, ld_x, ld_qt = 96, 72, 88, 112
    groups = rows // 32
    x = _bits((rows, cols), 19)
    _, xv = _padded(x, ld_x, NAN_BF16)
    qt = _out_u8(cols, ld_qt)
    s_row, s_group = 4, 1
    s = torch.full(((cols - 1) * s_row + groups + 16,), SENT_U8, dtype=torch.uint8, device="cuda")
    _say("mx quant_t padded")
    ops.mxfp8_quant_t(xv, rows, cols, ld_x, qt, ld_qt, s, s_row, s_group)
    qr, sr = oracle.mx_quant_32x1_t(x)
    _check_u8(qt, cols, rows, qr)
    _check_bytes(s, _grid(cols, groups, s_row, s_group), sr)


@pytest.mark.parametrize("block_rows", [1, 128])
def test_pow2_quant_padded(block_rows):
    rows, cols, ld_x, ld_q, ld_s = 130, 256, 264, 272, 8
    groups, ngr = cols // 128, (rows + block_rows - 1) // block_rows
    x = _bits((rows, cols), 20)
    _, xv = _padded(x, ld_x, NAN_BF16)
    q = _out_u8(rows, ld_q)
    s = torch.full((ngr * ld_s + 16,), SENT_U8, dtype=torch.uint8, device="cuda")
    _say("pow2 quant padded", block_rows)
    ops.fp8_quant_pow2(xv, rows, cols, ld_x, block_rows, q, ld_q, s, ld_s)
    qr, sr = oracle.quant_1x128_pow2(x) if block_rows == 1 else oracle.quant_128x128_pow2(x)
    _check_u8(q, rows, cols, qr)
    _check_bytes(s, _grid(ngr, groups, ld_s, 1), sr)


@pytest.mark.parametrize("mx", [0, 1])
def test_silu_mul_quant_padded(mx):
    rows, I, ld_q, ld_h = 50, 256, 272, 264
    ld_in = 2 * I + 24
    groups = I // (32 if mx else 128)
    gu = _bits((rows, 2 * I), 21)
    _, guv = _padded(gu, ld_in, NAN_BF16)
    q = _out_u8(rows, ld_q)
    h = torch.full((rows + 1, ld_h), 0x5A5A, dtype=torch.int16, device="cuda")
    s_row, s_group = 1, rows + 6
    n = (rows - 1) * s_row + (groups - 1) * s_group + 1 + 8
    s = _out_f32(n) if not mx else torch.full((n,), SENT_U8, dtype=torch.uint8, device="cuda")
    _say("silu_mul_quant padded, mx", mx)
    ops.fp8_silu_mul_quant(guv, rows, I, ld_in, mx, q, ld_q, s, s_row, s_group, h, ld_h)
    hr = oracle.silu_mul(gu)
    hh = host(h).view(np.uint16)
    assert np.array_equal(hh[:rows, :I], hr)
    assert np.all(hh[:rows, I:] == 0x5A5A) and np.all(hh[rows:] == 0x5A5A)
    qr, sr = oracle.mx_quant_1x32(hr) if mx else oracle.quant_1x128(hr)
    _check_u8(q, rows, I, qr)
    idx = _grid(rows, groups, s_row, s_group)
    if mx:
        _check_bytes(s, idx, sr)
    else:
        _check_scales(s, idx, sr)


# ------------------------------------------------------------------ GEMMs
def _ints(shape, rng):
    return oracle.e4m3_encode(rng.integers(-8, 9, size=shape).astype(np.float32))


def _check_c(c, rows, N, yref, out):
    b = host(c)
    if out == ops.OUT_FP32:
        assert np.array_equal(b[:rows, :N].astype(np.float64), yref)
        sent = np.float32(SENT_F32).view(np.uint32)
        assert np.all(b[:rows, N:].view(np.uint32) == sent) and np.all(b[rows:].view(np.uint32) == sent)
    else:
        bits = b.view(np.uint16)
        assert np.array_equal(bits[:rows, :N], oracle.f64_to_bf16(yref))
        assert np.all(bits[:rows, N:] == 0x5A5A) and np.all(bits[rows:] == 0x5A5A)


def _out_c(rows, ldc, out):
    if out == ops.OUT_FP32:
        return torch.full((rows + 1, ldc), SENT_F32, dtype=torch.float32, device="cuda")
    return torch.full((rows + 1, ldc), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)


@pytest.mark.parametrize("out", [ops.OUT_BF16, ops.OUT_FP32])
@pytest.mark.parametrize("mode", ["block128", "row128", "k_invariant"])
def test_gemm_padded_strides(mode, out):
    """lda, ldb, ldc above the row lengths, activation scales K-major with a
    padded row (the transpose of the default M-major layout), weight scales
    with a padded stride; NaN codes in every operand byte past K."""
    M, N, K, lda, ldb, ldc = 200, 384, 512, 528, 544, 400
    nkb = K // 128
    rng = np.random.default_rng(22)
    qa, qb = _ints((M, K), rng), _ints((N, K), rng)
    _, av = _padded(qa, lda, NAN_E4M3)
    _, bv = _padded(qb, ldb, NAN_E4M3)
    if mode == "k_invariant":
        sa_l = np.exp2(rng.integers(-1, 2, size=M)).astype(np.float32)
        sb_l = np.exp2(rng.integers(-1, 2, size=N)).astype(np.float32)
        sa_m, sa_k, sb_n, sb_k, bscale = 3, 0, 2, 0, ops.BSCALE_ROW128
        sa_buf = np.full(M * sa_m + 4, np.nan, np.float32); sa_buf[np.arange(M) * sa_m] = sa_l
        sb_buf = np.full(N * sb_n + 4, np.nan, np.float32); sb_buf[np.arange(N) * sb_n] = sb_l
        yref, _ = oracle.gemm_rowscaled(qa, sa_l, qb, sb_l, with_abs=False)
    else:
        nb = N // 128 if mode == "block128" else N
        sa_l = np.exp2(rng.integers(-1, 2, size=(M, nkb))).astype(np.float32)
        sb_l = np.exp2(rng.integers(-1, 2, size=(nb, nkb))).astype(np.float32)
        sa_m, sa_k = nkb + 3, 1                            # K-major rows, padded
        sb_n, sb_k = (1, nb + 2) if mode == "block128" else (nkb + 1, 1)
        sa_buf = np.full(M * sa_m + 4, np.nan, np.float32)
        sa_buf[_grid(M, nkb, sa_m, sa_k)] = sa_l
        sb_buf = np.full(max(nb * sb_n, nkb * sb_k) + nb + 4, np.nan, np.float32)
        sb_buf[_grid(nb, nkb, sb_n, sb_k)] = sb_l
        bscale = ops.BSCALE_BLOCK128 if mode == "block128" else ops.BSCALE_ROW128
        yref, _ = oracle.gemm_blockscaled(qa, sa_l, qb, sb_l, oracle.BSCALE_BLOCK128 if mode == "block128"
                                          else oracle.BSCALE_ROW128, with_abs=False)
    c = _out_c(M, ldc, out)
    _say("gemm padded", mode, out)
    ops.fp8_blockscaled_gemm(M, N, K, av, lda, dev(sa_buf), sa_m, sa_k, bv, ldb, dev(sb_buf), sb_n, sb_k, bscale,
                             c, ldc, out)
    _check_c(c, M, N, yref, out)


@pytest.mark.parametrize("out", [ops.OUT_BF16, ops.OUT_FP32])
def test_pow2_gemm_padded(out):
    M, N, K, lda, ldb, ldc, lds_a, lds_b = 130, 256, 1024, 1040, 1056, 272, 12, 8
    nkb = K // 128
    rng = np.random.default_rng(23)
    qa, qb = _ints((M, K), rng), _ints((N, K), rng)
    _, av = _padded(qa, lda, NAN_E4M3)
    _, bv = _padded(qb, ldb, NAN_E4M3)
    ea = rng.integers(126, 129, size=(M, nkb)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(N // 128, nkb)).astype(np.uint8)
    _, sav = _padded(ea, lds_a, 0xFF)          # 0xFF is the UE8M0 NaN byte
    _, sbv = _padded(eb, lds_b, 0xFF)
    yref, _ = oracle.gemm_blockscaled(qa, oracle.pow2_scales(ea), qb, oracle.pow2_scales(eb), with_abs=False)
    c = _out_c(M, ldc, out)
    _say("pow2 gemm padded", out)
    ops.fp8_blockscaled_gemm_pow2(M, N, K, av, lda, sav, lds_a, bv, ldb, sbv, lds_b, c, ldc, out)
    _check_c(c, M, N, yref, out)


@pytest.mark.parametrize("out", [ops.OUT_BF16, ops.OUT_FP32])
def test_mx_gemm_dense_padded(out):
    M, N, K, lda, ldb, ldc, lds_a, lds_b = 130, 256, 512, 528, 544, 272, 20, 24
    rng = np.random.default_rng(24)
    qa, qb = _ints((M, K), rng), _ints((N, K), rng)
    _, av = _padded(qa, lda, NAN_E4M3)
    _, bv = _padded(qb, ldb, NAN_E4M3)
    ea = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    _, sav = _padded(ea, lds_a, 0xFF)
    _, sbv = _padded(eb, lds_b, 0xFF)
    yref, _ = oracle.gemm_mx(qa, ea, qb, eb)
    c = _out_c(M, ldc, out)
    _say("mx gemm padded", out)
    ops.mxfp8_gemm(M, N, K, 0, None, None, M, av, lda, sav, lds_a, bv, ldb, 0, sbv, lds_b, 0, c, ldc, out)
    _check_c(c, M, N, yref, out)


@pytest.mark.parametrize("out", [ops.OUT_BF16, ops.OUT_FP32])
def test_grouped_gemm_padded(out):
    """Expert weights with a padded expert stride and row length, scales with
    padded strides along experts, blocks and slices; three experts, one
    empty."""
    N, K, lda, ldb, ldc = 256, 384, 400, 416, 272
    nkb, nb = K // 128, N // 128
    offsets = np.array([0, 100, 100, 300], np.int32)
    G, rows = 3, 300
    rng = np.random.default_rng(25)
    qa = _ints((rows, K), rng)
    qbs = np.stack([_ints((N, K), rng) for _ in range(G)])
    _, av = _padded(qa, lda, NAN_E4M3)
    b_stride_g = (N + 2) * ldb
    bbuf = np.full((G * (N + 2) + 1, ldb), NAN_E4M3, np.uint8)
    for g in range(G):
        bbuf[g * (N + 2):g * (N + 2) + N, :K] = qbs[g]
    sa_l = np.exp2(rng.integers(-1, 2, size=(rows, nkb))).astype(np.float32)
    sb_l = np.exp2(rng.integers(-1, 2, size=(G, nb, nkb))).astype(np.float32)
    sa_m, sa_k = 1, rows + 5                            # M-major, padded
    sb_g, sb_n, sb_k = nb * nkb + 7, 1, nb + 1           # per expert: [kb][nb], padded
    sa_buf = np.full(sa_k * nkb + 8, np.nan, np.float32)
    sa_buf[_grid(rows, nkb, sa_m, sa_k)] = sa_l
    sb_buf = np.full(G * sb_g + 8, np.nan, np.float32)
    for g in range(G):
        sb_buf[g * sb_g + _grid(nb, nkb, sb_n, sb_k)] = sb_l[g]
    yref, _ = oracle.grouped_gemm_blockscaled(qa, sa_l, offsets, qbs, sb_l)
    c = _out_c(rows, ldc, out)
    _say("grouped gemm padded", out)
    ops.fp8_grouped_gemm(rows, N, K, G, dev(offsets), None, rows, av, lda, dev(sa_buf), sa_m, sa_k, dev(bbuf), ldb,
                         b_stride_g, dev(sb_buf), sb_g, sb_n, sb_k, c, ldc, out)
    _check_c(c, rows, N, yref, out)


@pytest.mark.parametrize("out", [ops.OUT_BF16, ops.OUT_FP32])
def test_moe_combine_padded(out):
    """Grouped rows and output with padded leading dimensions; integer rows
    and power-of-two weights, so the fp32 sum is exact."""
    rows, H, ld_y, T, k, ld_out = 96, 136, 152, 40, 3, 144
    rng = np.random.default_rng(26)
    yv = rng.integers(-64, 65, size=(rows, H)).astype(np.float64)
    y = oracle.f64_to_bf16(yv)
    _, ydv = _padded(y, ld_y, NAN_BF16)
    pos = rng.integers(0, rows, size=(T, k)).astype(np.int32)
    w = np.exp2(rng.integers(-3, 1, size=(T, k))).astype(np.float32)
    ref = oracle.moe_combine(y, pos, w)
    o = _out_c(T, ld_out, out)
    _say("combine padded", out)
    ops.fp8_moe_combine(ydv, rows, H, ld_y, dev(pos), dev(w), T, k, o, ld_out, out)
    _check_c(o, T, H, ref, out)


@pytest.mark.parametrize("mx", [0, 1])
def test_fused_gate_up_padded_gather(mx):
    """The gate/up GEMM with SiLU*mul and the quantization of h in its
    epilogue (FP32 1x128 scales, or UE8M0 1x32), reading its activation rows
    through the dispatch gather from a padded buffer, expert weights with
    padded rows and expert stride, and writing h codes and scales through
    padded layouts.  Against the oracle chain: the exact grouped GEMM,
    rounded to bf16, SiLU*mul, then the quantization of h."""
    T, K, I, G = 120, 256, 128, 3
    N2, lda, ldb, ld_hq = 2 * I, 272, 288, 144
    offsets = np.array([0, 90, 90, 200], np.int32)
    rows = int(offsets[-1])
    rng = np.random.default_rng(27 + mx)
    a_rows = rng.integers(0, T, size=rows).astype(np.int32)
    qx = _ints((T, K), rng)
    qgu = np.stack([_ints((N2, K), rng) for _ in range(G)])
    _, av = _padded(qx, lda, NAN_E4M3)
    b_stride_g = (N2 + 1) * ldb
    bbuf = np.full((G * (N2 + 1) + 1, ldb), NAN_E4M3, np.uint8)
    for g in range(G):
        bbuf[g * (N2 + 1):g * (N2 + 1) + N2, :K] = qgu[g]
    qa_g = qx[a_rows]
    y = np.zeros((rows, N2))
    if mx:
        lds_a, lds_b = K // 32 + 4, K // 32 + 8
        ea = rng.integers(126, 129, size=(T, K // 32)).astype(np.uint8)
        eb = rng.integers(126, 129, size=(G, N2, K // 32)).astype(np.uint8)
        _, sav = _padded(ea, lds_a, 0xFF)
        sb_g = N2 * lds_b + 16
        sbuf = np.full(G * sb_g + 16, 0xFF, np.uint8)
        for g in range(G):
            sbuf[g * sb_g + _grid(N2, K // 32, lds_b, 1)] = eb[g]
        for g in range(G):
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            if r1 > r0:
                y[r0:r1], _ = oracle.gemm_mx(qa_g[r0:r1], ea[a_rows[r0:r1]], qgu[g], eb[g])
    else:
        nkb, nb = K // 128, N2 // 128
        sx = np.exp2(rng.integers(-1, 2, size=(T, nkb))).astype(np.float32)
        sgu = np.exp2(rng.integers(-1, 2, size=(G, nb, nkb))).astype(np.float32)
        sa_m, sa_k = nkb + 2, 1                                  # K-major, padded
        sb_g, sb_n, sb_k = nb * nkb + 5, nkb + 1, 1
        sa_buf = np.full(T * sa_m + 4, np.nan, np.float32)
        sa_buf[_grid(T, nkb, sa_m, sa_k)] = sx
        sb_buf = np.full(G * sb_g + 4, np.nan, np.float32)
        for g in range(G):
            sb_buf[g * sb_g + _grid(nb, nkb, sb_n, sb_k)] = sgu[g]
        y, _ = oracle.grouped_gemm_blockscaled(qa_g, sx[a_rows], offsets, qgu, sgu)
    h = oracle.silu_mul(oracle.f64_to_bf16(y))
    qr, sr = oracle.mx_quant_1x32(h) if mx else oracle.quant_1x128(h)
    groups = I // (32 if mx else 128)
    hq = _out_u8(rows, ld_hq)
    hs_row, hs_group = (groups + 3, 1) if mx else (1, rows + 9)
    n = (rows - 1) * hs_row + (groups - 1) * hs_group + 1 + 8
    hs = torch.full((n,), SENT_U8, dtype=torch.uint8, device="cuda") if mx else _out_f32(n)
    _say("fused gate_up padded gather, mx", mx)
    if mx:
        ops.mxfp8_grouped_gemm_swiglu_quant(rows, I, K, G, dev(offsets), dev(a_rows), T, av, lda, sav, lds_a,
                                            dev(bbuf), ldb, b_stride_g, dev(sbuf), lds_b, sb_g, hq, ld_hq, hs,
                                            hs_row, hs_group)
    else:
        ops.fp8_grouped_gemm_swiglu_quant(rows, I, K, G, dev(offsets), dev(a_rows), T, av, lda, dev(sa_buf), sa_m,
                                          sa_k, dev(bbuf), ldb, b_stride_g, dev(sb_buf), sb_g, sb_n, sb_k, hq, ld_hq,
                                          hs, hs_row, hs_group)
    _check_u8(hq, rows, I, qr)
    idx = _grid(rows, groups, hs_row, hs_group)
    if mx:
        _check_bytes(hs, idx, sr)
    else:
        _check_scales(hs, idx, sr)
