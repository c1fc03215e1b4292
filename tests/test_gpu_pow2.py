"""GPU parity of the block-wise recipe with power-of-two (UE8M0) scales.

The 1x128 / 128x128 groups of "Low Precision RL", section "2. Unified
block-wise FP8 (DeepSeek-style)", with each group's scale rounded up to a
power of two (the MX exponent rule on the group's amax), the form
TransformerEngine uses when it runs that recipe through MXFP8 on Blackwell.
Quantizer codes and scale bytes must be bit-identical to the oracle's; the
GEMM, which applies the scales inside the scaled matrix instruction, is
checked against the fp64 oracle (the block-scaled definition with the decoded
scales) and against the datapath truncation model, and bit for bit on
operands whose sums are exact.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16, host, sample_indices, verify

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed, sigma=1.0, frac=0.01, mult=50.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def _same(q_gpu, s_gpu, qr, sr):
    qg = host(q_gpu)
    bad = np.flatnonzero(qg != qr)
    assert bad.size == 0, "%d code mismatches, first at %s" % (bad.size, bad[:5])
    sg = host(s_gpu)[:, :sr.shape[1]]
    assert np.array_equal(sg, sr), "scale byte mismatch at %s" % (np.argwhere(sg != sr)[:5],)


@pytest.mark.parametrize("shape", [(256, 512), (7, 264), (1, 8), (300, 1000), (4096, 2560)])
def test_quant_1x128_pow2(shape):
    _say("pow2 1x128", shape)
    x = _bits(shape, 70)
    if shape[0] >= 3 and shape[1] >= 128:
        x[0, :128] = 0
        x[1, :128] = inputs.to_bf16_bits(np.full(128, 448.0 * 2.0 ** -3, np.float32))
        x[2, :128] = inputs.to_bf16_bits(np.linspace(-3e38, 3e38, 128).astype(np.float32))
    q, s = ops.quant_pow2(dev_bf16(x), 1)
    torch.cuda.synchronize()
    _same(q, s, *oracle.quant_1x128_pow2(x))


@pytest.mark.parametrize("rows,w_rows,cols", [(4096, 9728, 2560), (300, 200, 1000), (7, 130, 264), (0, 256, 512),
                                             (256, 0, 512)])
def test_quant_linear_pow2(rows, w_rows, cols):
    """Both operands in one launch with power-of-two scales: codes and scale
    bytes of X (1x128) and W (128x128) equal to the oracle's, with padded
    scale rows (ld 4 * ceil(cols / 512), as the GEMM wants them); an empty
    operand's buffers are left alone."""
    _say("pow2 operand pair", rows, w_rows, cols)
    x, w = _bits((max(rows, 1), cols), 72), _bits((max(w_rows, 1), cols), 73, 0.02)
    g = (cols + 127) // 128
    lds = 4 * ((cols + 511) // 512)
    SENT = 0xA5
    qx = torch.full((max(rows, 1), cols), SENT, dtype=torch.uint8, device="cuda")
    sx = torch.full((max(rows, 1), lds), SENT, dtype=torch.uint8, device="cuda")
    qw = torch.full((max(w_rows, 1), cols), SENT, dtype=torch.uint8, device="cuda")
    sw = torch.full(((max(w_rows, 1) + 127) // 128, lds), SENT, dtype=torch.uint8, device="cuda")
    ops.fp8_quant_linear_pow2(dev_bf16(x), rows, cols, cols, qx, cols, sx, lds, dev_bf16(w), w_rows, cols, qw, cols,
                              sw, lds)
    torch.cuda.synchronize()
    if rows:
        _same(qx, sx, *oracle.quant_1x128_pow2(x))
        assert torch.all(sx[:, g:] == SENT)
    else:
        assert torch.all(qx == SENT) and torch.all(sx == SENT)
    if w_rows:
        _same(qw, sw, *oracle.quant_128x128_pow2(w))
        assert torch.all(sw[:, g:] == SENT)
    else:
        assert torch.all(qw == SENT) and torch.all(sw == SENT)


@pytest.mark.parametrize("shape", [(512, 512), (200, 264), (9728, 2560)])
def test_quant_128x128_pow2(shape):
    _say("pow2 128x128", shape)
    x = _bits(shape, 71, 0.02)
    x[:128, :128] = 0
    q, s = ops.quant_pow2(dev_bf16(x), 128)
    torch.cuda.synchronize()
    _same(q, s, *oracle.quant_128x128_pow2(x))


def _operands(M, N, K, seed):
    x = _bits((M, K), seed, 1.0, 0.001, 100.0)
    w = _bits((N, K), seed + 1, 0.02, 0.0, 1.0)
    qa, sa = ops.quant_pow2(dev_bf16(x), 1)
    qb, sb = ops.quant_pow2(dev_bf16(w), 128)
    return qa, sa, qb, sb


def _check(qa, sa, qb, sb, mi=None, ni=None):
    K = qa.shape[1]
    nk = K // 128
    y16 = ops.gemm_pow2(qa, sa, qb, sb, torch.bfloat16)
    y32 = ops.gemm_pow2(qa, sa, qb, sb, torch.float32)
    torch.cuda.synchronize()
    verify(host(qa), oracle.pow2_scales(host(sa)[:, :nk]), host(qb), oracle.pow2_scales(host(sb)[:, :nk]),
           host(y32), host(y16), mi=mi, ni=ni)


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (300, 384, 1024), (1, 128, 128), (513, 640, 384),
                                   (130, 128, 640)])
def test_gemm_pow2_small(M, N, K):
    """Every output; ragged M, K/128 not a multiple of 4, one-block N."""
    _say("pow2 gemm", M, N, K)
    _check(*_operands(M, N, K, M + N + K))


@pytest.mark.parametrize("M,N,K", [(4096, 9728, 2560), (4100, 9728, 384), (4096, 2560, 9728), (3200, 10112, 2048)])
def test_gemm_pow2_planned_tilings(M, N, K):
    """The MLP shapes, a ragged one and one the planner splits: its tilings
    (128-row weight tiles two per compute unit, 160-row tiles, and a 256 x 128
    region beside a 128 x 256 one); sampled outputs, tile corners and the
    columns around the region boundary."""
    split = ops.fp8_blockscaled_gemm_plan(M, N, K)[2]
    _say("pow2 gemm", M, N, K, "split", split)
    opnds = _operands(M, N, K, 9)
    mi, ni = sample_indices(M, N, 3000, 11)
    cols = np.arange(max(split - 40, 0), min(split + 40, N))
    mi = np.concatenate([mi, np.repeat(np.arange(0, M, 131), cols.size)])
    ni = np.concatenate([ni, np.tile(cols, (M + 130) // 131)])
    _check(*opnds, mi=mi, ni=ni)


@pytest.mark.parametrize("M,N,K", [(384, 640, 1024), (260, 2560, 640)])
def test_gemm_pow2_exact(M, N, K):
    """Small-integer codes and scale bytes 126..128 (slice factors 2^-2 ..
    2^2): every partial sum fits fp32's significand, so the result equals the
    oracle's bit for bit."""
    rng = np.random.default_rng(M + K)
    nk, lds = K // 128, 4 * ((K + 511) // 512)
    qa = oracle.e4m3_encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    qb = oracle.e4m3_encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    sa = np.zeros((M, lds), np.uint8)
    sb = np.zeros((N // 128, lds), np.uint8)
    sa[:, :nk] = rng.integers(126, 129, (M, nk))
    sb[:, :nk] = rng.integers(126, 129, (N // 128, nk))
    y = ops.gemm_pow2(dev(qa), dev(sa), dev(qb), dev(sb), torch.float32)
    torch.cuda.synchronize()
    yref, _ = oracle.gemm_blockscaled(qa, oracle.pow2_scales(sa[:, :nk]), qb, oracle.pow2_scales(sb[:, :nk]),
                                      with_abs=False)
    assert np.array_equal(host(y).astype(np.float64), yref)


def test_pow2_rejects_bad_layouts():
    qa = torch.zeros((128, 640), dtype=torch.uint8, device="cuda")
    qb = torch.zeros((128, 640), dtype=torch.uint8, device="cuda")
    c = torch.empty((128, 128), dtype=torch.float32, device="cuda")
    s_ok = torch.zeros((128, 8), dtype=torch.uint8, device="cuda")
    s_short = torch.zeros((128, 4), dtype=torch.uint8, device="cuda")
    ops.fp8_blockscaled_gemm_pow2(128, 128, 640, qa, 640, s_ok, 8, qb, 640, s_ok, 8, c, 128, ops.OUT_FP32)
    torch.cuda.synchronize()
    for args in ((s_short, 4), (s_ok, 6)):                # lds < 4 ceil(K/512), lds % 4
        with pytest.raises(ops.Fp8bsError):
            ops.fp8_blockscaled_gemm_pow2(128, 128, 640, qa, 640, args[0], args[1], qb, 640, s_ok, 8, c, 128,
                                          ops.OUT_FP32)
    x = dev_bf16(_bits((4, 256), 1))
    with pytest.raises(ops.Fp8bsError):
        ops.fp8_quant_pow2(x, 4, 256, 256, 64, qa, 256, s_ok, 8)      # block_rows must be 1 or 128
