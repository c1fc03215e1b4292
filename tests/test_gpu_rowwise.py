"""GPU parity of rowwise and tensorwise FP8 scaling against the CPU oracle.

Rowwise scaling keeps one FP32 scale per row, tensorwise one per tensor
("Towards Full Pipeline FP8 Reinforcement Learning for LLMs", its comparison
of tensorwise and rowwise scaling; "Unified FP8: Beyond Mixed Precision...",
section "FP8 Quantization", the per-tensor case).  The scale is amax / 448 and
the codes are round-to-nearest-even E4M3 of x / S, as for the block groups:
codes and scales must be bit-identical.  The GEMM on such operands is the
block-scaled GEMM whose per-slice scales repeat in every slice; the library
takes scale views of K stride 0 through a path that accumulates the whole
contraction in the matrix unit and applies sa(m) sb(n) once, so it is checked
like every other GEMM: against the fp64 oracle and against the datapath
truncation model.  Every call goes through the C ABI."""
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


def _same_codes(q_gpu, q_ref):
    a = host(q_gpu)
    bad = np.flatnonzero(a != q_ref)
    assert bad.size == 0, "%d code mismatches, first at %s: gpu %s ref %s" % (
        bad.size, bad[:5], a.reshape(-1)[bad[:5]], q_ref.reshape(-1)[bad[:5]])


def _same_scales(s_gpu, s_ref):
    a = np.ascontiguousarray(host(s_gpu)).view(np.uint32).reshape(-1)
    b = np.ascontiguousarray(s_ref).view(np.uint32).reshape(-1)
    assert a.shape == b.shape
    bad = np.flatnonzero(a != b)
    assert bad.size == 0, "scale mismatch at %s: gpu %s ref %s" % (bad[:5], a[bad[:5]], b[bad[:5]])


# -------------------------------------------------------------- quantizers
@pytest.mark.parametrize("shape", [(256, 512), (7, 264), (1, 8), (300, 1000), (50, 2048), (513, 2560),
                                   (21, 4104), (64, 7168), (3, 40000)])
def test_rowwise_quant(shape):
    """One wave per row with the row in registers up to 8192 columns (2, 4, 8
    or 16 chunks per lane: each size and each boundary), one workgroup and
    two passes beyond."""
    _say("rowwise", shape)
    x = _bits(shape, 11)
    q, s = ops.quant_rowwise(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.quant_rowwise(x)
    _same_codes(q, qr)
    _same_scales(s, sr)


def test_rowwise_special_rows_and_stride():
    """Zero, -0, subnormal-scale, huge and exactly-448 rows; an input row
    stride larger than the row."""
    rows, cols, ld = 6, 264, 304
    full = _bits((rows, ld), 12)
    full[0, :] = 0
    full[1, :] = 0x8000
    full[2, :cols] = inputs.to_bf16_bits(np.linspace(-1e-38, 1e-38, cols).astype(np.float32))
    full[3, :cols] = inputs.to_bf16_bits(np.linspace(-3e38, 3e38, cols).astype(np.float32))
    full[4, :cols] = inputs.to_bf16_bits(np.full(cols, 448.0, np.float32))
    full[5, :cols] = inputs.to_bf16_bits((np.arange(cols) * 1e-20).astype(np.float32))
    xd = dev_bf16(full)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows,), dtype=torch.float32, device="cuda")
    ops.fp8_quant_rowwise(xd, rows, cols, ld, q, cols, s)
    torch.cuda.synchronize()
    qr, sr = oracle.quant_rowwise(np.ascontiguousarray(full[:, :cols]))
    _same_codes(q, qr)
    _same_scales(s, sr)


@pytest.mark.parametrize("shape", [(256, 512), (7, 264), (1, 8), (4096, 7168), (10001, 136), (4096, 2560)])
def test_tensorwise_quant(shape):
    """Sizes from one workgroup to more than the amax grid (many atomics)."""
    _say("tensorwise", shape)
    x = _bits(shape, 13)
    q, s = ops.quant_tensorwise(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.quant_tensorwise(x)
    _same_codes(q, qr)
    _same_scales(s, sr)


def test_tensorwise_amax_position_and_reuse():
    """The largest |x| sits in the last element, then in the first; the scale
    buffer holds a stale larger value from the previous call (it must be
    reset by each call)."""
    x = _bits((513, 1024), 14, frac=0.0, mult=1.0)
    xd = dev_bf16(x)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    for pos in ((-1, -1), (0, 0)):
        y = x.copy()
        y[pos] = inputs.to_bf16_bits(np.array([-977.0], np.float32))[0]
        xd.copy_(dev_bf16(y))
        ops.fp8_quant_tensorwise(xd, y.shape[0], y.shape[1], y.shape[1], q, y.shape[1], s)
        torch.cuda.synchronize()
        qr, sr = oracle.quant_tensorwise(y)
        _same_codes(q, qr)
        _same_scales(s, sr)


def test_empty_inputs():
    q = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    s = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ops.fp8_quant_rowwise(x, 0, 64, 64, q, 64, s)
    ops.fp8_quant_tensorwise(x, 0, 64, 64, q, 64, s)
    torch.cuda.synchronize()
    assert host(s)[0] == 0.0                        # an empty tensor has amax 0
    with pytest.raises(ops.Fp8bsError):
        ops.fp8_quant_rowwise(dev_bf16(_bits((4, 12), 1)), 4, 12, 12, q, 12, s)   # cols % 8


# ------------------------------------------------------------------- GEMM
def _rowwise_operands(M, N, K, seed, tensor=False):
    x = _bits((M, K), seed, frac=0.0, mult=1.0)
    w = _bits((N, K), seed + 1, sigma=0.02, frac=0.0, mult=1.0)
    f = ops.quant_tensorwise if tensor else ops.quant_rowwise
    qa, sa = f(dev_bf16(x))
    qb, sb = f(dev_bf16(w))
    return qa, sa, qb, sb


def _check(qa, sa, qb, sb, mi=None, ni=None):
    M, K = qa.shape
    N = qb.shape[0]
    y16 = ops.gemm_rowscaled(qa, sa, qb, sb, torch.bfloat16)
    y32 = ops.gemm_rowscaled(qa, sa, qb, sb, torch.float32)
    torch.cuda.synchronize()
    sae, sbe = oracle.expand_rowscales(host(sa), host(sb), M, N, K)
    verify(host(qa), sae, host(qb), sbe, host(y32), host(y16), bscale_row=True, mi=mi, ni=ni)


@pytest.mark.parametrize("tensor", [False, True])
@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (300, 384, 1024), (1, 128, 128), (513, 640, 384)])
def test_rowscaled_gemm_small(M, N, K, tensor):
    """Every output, ragged M, several tiles."""
    _say("rowscaled gemm", M, N, K, "tensor" if tensor else "row")
    _check(*_rowwise_operands(M, N, K, M + N + K, tensor))


@pytest.mark.parametrize("M,N,K", [(3200, 10112, 2048), (2816, 9344, 4096)])
def test_rowscaled_gemm_two_regions(M, N, K):
    """Shapes the planner splits into two column regions of different tilings:
    sampled outputs, tile corners and the columns around the boundary."""
    first, second, split = ops.fp8_blockscaled_gemm_plan(M, N, K)
    assert second is not None and 0 < split < N
    _say("rowscaled gemm two regions", M, N, K, "split", split)
    ops_ = _rowwise_operands(M, N, K, 7)
    mi, ni = sample_indices(M, N, 3000, 5)
    cols = np.arange(max(split - 40, 0), min(split + 40, N))
    mi = np.concatenate([mi, np.repeat(np.arange(0, M, 97), cols.size)])
    ni = np.concatenate([ni, np.tile(cols, (M + 96) // 97)])
    _check(*ops_, mi=mi, ni=ni)


def test_rowscaled_gemm_matches_blockscaled_call():
    """With the same scales written out per K slice (K stride 1) the GEMM takes
    the per-slice path; both paths must agree with the oracle, and exactly
    with each other on operands whose sums are exact in any order."""
    M, N, K = 384, 640, 1024
    rng = np.random.default_rng(21)
    qa = oracle.e4m3_encode(rng.integers(-8, 9, (M, K)).astype(np.float32))
    qb = oracle.e4m3_encode(rng.integers(-8, 9, (N, K)).astype(np.float32))
    sa = np.exp2(rng.integers(-6, 7, M)).astype(np.float32)
    sb = np.exp2(rng.integers(-6, 7, N)).astype(np.float32)
    sae, sbe = oracle.expand_rowscales(sa, sb, M, N, K)
    y_kinv = ops.gemm_rowscaled(dev(qa), dev(sa), dev(qb), dev(sb), torch.float32)
    y_blk = ops.gemm(dev(qa), dev(sae), dev(qb), dev(sbe), ops.BSCALE_ROW128, torch.float32)
    torch.cuda.synchronize()
    yref, _ = oracle.gemm_rowscaled(qa, sa, qb, sb, with_abs=False)
    assert np.array_equal(host(y_kinv).astype(np.float64), yref)
    assert np.array_equal(host(y_blk), host(y_kinv))


def test_rowscaled_gemm_tensor_scale_product_shapes():
    """Mixed: rowwise activations with a tensorwise weight scale."""
    M, N, K = 520, 768, 640
    x = _bits((M, K), 31, frac=0.0, mult=1.0)
    w = _bits((N, K), 32, sigma=0.02, frac=0.0, mult=1.0)
    qa, sa = ops.quant_rowwise(dev_bf16(x))
    qb, sb = ops.quant_tensorwise(dev_bf16(w))
    _check(qa, sa, qb, sb)
