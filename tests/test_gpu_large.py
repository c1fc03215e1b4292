"""The largest operands the ABI accepts: the GEMMs address operand rows with
32-bit byte offsets, so the host admits an operand only below 4 GiB.  An
activation operand just under that bound goes through the block-scaled and
the MXFP8 GEMMs; rows spread over the whole operand, the last ones
included, are compared bit for bit with the oracle (small-integer codes and
power-of-two scales make every sum exact; "Low Precision RL", section "2.
Unified block-wise FP8 (DeepSeek-style)" for the GEMM)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import ops
from gpu_util import host

pytestmark = pytest.mark.gpu

M, N, K = 1048000, 256, 4096          # A: 4,292,608,000 bytes, 2,359,296 below 4 GiB


def _say(*a):
    print(*a, flush=True)


def _rows():
    r = np.linspace(0, M - 1, 60).astype(np.int64)
    return np.unique(np.concatenate([r, np.arange(M - 4, M)]))


def _codes(shape, g):
    """E4M3 codes of +-2^k, k = 0..3 (exponent field k + 7, mantissa 0), made
    with byte arithmetic on the device (no index temporaries)."""
    c = torch.randint(0, 4, shape, device="cuda", generator=g, dtype=torch.uint8)
    c.add_(7).mul_(8)
    return c.bitwise_or_(torch.randint(0, 2, shape, device="cuda", generator=g, dtype=torch.uint8).mul_(128))


@pytest.fixture(scope="module")
def operands():
    assert M * K < (1 << 32) and M * K > (1 << 32) - (1 << 22)
    g = torch.Generator(device="cuda").manual_seed(40)
    a, b = _codes((M, K), g), _codes((N, K), g)
    _say("operand A: %d bytes" % a.numel())
    yield a, b, g
    del a, b
    torch.cuda.empty_cache()


def test_blockscaled_gemm_operand_just_under_4gib(operands):
    a, b, g = operands
    sa_e = torch.randint(-1, 2, (K // 128, M), device="cuda", generator=g, dtype=torch.int32)
    sb_e = torch.randint(-1, 2, (N // 128, K // 128), device="cuda", generator=g, dtype=torch.int32)
    sa = torch.exp2(sa_e.float())                     # M-major [K/128][M]
    sb = torch.exp2(sb_e.float())
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _say("block-scaled GEMM", M, N, K)
    ops.fp8_blockscaled_gemm(M, N, K, a, K, sa, 1, M, b, K, sb, K // 128, 1, ops.BSCALE_BLOCK128, c, N, ops.OUT_BF16)
    torch.cuda.synchronize()
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    yref, _ = oracle.gemm_blockscaled(host(a[ri]), host(sa[:, ri].t().contiguous()), host(b), host(sb),
                                      with_abs=False)
    assert np.array_equal(host(c[ri]), oracle.f64_to_bf16(yref))


def test_mx_gemm_operand_just_under_4gib(operands):
    a, b, g = operands
    ea = torch.randint(126, 129, (M, K // 32), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    eb = torch.randint(126, 129, (N, K // 32), device="cuda", generator=g, dtype=torch.int32).to(torch.uint8)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _say("MXFP8 GEMM", M, N, K)
    ops.mxfp8_gemm(M, N, K, 0, None, None, M, a, K, ea, K // 32, b, K, 0, eb, K // 32, 0, c, N, ops.OUT_BF16)
    torch.cuda.synchronize()
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    yref, _ = oracle.gemm_mx(host(a[ri]), host(ea[ri]), host(b), host(eb))
    assert np.array_equal(host(c[ri]), oracle.f64_to_bf16(yref))


def test_operand_of_4gib_rejected(operands):
    """2^32 / K rows make the operand exactly 4 GiB: rejected on the host with
    FP8BS_ERR_SHAPE before anything is launched (no buffer is touched)."""
    a, b, _ = operands
    rows = (1 << 32) // K
    s = torch.ones((K // 128, 8), dtype=torch.float32, device="cuda")
    c = torch.empty((2, N), dtype=torch.bfloat16, device="cuda")
    st = ops.fp8_blockscaled_gemm(rows, N, K, a, K, s, 0, 1, b, K, s, 1, 1, ops.BSCALE_BLOCK128, c, N,
                                  ops.OUT_BF16, raise_on_error=False)
    assert st == 2
