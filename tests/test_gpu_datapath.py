"""GPU pin of gfx950's FP8 dot-product datapath through the public GEMMs:
hand-built 8-K runs (tests/datapath_cases.py) must give the hand-derived
outputs exactly, in every GEMM mode (FP32 block scales with per-slice
promotion, per-row scales, K-invariant scales, power-of-two block scales,
dense and grouped MXFP8, the grouped block-scaled GEMM), fp32 and bf16 out.
The same literals pin the datapath model on the CPU
(tests/test_datapath_model.py), so together they tie the model that the
parity tests compare against to the hardware."""
import numpy as np
import pytest
import torch

import oracle
from datapath_cases import expected_full, operands
from fp8_block_scaled_x128_amd import ops
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

QA, QB = operands()
M, K = QA.shape
N = QB.shape[0]
REF = expected_full()


def _check(y, out):
    y = host(y)
    if out == ops.OUT_FP32:
        bad = np.argwhere(y.astype(np.float64) != REF)
        assert bad.size == 0, ["C[%d, %d] = %r, expected %r" % (m, n, float(y[m, n]), REF[m, n]) for m, n in bad[:8]]
    else:
        assert np.array_equal(y, oracle.f64_to_bf16(REF))


@pytest.mark.parametrize("out", [ops.OUT_FP32, ops.OUT_BF16])
@pytest.mark.parametrize("mode", ["block128", "row128", "kinv"])
def test_fp32_scale_modes(mode, out):
    print("datapath", mode, out, flush=True)
    a, b = dev(QA), dev(QB)
    dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
    c = torch.empty((M, N), dtype=dt, device="cuda")
    sa = torch.ones((K // 128, M), dtype=torch.float32, device="cuda")       # M-major
    if mode == "block128":
        sb = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
        ops.fp8_blockscaled_gemm(M, N, K, a, K, sa, 1, M, b, K, sb, K // 128, 1, ops.BSCALE_BLOCK128, c, N, out)
    elif mode == "row128":
        sb = torch.ones((N, K // 128), dtype=torch.float32, device="cuda")
        ops.fp8_blockscaled_gemm(M, N, K, a, K, sa, 1, M, b, K, sb, K // 128, 1, ops.BSCALE_ROW128, c, N, out)
    else:
        sa1 = torch.ones(M, dtype=torch.float32, device="cuda")
        sb1 = torch.ones(N, dtype=torch.float32, device="cuda")
        ops.fp8_blockscaled_gemm(M, N, K, a, K, sa1, 1, 0, b, K, sb1, 1, 0, ops.BSCALE_ROW128, c, N, out)
    torch.cuda.synchronize()
    _check(c, out)


@pytest.mark.parametrize("out", [ops.OUT_FP32, ops.OUT_BF16])
def test_pow2_scales(out):
    a, b = dev(QA), dev(QB)
    sa = torch.full((M, 4), 127, dtype=torch.uint8, device="cuda")
    sb = torch.full((N // 128, 4), 127, dtype=torch.uint8, device="cuda")
    dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
    c = torch.empty((M, N), dtype=dt, device="cuda")
    ops.fp8_blockscaled_gemm_pow2(M, N, K, a, K, sa, 4, b, K, sb, 4, c, N, out)
    torch.cuda.synchronize()
    _check(c, out)


@pytest.mark.parametrize("out", [ops.OUT_FP32, ops.OUT_BF16])
@pytest.mark.parametrize("groups", [0, 1, 2])
def test_mxfp8(groups, out):
    """Dense (groups 0) and grouped MXFP8 with unit UE8M0 scales; grouped
    runs put rows [0, 9) in expert 0 and [9, 17) in expert 1, both holding B."""
    a = dev(QA)
    G = max(groups, 1)
    b = dev(np.concatenate([QB] * G))
    sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
    sb = torch.full((G * N, K // 32), 127, dtype=torch.uint8, device="cuda")
    dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
    c = torch.empty((M, N), dtype=dt, device="cuda")
    offs = None
    if groups:
        offs = dev(np.array([0, M] if groups == 1 else [0, 9, M], np.int32))
    ops.mxfp8_gemm(M, N, K, groups, offs, None, M, a, K, sa, K // 32, b, K, N * K, sb, K // 32, N * (K // 32),
                   c, N, out)
    torch.cuda.synchronize()
    _check(c, out)


@pytest.mark.parametrize("out", [ops.OUT_FP32, ops.OUT_BF16])
def test_grouped_block128(out):
    a = dev(QA)
    b = dev(np.concatenate([QB, QB]))
    sa = torch.ones((K // 128, M), dtype=torch.float32, device="cuda")
    sb = torch.ones((2, N // 128, K // 128), dtype=torch.float32, device="cuda")
    offs = dev(np.array([0, 9, M], np.int32))
    dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
    c = torch.empty((M, N), dtype=dt, device="cuda")
    ops.fp8_grouped_gemm(M, N, K, 2, offs, None, M, a, K, sa, 1, M, b, K, N * K, sb, (N // 128) * (K // 128),
                         K // 128, 1, c, N, out)
    torch.cuda.synchronize()
    _check(c, out)
