"""The allocation-free K-split GEMM (fp8_blockscaled_gemm_splitk_noalloc,
for callers that cannot allocate): two calls in a row through the C ABI,
the second on a smaller problem (the scratch keeps the first call's
partials), each byte-identical to fp8_blockscaled_gemm_splitk with a
caller workspace and the same split count; both results meet the oracle bit
for bit on exact operands.  A split count whose partials do not fit the
64 MiB scratch is rejected; the planner's count is capped to what fits."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import ops
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

LIMIT = 64 << 20


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    qa = oracle.e4m3_encode(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    qb = oracle.e4m3_encode(rng.integers(-8, 9, size=(N, K)).astype(np.float32))
    sa = np.exp2(rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-1, 2, size=(N // 128, K // 128))).astype(np.float32)
    return qa, sa, qb, sb


def _both(M, N, K, qa, sa, qb, sb, splits, out):
    dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
    a, b, sad, sbd = dev(qa), dev(qb), dev(np.ascontiguousarray(sa.T)), dev(sb)
    c0 = torch.full((M, N), 7.0, dtype=dt, device="cuda")
    c1 = torch.full((M, N), 7.0, dtype=dt, device="cuda")
    ops.fp8_blockscaled_gemm_splitk_noalloc(M, N, K, a, K, sad, 1, M, b, K, sbd, K // 128, 1, ops.BSCALE_BLOCK128,
                                            c0, N, out, splits)
    ws = torch.empty(max(splits, 1) * M * N, dtype=torch.float32, device="cuda")
    ops.fp8_blockscaled_gemm_splitk(M, N, K, a, K, sad, 1, M, b, K, sbd, K // 128, 1, ops.BSCALE_BLOCK128, c1, N,
                                    out, splits, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    return host(c0), host(c1)


def test_noalloc_two_calls_match_workspace_entry_point():
    for (M, N, K, splits, seed) in [(256, 2560, 9728, 11, 1), (96, 1280, 2048, 5, 2)]:
        assert splits * M * N * 4 <= LIMIT
        qa, sa, qb, sb = _case(M, N, K, seed)
        yref, _ = oracle.gemm_blockscaled(qa, sa, qb, sb, with_abs=False)
        for out in (ops.OUT_BF16, ops.OUT_FP32):
            y0, y1 = _both(M, N, K, qa, sa, qb, sb, splits, out)
            assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8)), "noalloc differs from the workspace call"
            if out == ops.OUT_FP32:
                assert np.array_equal(y0.astype(np.float64), yref)
            else:
                assert np.array_equal(y0, oracle.f64_to_bf16(yref))


def test_noalloc_planner_count_capped_and_oversize_rejected():
    M, N, K = 2048, 2560, 9728           # planner: 3 splits = 62.9 MB, fits
    qa, sa, qb, sb = _case(M, N, K, 3)
    splits, wsb = ops.fp8_blockscaled_gemm_splitk_plan(M, N, K, ops.OUT_BF16)
    assert splits > 1 and wsb <= LIMIT
    y0, y1 = _both(M, N, K, qa, sa, qb, sb, splits, ops.OUT_BF16)
    assert np.array_equal(y0, y1)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    a, b = dev(qa), dev(qb)
    sad, sbd = dev(np.ascontiguousarray(sa.T)), dev(sb)
    # splits 0 -> the planner's count (fits): same bytes as the explicit call
    ops.fp8_blockscaled_gemm_splitk_noalloc(M, N, K, a, K, sad, 1, M, b, K, sbd, K // 128, 1, ops.BSCALE_BLOCK128,
                                            c, N, ops.OUT_BF16, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host(c), y0)
    # 4 splits of 2048 x 2560 fp32 = 83.9 MB > 64 MiB: rejected, nothing launched
    st = ops.fp8_blockscaled_gemm_splitk_noalloc(M, N, K, a, K, sad, 1, M, b, K, sbd, K // 128, 1,
                                                 ops.BSCALE_BLOCK128, c, N, ops.OUT_BF16, 4, raise_on_error=False)
    assert st == 2
    assert b"scratch" in ops.load().fp8bs_last_error_detail()
