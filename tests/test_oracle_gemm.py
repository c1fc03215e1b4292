"""Pins for the oracle's reference GEMMs, SiLU-mul and grouped composition.

The block-scaled GEMM is the product of the dequantized operands,
Y = (dec(qa) * sa) (dec(qb) * sb)^T, accumulated here in fp64; the scales come
from the quantizers of "Unified FP8: Beyond Mixed Precision...", section
"FP8 Quantization", with 128x128 weight blocks / 1x128 activation groups
("Low Precision RL", section "2. Unified block-wise FP8 (DeepSeek-style)")
and 1x32 UE8M0 blocks for MXFP8 (section "3. Unified MXFP8 (Blackwell)").

Checks: numpy float64 matmul on operands dequantized independently (torch's
float8 decode), an exact integer special case, and grouped == per-expert
dense on a brute-force loop.
"""
import numpy as np
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs


def _dequant_torch(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _expand(s, rows, cols, rblk, cblk):
    return np.repeat(np.repeat(s.astype(np.float64), rblk, axis=0), cblk, axis=1)[:rows, :cols]


def _rand_operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    xa = inputs.normal_bf16(rng, (M, K), 1.0, 0.01, 30.0)
    xb = inputs.normal_bf16(rng, (N, K), 0.02)
    qa, sa = oracle.quant_1x128(xa)
    qb, sb = oracle.quant_128x128(xb)
    return qa, sa, qb, sb


def test_gemm_block128_vs_numpy():
    M, N, K = 48, 256, 384
    qa, sa, qb, sb = _rand_operands(M, N, K, 0)
    y, yabs = oracle.gemm_blockscaled(qa, sa, qb, sb, oracle.BSCALE_BLOCK128)
    A = _dequant_torch(qa) * _expand(sa, M, K, 1, 128)
    B = _dequant_torch(qb) * _expand(sb, N, K, 128, 128)
    ref = A @ B.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(A) @ np.abs(B).T)
    assert np.allclose(yabs, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)


def test_gemm_row128_vs_numpy():
    M, N, K = 40, 72, 256
    rng = np.random.default_rng(1)
    qa, sa = oracle.quant_1x128(inputs.normal_bf16(rng, (M, K), 1.0))
    qb, sb = oracle.quant_1x128(inputs.normal_bf16(rng, (N, K), 1.0))
    y, _ = oracle.gemm_blockscaled(qa, sa, qb, sb, oracle.BSCALE_ROW128)
    A = _dequant_torch(qa) * _expand(sa, M, K, 1, 128)
    B = _dequant_torch(qb) * _expand(sb, N, K, 1, 128)
    ref = A @ B.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(A) @ np.abs(B).T)


def test_gemm_sampled_equals_full():
    qa, sa, qb, sb = _rand_operands(32, 128, 256, 2)
    y, yabs = oracle.gemm_blockscaled(qa, sa, qb, sb)
    mi = np.array([0, 5, 31, 17])
    ni = np.array([0, 127, 64, 3])
    ys, ysabs = oracle.gemm_blockscaled_sampled(qa, sa, qb, sb, mi, ni)
    assert np.array_equal(ys, y[mi, ni]) and np.array_equal(ysabs, yabs[mi, ni])


def exact_operands(M, N, K, seed):
    """Integer codes in [-8, 8] and power-of-two scales: every product and
    partial sum is exactly representable, so the result is exact in any
    summation order and equals an integer matmul."""
    rng = np.random.default_rng(seed)
    ia = rng.integers(-8, 9, size=(M, K))
    ib = rng.integers(-8, 9, size=(N, K))
    enc = lambda v: oracle.e4m3_encode(v.astype(np.float32))
    ja = rng.integers(-1, 2, size=(M, K // 128))
    jb = rng.integers(-1, 2, size=(N // 128, K // 128))
    return ia, ib, enc(ia), enc(ib), ja, jb


def test_gemm_exact_integer_case():
    M, N, K = 64, 256, 512
    ia, ib, qa, qb, ja, jb = exact_operands(M, N, K, 3)
    sa = np.exp2(ja).astype(np.float32)
    sb = np.exp2(jb).astype(np.float32)
    y, _ = oracle.gemm_blockscaled(qa, sa, qb, sb)
    # exact: sum over k-blocks of integer dot * 2^(ja + jb), in units of 2^-2
    ref = np.zeros((M, N), np.int64)
    for kb in range(K // 128):
        d = ia[:, kb * 128:(kb + 1) * 128].astype(np.int64) @ ib[:, kb * 128:(kb + 1) * 128].T.astype(np.int64)
        ea = ja[:, kb][:, None] + 1
        eb = np.repeat(jb[:, kb], 128)[None, :] + 1
        ref += d * (2 ** (ea + eb))
    assert np.array_equal(y, ref.astype(np.float64) / 4.0)


def test_gemm_mx_vs_numpy_and_exact():
    M, N, K = 16, 48, 256
    rng = np.random.default_rng(4)
    qa, sa = oracle.mx_quant_1x32(inputs.normal_bf16(rng, (M, K), 1.0, 0.02, 40.0))
    qb, sb = oracle.mx_quant_1x32(inputs.normal_bf16(rng, (N, K), 0.02))
    y, yabs = oracle.gemm_mx(qa, sa, qb, sb)
    A = _dequant_torch(qa) * np.repeat(np.exp2(sa.astype(np.float64) - 127), 32, axis=1)
    B = _dequant_torch(qb) * np.repeat(np.exp2(sb.astype(np.float64) - 127), 32, axis=1)
    assert np.max(np.abs(y - A @ B.T)) <= 1e-12 * np.max(np.abs(A) @ np.abs(B).T)
    # exact case: integer codes, UE8M0 codes 126..128
    ia = rng.integers(-8, 9, size=(M, K))
    ib = rng.integers(-8, 9, size=(N, K))
    ea = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    y2, _ = oracle.gemm_mx(oracle.e4m3_encode(ia.astype(np.float32)), ea,
                           oracle.e4m3_encode(ib.astype(np.float32)), eb)
    ref = np.zeros((M, N), np.int64)
    for kb in range(K // 32):
        d = ia[:, kb * 32:(kb + 1) * 32] @ ib[:, kb * 32:(kb + 1) * 32].T
        ref += d * 2 ** ((ea[:, kb].astype(np.int64) - 126)[:, None] + (eb[:, kb].astype(np.int64) - 126)[None, :])
    assert np.array_equal(y2, ref / 4.0)


def test_grouped_equals_per_expert_loop():
    moe = inputs.small_moe()
    r = moe["routing"]
    assert np.any(np.diff(r.offsets) == 0)          # the skewed draw has empty groups
    x = moe["x"][r.row_token]
    qa, sa = oracle.quant_1x128(x)
    G = r.offsets.size - 1
    wq, ws = zip(*(oracle.quant_128x128(moe["w_gu"][g]) for g in range(G)))
    wq, ws = np.stack(wq), np.stack(ws)
    y, yabs = oracle.grouped_gemm_blockscaled(qa, sa, r.offsets, wq, ws)
    A = _dequant_torch(qa) * _expand(sa, *qa.shape, 1, 128)
    for i in range(0, x.shape[0], 37):
        g = int(np.searchsorted(r.offsets, i, side="right") - 1)
        B = _dequant_torch(wq[g]) * _expand(ws[g], *wq[g].shape, 128, 128)
        ref = B @ A[i]
        assert np.allclose(y[i], ref, rtol=1e-12, atol=1e-14)


def test_silu_mul_vs_torch():
    rng = np.random.default_rng(5)
    gu = inputs.normal_bf16(rng, (64, 256), 3.0)
    h = oracle.silu_mul(gu)
    g = oracle.bf16_to_f32(gu[:, :128]).astype(np.float64)
    u = oracle.bf16_to_f32(gu[:, 128:]).astype(np.float64)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    hv = oracle.bf16_to_f32(h).astype(np.float64)
    # h is the bf16 value nearest to the fp64 product: within half a bf16 ulp
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(hv - ref) <= ulp / 2 * (1 + 1e-9))
    # gate / up order matters: swapping them changes the result
    swapped = oracle.silu_mul(np.concatenate([gu[:, 128:], gu[:, :128]], axis=1))
    assert not np.array_equal(swapped, h)


def test_gemm_rowscaled_vs_numpy():
    """Scales constant along K (rowwise and tensorwise): fp64 product of the
    independently decoded operands, each row scaled once."""
    M, N, K = 40, 96, 384
    rng = np.random.default_rng(5)
    xa = inputs.normal_bf16(rng, (M, K), 1.0, 0.01, 30.0)
    xb = inputs.normal_bf16(rng, (N, K), 0.02)
    for quant in (oracle.quant_rowwise, oracle.quant_tensorwise):
        qa, sa = quant(xa)
        qb, sb = quant(xb)
        y, yabs = oracle.gemm_rowscaled(qa, sa, qb, sb)
        A = _dequant_torch(qa) * np.broadcast_to(sa.astype(np.float64).reshape(-1, 1), (M, 1))
        B = _dequant_torch(qb) * np.broadcast_to(sb.astype(np.float64).reshape(-1, 1), (N, 1))
        ref = A @ B.T
        assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(A) @ np.abs(B).T)
        assert np.allclose(yabs, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)
