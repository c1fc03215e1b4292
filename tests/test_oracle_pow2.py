"""Pins for the oracle's block-wise quantizers with power-of-two scales (CPU).

The block-wise recipe (1x128 activation groups, 128x128 weight blocks, "Low
Precision RL", section "2. Unified block-wise FP8 (DeepSeek-style)") with
each group's scale rounded up to a power of two and stored as a UE8M0 byte,
the form TransformerEngine uses when it runs that recipe through MXFP8 on
Blackwell (the same page, on NVTE_FP8_BLOCK_SCALING_FP32_SCALES); the
exponent rule is the MX one: the smallest e with amax <= 448 * 2^e.

Checks: an independent re-derivation (exponent by exact fp64 search, codes
by torch's float8 cast of x * 2^-e), the scale's bracket around amax / 448,
exact power-of-two metamorphic shifts, the decoded scale values, and the
accuracy cost against FP32 scales on the MLP workload's tensors.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs


def _f32(bits):
    return oracle.bf16_to_f32(bits)


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _exp_rule(amax):
    """Smallest integer e with amax <= 448 * 2^e (exact fp64), in [-127, 127]."""
    if amax == 0.0:
        return -127
    e = int(np.floor(np.log2(amax))) - 10
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return max(-127, min(127, e))


def independent_pow2(x_bits, block_rows):
    x = _f32(x_bits).astype(np.float64)
    rows, cols = x.shape
    ngr, ngc = -(-rows // block_rows), -(-cols // 128)
    q = np.zeros((rows, cols), np.uint8)
    s = np.zeros((ngr, ngc), np.uint8)
    for i in range(ngr):
        for g in range(ngc):
            blk = x[i * block_rows:(i + 1) * block_rows, g * 128:(g + 1) * 128]
            amax = float(np.abs(blk).max())
            e = _exp_rule(amax)
            s[i, g] = e + 127
            if amax > 0:
                q[i * block_rows:(i + 1) * block_rows, g * 128:(g + 1) * 128] = _torch_e4m3(blk * 2.0 ** -e)
    return q, s


@pytest.mark.parametrize("shape", [(3, 128), (7, 300), (130, 260), (1, 8)])
def test_1x128_pow2_matches_independent(shape):
    x = inputs.normal_bf16(np.random.default_rng(1), shape, 1.0, 0.02, 60.0)
    q, s = oracle.quant_1x128_pow2(x)
    qi, si = independent_pow2(x, 1)
    assert np.array_equal(s, si) and np.array_equal(q, qi)


@pytest.mark.parametrize("shape", [(128, 128), (200, 300), (256, 136)])
def test_128x128_pow2_matches_independent(shape):
    x = inputs.normal_bf16(np.random.default_rng(2), shape, 0.02, 0.01, 40.0)
    q, s = oracle.quant_128x128_pow2(x)
    qi, si = independent_pow2(x, 128)
    assert np.array_equal(s, si) and np.array_equal(q, qi)


def test_scale_brackets_fp32_scale_and_special_groups():
    x = inputs.normal_bf16(np.random.default_rng(3), (64, 512), 1.0, 0.02, 60.0)
    x[0, :128] = 0                                                    # zero group
    x[1, :128] = inputs.to_bf16_bits(np.full(128, 448.0 * 2.0 ** -3, np.float32))   # amax = 448 * 2^-3
    x[2, :128] = inputs.to_bf16_bits(np.linspace(-3e38, 3e38, 128).astype(np.float32))
    q, s = oracle.quant_1x128_pow2(x)
    amax = np.abs(_f32(x).astype(np.float64)).reshape(64, 4, 128).max(axis=2)
    p2 = np.exp2(s.astype(np.float64) - 127)
    live = (amax > 0) & (s < 254)
    assert np.all(amax[live] <= 448 * p2[live]) and np.all(amax[live] > 224 * p2[live])
    assert s[0, 0] == 0 and not q[0, :128].any()                      # e = -127, all codes 0x00
    assert s[1, 0] == 127 - 3 and np.all(q[1, :128] == 0x7E)           # exactly 448 after scaling
    assert s[2, 0] == 127 + 120                                       # 3e38 / 448 rounds up to 2^120


def test_power_of_two_input_scaling_shifts_the_byte():
    x = inputs.normal_bf16(np.random.default_rng(4), (130, 384), 1.0)
    q, s = oracle.quant_128x128_pow2(x)
    for j in (-5, 3, 11):
        y = inputs.to_bf16_bits(_f32(x) * np.float32(2.0 ** j))
        qj, sj = oracle.quant_128x128_pow2(y)
        assert np.array_equal(qj, q) and np.array_equal(sj.astype(int), s.astype(int) + j)


def test_decoded_scales():
    c = np.arange(255, dtype=np.uint8)
    v = oracle.pow2_scales(c)
    assert v.dtype == np.float32
    assert np.array_equal(v.astype(np.float64), 2.0 ** (c.astype(np.float64) - 127))


def test_accuracy_cost_against_fp32_scales():
    """The MLP workload's X_up (first 512 tokens) and W_up (first 512 rows).
    Invariant: with either scale S every element's dequantization error is at
    most 2^-4 |x| (E4M3's 3-bit significand) plus half the smallest subnormal
    step, 2^-10 S.  Measured (printed): a power-of-two S sits up to 2x above
    amax / 448, so a group's largest elements land on a coarser part of the
    grid.  On W (no outliers) the RMS error is unchanged within 5%; on X the
    x100 outliers, which are their group's maximum, dominate the norm and
    the error grows; the sampled GEMM outputs' error grows less than 2x."""
    d = inputs.qwen3_4b_mlp(1, parts=("up",))
    x, w = d["x_up"][:512], d["w_up"][:512]
    res = {}
    for name, data, bl in (("x", x, 1), ("w", w, 128)):
        ref = _f32(data).astype(np.float64)
        if bl == 1:
            q32, s32 = oracle.quant_1x128(data)
            deq32 = oracle.e4m3_decode(q32) * np.repeat(s32.astype(np.float64), 128, axis=1)[:, :data.shape[1]]
            q2, s2 = oracle.quant_1x128_pow2(data)
            deq2 = oracle.e4m3_decode(q2) * np.repeat(oracle.pow2_scales(s2).astype(np.float64), 128,
                                                      axis=1)[:, :data.shape[1]]
        else:
            q32, s32 = oracle.quant_128x128(data)
            e32 = np.repeat(np.repeat(s32.astype(np.float64), 128, axis=0), 128, axis=1)
            deq32 = oracle.e4m3_decode(q32) * e32[:data.shape[0], :data.shape[1]]
            q2, s2 = oracle.quant_128x128_pow2(data)
            e2 = np.repeat(np.repeat(oracle.pow2_scales(s2).astype(np.float64), 128, axis=0), 128, axis=1)
            deq2 = oracle.e4m3_decode(q2) * e2[:data.shape[0], :data.shape[1]]
            s32e = e32[:data.shape[0], :data.shape[1]]
            s2e = e2[:data.shape[0], :data.shape[1]]
        if bl == 1:
            s32e = np.repeat(s32.astype(np.float64), 128, axis=1)[:, :data.shape[1]]
            s2e = np.repeat(oracle.pow2_scales(s2).astype(np.float64), 128, axis=1)[:, :data.shape[1]]
        for deq, se in ((deq32, s32e), (deq2, s2e)):
            assert np.all(np.abs(deq - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * se)
        n = np.linalg.norm(ref)
        res[name] = (np.linalg.norm(deq32 - ref) / n, np.linalg.norm(deq2 - ref) / n)
    print("relative RMS dequantization error (fp32 scales, pow2 scales):", res)
    assert abs(res["w"][1] / res["w"][0] - 1.0) < 0.05
    assert res["x"][1] > res["x"][0]
    # GEMM outputs on sampled (token, feature) pairs against the exact bf16 product
    rng = np.random.default_rng(9)
    mi, ni = rng.integers(0, 512, 4000), rng.integers(0, 512, 4000)
    exact = np.einsum("ij,ij->i", _f32(x)[mi].astype(np.float64), _f32(w)[ni].astype(np.float64))
    qa, sa = oracle.quant_1x128(x)
    qb, sb = oracle.quant_128x128(w)
    y32, _ = oracle.gemm_blockscaled_sampled(qa, sa, qb, sb, mi, ni)
    qa2, sa2 = oracle.quant_1x128_pow2(x)
    qb2, sb2 = oracle.quant_128x128_pow2(w)
    y2, _ = oracle.gemm_blockscaled_sampled(qa2, oracle.pow2_scales(sa2), qb2, oracle.pow2_scales(sb2), mi, ni)
    r32 = np.linalg.norm(y32 - exact) / np.linalg.norm(exact)
    r2 = np.linalg.norm(y2 - exact) / np.linalg.norm(exact)
    print("relative GEMM output error vs the exact bf16 product: fp32 scales %.4g, pow2 scales %.4g" % (r32, r2))
    assert r32 < r2 < 2.0 * r32
