"""Pins for the oracle's quantizers (CPU only).

Quantizer: S = max|X| / V_max with V_max = 448, Q(x) = round(x / S)
("Unified FP8: Beyond Mixed Precision...", section "FP8 Quantization",
Steps 1 and 2), over 1x128 / 128x1 / 128x128 groups with FP32 scales
("Low Precision RL", table "Choose a precision", section
"2. Unified block-wise FP8 (DeepSeek-style)") and over 1x32 blocks with
UE8M0 scales (section "3. Unified MXFP8 (Blackwell)").

The checks are an independent vectorised implementation (numpy fp32 division
and torch's float8 cast), the invariants fixed by the definition (the amax
element lands on +-448; the dequantization error bound), and metamorphic
relations (power-of-two scaling, sign flip, transpose, permutation,
locality).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs


def _bf16(x):
    return inputs.to_bf16_bits(np.asarray(x, np.float32))


def _f32(bits):
    return oracle.bf16_to_f32(bits)


def _torch_e4m3(v32):
    v = np.clip(v32, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def independent_rowblock(x_bits, group=128):
    """numpy/torch re-derivation of 1xG quantization (ragged last group)."""
    x = _f32(x_bits)
    rows, cols = x.shape
    ng = -(-cols // group)
    pad = np.zeros((rows, ng * group), np.float32)
    pad[:, :cols] = x
    g = pad.reshape(rows, ng, group)
    amax = np.abs(g).max(axis=2).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / s[:, :, None]).astype(np.float32)
    codes = _torch_e4m3(np.nan_to_num(ratio, nan=0.0)).reshape(rows, ng * group)[:, :cols]
    zero = np.repeat(s == 0, group, axis=1)[:, :cols]
    codes = np.where(zero, 0, codes).astype(np.uint8)
    return codes, s


def _rand_bits(shape, seed, outliers=True):
    rng = np.random.default_rng(seed)
    if outliers:
        return inputs.normal_bf16(rng, shape, 1.0, 0.01, 50.0)
    return inputs.normal_bf16(rng, shape, 1.0)


@pytest.mark.parametrize("shape", [(3, 128), (7, 300), (64, 512), (5, 1)])
def test_1x128_matches_independent(shape):
    x = _rand_bits(shape, 1)
    q, s = oracle.quant_1x128(x)
    q2, s2 = independent_rowblock(x)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q, q2)


def test_128x1_t_is_1x128_of_transpose():
    x = _rand_bits((300, 70), 2)
    qt, s = oracle.quant_128x1_t(x)
    q2, s2 = oracle.quant_1x128(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))


def test_128x128_matches_independent():
    x = _rand_bits((300, 260), 3)
    q, s = oracle.quant_128x128(x)
    xf = _f32(x)
    for br in range(3):
        for bc in range(3):
            blk = xf[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
            sc = np.float32(np.abs(blk).max()) / np.float32(448.0)
            assert s[br, bc].view(np.uint32) == np.float32(sc).view(np.uint32)
            ref = _torch_e4m3((blk / np.float32(sc)).astype(np.float32))
            assert np.array_equal(q[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128], ref)


def test_128x128_transpose_invariant():
    x = _rand_bits((384, 256), 4)
    q, s = oracle.quant_128x128(x)
    qt, st = oracle.quant_128x128(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_amax_element_lands_on_448():
    x = _rand_bits((64, 1024), 5)
    q, s = oracle.quant_1x128(x)
    xf = _f32(x).reshape(64, 8, 128)
    idx = np.abs(xf).argmax(axis=2)
    qq = q.reshape(64, 8, 128)
    picked = np.take_along_axis(qq, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all((picked == 0x7E) | (picked == 0xFE))
    assert np.all(s >= np.float32(2.0 ** -126))    # invariant holds for normal S


def test_dequant_error_bound():
    """|dec(q) S - x| <= S (ulp_E4M3(x/S)/2 + 2^-24 |x/S|)."""
    x = _rand_bits((32, 512), 6)
    q, s = oracle.quant_1x128(x)
    xf = _f32(x).astype(np.float64).reshape(32, 4, 128)
    S = s.astype(np.float64)[:, :, None]
    deq = oracle.e4m3_decode(q).reshape(32, 4, 128) * S
    r = np.abs(xf / S)
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -9)))
    ulp = np.exp2(np.maximum(e, -6) - 3)
    bound = S * (ulp / 2 + 2.0 ** -24 * r) * (1 + 1e-12)
    assert np.all(np.abs(deq - xf) <= bound)


def test_metamorphic_power_of_two_and_sign():
    x = _rand_bits((16, 256), 7)
    q, s = oracle.quant_1x128(x)
    for j in (-3, 1, 5):
        xs = _bf16(_f32(x) * np.float32(2.0 ** j))
        qj, sj = oracle.quant_1x128(xs)
        assert np.array_equal(qj, q) and np.array_equal(sj, s * np.float32(2.0 ** j))
    qn, sn = oracle.quant_1x128(x ^ np.uint16(0x8000))
    nz = _f32(x) != 0
    assert np.array_equal(qn[nz], q[nz] ^ np.uint8(0x80)) and np.array_equal(sn, s)


def test_metamorphic_row_permutation_and_locality():
    x = _rand_bits((40, 384), 8)
    q, s = oracle.quant_1x128(x)
    perm = np.random.default_rng(0).permutation(40)
    qp, sp = oracle.quant_1x128(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    y = x.copy()
    y[3, 130:200] = _bf16(np.full(70, 1000.0))       # edit group (3, 1) only
    qy, sy = oracle.quant_1x128(y)
    mask = np.ones_like(s, bool)
    mask[3, 1] = False
    assert np.array_equal(sy[mask], s[mask])
    qmask = np.ones_like(q, bool)
    qmask[3, 128:256] = False
    assert np.array_equal(qy[qmask], q[qmask])
    assert sy[3, 1] != s[3, 1]


def test_zero_and_tiny_groups():
    x = np.zeros((2, 256), np.uint16)
    x[0, :128] = 0x8000                        # -0.0 everywhere in group (0,0)
    x[1, 128:] = _bf16(np.full(128, 1e-38))   # subnormal-scale group
    x[1, 200] = _bf16(np.array([-3e-38], np.float32))[0]
    q, s = oracle.quant_1x128(x)
    assert s[0, 0] == 0 and np.all(q[0, :128] == 0) and s[0, 1] == 0 and np.all(q[0, 128:] == 0)
    assert s[1, 1] > 0 and s[1, 1] < np.float32(2.0 ** -126)      # S is an fp32 subnormal
    q2, s2 = independent_rowblock(x)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert q[1, 200] == 0xFE


# ------------------------------------------------------------------ MX
def independent_mx(x_bits):
    x = _f32(x_bits)
    rows, cols = x.shape
    g = x.reshape(rows, cols // 32, 32)
    amax = np.abs(g).max(axis=2)
    e = np.empty(amax.shape, np.int64)
    for idx, a in np.ndenumerate(amax):
        if a == 0:
            e[idx] = -127
        else:   # brute force: smallest k with a <= 448 * 2^k
            k = -127
            while a > 448.0 * 2.0 ** k:
                k += 1
            e[idx] = k
    scaled = (g.astype(np.float64) * np.exp2(-e)[:, :, None]).astype(np.float32)
    codes = _torch_e4m3(scaled).reshape(rows, cols)
    codes = np.where(np.repeat(amax == 0, 32, axis=1), 0, codes).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def test_mx_matches_independent():
    x = _rand_bits((24, 256), 9)
    x[0, :32] = 0
    x[1, 32:64] = _bf16(np.full(32, 448.0))
    x[2, 64:96] = _bf16(np.linspace(-3e-30, 5e-30, 32))
    q, s = oracle.mx_quant_1x32(x)
    q2, s2 = independent_mx(x)
    assert np.array_equal(s, s2) and np.array_equal(q, q2)
    assert s[0, 0] == 0 and s[1, 1] == 127


def test_mx_amax_code_range():
    x = _rand_bits((32, 512), 10)
    q, s = oracle.mx_quant_1x32(x)
    xf = _f32(x).reshape(32, 16, 32)
    idx = np.abs(xf).argmax(axis=2)
    picked = np.take_along_axis(q.reshape(32, 16, 32), idx[:, :, None], axis=2)[:, :, 0] & 0x7F
    assert np.all((picked >= 0x76) & (picked <= 0x7E))


# ----------------------------------------------------- rowwise / tensorwise
# One group per row or per tensor: the per-tensor strategy of "Unified FP8:
# Beyond Mixed Precision..." (section "FP8 Quantization") and the tensorwise
# and rowwise scalings compared in "Towards Full Pipeline FP8 Reinforcement
# Learning for LLMs".

@pytest.mark.parametrize("shape", [(5, 300), (16, 2560), (3, 9728), (1, 8)])
def test_rowwise_matches_independent(shape):
    """Each row is one 1xcols group: the numpy/torch re-derivation with the
    group as wide as the row."""
    x = _rand_bits(shape, 20)
    q, s = oracle.quant_rowwise(x)
    q2, s2 = independent_rowblock(x, group=shape[1])
    assert np.array_equal(s.view(np.uint32), s2[:, 0].view(np.uint32))
    assert np.array_equal(q, q2)


def test_rowwise_on_128_columns_is_1x128():
    x = _rand_bits((40, 128), 21)
    q, s = oracle.quant_rowwise(x)
    q2, s2 = oracle.quant_1x128(x)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2[:, 0].view(np.uint32))


def test_tensorwise_on_one_block_is_128x128():
    x = _rand_bits((128, 128), 22)
    q, s = oracle.quant_tensorwise(x)
    q2, s2 = oracle.quant_128x128(x)
    assert np.array_equal(q, q2) and s[0].view(np.uint32) == s2[0, 0].view(np.uint32)


def test_tensorwise_matches_independent():
    """S = max|x| / 448 over the whole tensor (fp32), codes E4M3(x / S)."""
    x = _rand_bits((300, 520), 23)
    q, s = oracle.quant_tensorwise(x)
    xf = _f32(x)
    sc = np.float32(np.float32(np.abs(xf).max()) / np.float32(448.0))
    assert s[0].view(np.uint32) == sc.view(np.uint32)
    assert np.array_equal(q, _torch_e4m3((xf / sc).astype(np.float32)))
    # the amax element of the tensor lands on +-448, and every element obeys
    # the dequantization bound
    i = np.unravel_index(np.abs(xf).argmax(), xf.shape)
    assert q[i] in (0x7E, 0xFE)
    r = np.abs(xf.astype(np.float64) / np.float64(sc))
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -9)))
    ulp = np.exp2(np.maximum(e, -6) - 3)
    deq = oracle.e4m3_decode(q) * np.float64(sc)
    assert np.all(np.abs(deq - xf) <= sc * (ulp / 2 + 2.0 ** -24 * r) * (1 + 1e-12))


def test_rowwise_and_tensorwise_zero_input():
    x = np.zeros((3, 64), np.uint16)
    q, s = oracle.quant_rowwise(x)
    assert np.all(q == 0) and np.all(s == 0)
    q, s = oracle.quant_tensorwise(x)
    assert np.all(q == 0) and s[0] == 0
