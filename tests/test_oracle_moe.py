"""Pins for the oracle's MoE combine (the weighted sum of each token's expert
outputs after the grouped down projection) and for the routing positions the
combine reads.

The combine's definition: out[t] = sum_j w[t, j] * y[pos[t, j]], where pos
maps (token, slot) to the token's row in the expert-sorted grouped order.
Checks: the single-slot unit-weight case is a gather; small integers with
power-of-two weights give exact rationals (brute force over Python
fractions); linearity in the weights and independence from slot order; and
the whole one-projection MoE layer through the oracle against a per-token
dense computation that never uses the grouped order.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs


def _bf16(v):
    return inputs.to_bf16_bits(np.asarray(v, np.float32))


def test_routing_positions_are_inverse_of_grouped_order():
    r = inputs.small_moe()["routing"]
    T, k = r.token_rows.shape
    rows = r.token_rows.reshape(-1)
    assert np.array_equal(np.sort(rows), np.arange(T * k))            # a permutation
    assert np.array_equal(r.row_token[r.token_rows], np.repeat(np.arange(T), k).reshape(T, k))
    expert_of_row = np.searchsorted(r.offsets, np.arange(T * k), side="right") - 1
    assert np.array_equal(expert_of_row[r.token_rows], r.topk_experts)
    assert np.allclose(r.weights.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(r.weights, axis=1) <= 0)                     # slots in logit order


def test_single_slot_unit_weight_is_gather():
    rng = np.random.default_rng(1)
    y = inputs.normal_bf16(rng, (50, 24), 1.0)
    pos = rng.permutation(50)[:30].reshape(30, 1).astype(np.int32)
    out = oracle.moe_combine(y, pos, np.ones((30, 1), np.float32))
    assert np.array_equal(out, oracle.bf16_to_f32(y[pos[:, 0]]).astype(np.float64))


def test_exact_small_integers_brute_force():
    rng = np.random.default_rng(2)
    T, k, rows, H = 7, 3, 12, 8
    yv = rng.integers(-20, 21, (rows, H))
    wv = [[Fraction(int(rng.integers(-8, 9)), 2 ** int(rng.integers(0, 6))) for _ in range(k)] for _ in range(T)]
    pos = rng.integers(0, rows, (T, k)).astype(np.int32)
    w = np.array([[float(f) for f in row] for row in wv], np.float32)
    out = oracle.moe_combine(_bf16(yv), pos, w)
    for t in range(T):
        for n in range(H):
            ref = sum(wv[t][j] * int(yv[pos[t, j], n]) for j in range(k))
            assert out[t, n] == float(ref)


def test_linear_in_weights_and_slot_order_free():
    rng = np.random.default_rng(3)
    y = inputs.normal_bf16(rng, (40, 64), 1.0)
    pos = rng.integers(0, 40, (16, 4)).astype(np.int32)
    w1 = rng.standard_normal((16, 4)).astype(np.float32)
    w2 = rng.standard_normal((16, 4)).astype(np.float32)
    a = oracle.moe_combine(y, pos, w1) + oracle.moe_combine(y, pos, w2)
    b = oracle.moe_combine(y, pos, (w1.astype(np.float64) + w2).astype(np.float32))
    scale = oracle.moe_combine(y & np.uint16(0x7FFF), pos, np.abs(w1) + np.abs(w2))    # sum |w| |y|
    assert np.all(np.abs(a - b) <= 1e-6 * np.abs(scale) + 1e-12)    # w1 + w2 rounded once to fp32
    perm = np.array([2, 0, 3, 1])
    c = oracle.moe_combine(y, pos[:, perm], w1[:, perm])
    assert np.allclose(c, oracle.moe_combine(y, pos, w1), rtol=1e-13, atol=1e-13)
    d = oracle.moe_combine(y, pos, -w1)
    assert np.array_equal(d, -oracle.moe_combine(y, pos, w1))


def _dequant(q, s, rblk, cblk):
    d = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return d * np.repeat(np.repeat(s.astype(np.float64), rblk, axis=0), cblk, axis=1)[:q.shape[0], :q.shape[1]]


def test_moe_layer_vs_per_token_dense():
    """Grouped GEMM in expert-sorted order, bf16 outputs, combine through the
    routing positions == for every token, sum over its top-k experts of
    weight * (its own activation row times that expert's weights), computed
    per token without the grouped order (to half a bf16 ulp per term)."""
    moe = inputs.small_moe()
    r = moe["routing"]
    x = moe["x"]
    G = r.offsets.size - 1
    wd = moe["w_gu"][:, :128, :]                       # any [G, N, K] expert stack
    qx, sx = oracle.quant_1x128(x)
    wq, ws = zip(*(oracle.quant_128x128(wd[g]) for g in range(G)))
    wq, ws = np.stack(wq), np.stack(ws)
    y, _ = oracle.grouped_gemm_blockscaled(qx[r.row_token], sx[r.row_token], r.offsets, wq, ws)
    yb = oracle.f64_to_bf16(y)
    out = oracle.moe_combine(yb, r.token_rows, r.weights)

    A = _dequant(qx, sx, 1, 128)
    B = [_dequant(wq[g], ws[g], 128, 128) for g in range(G)]
    T, k = r.topk_experts.shape
    for t in range(0, T, 11):
        terms = [r.weights[t, j].astype(np.float64) * (B[r.topk_experts[t, j]] @ A[t]) for j in range(k)]
        ref = np.sum(terms, axis=0)
        tol = sum(np.abs(tm) for tm in terms) * 2.0 ** -8 + 1e-12
        assert np.all(np.abs(out[t] - ref) <= tol), t
    # a wrong position map (rows in token order) must fail the same check
    bad = oracle.moe_combine(yb, np.arange(T * k, dtype=np.int32).reshape(T, k), r.weights)
    assert not np.allclose(bad, out, rtol=1e-2, atol=1e-3)
