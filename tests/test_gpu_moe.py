"""GPU parity of the full-size MoE chains against the oracle (Qwen3-30B-A3B
shapes: 16384 tokens, hidden 2048, 128 experts, intermediate 768, top-8).

Block-wise FP8 chain ("Low Precision RL", section "2. Unified block-wise FP8
(DeepSeek-style)"): X 1x128 -> gather by expert -> grouped gate_up GEMM with
128x128-block weights -> h = bf16(silu(gate) * up) -> 1x128 requantization
-> grouped down GEMM.  MXFP8 chain (section "3. Unified MXFP8 (Blackwell)"):
the same with 1x32 UE8M0 scales on both operands.

Every stage is checked on the device's own inputs to that stage (stage-wise
parity): quantizer codes and scales bit-exact on sampled rows and experts,
h = bf16(silu(gate) * up) and its requantization bit-exact against the
oracle's fp64 h and the oracle's quantization of it, and each GEMM on
sampled outputs of sampled groups against the fp64 oracle and the datapath
truncation model.

The combine that closes the layer (each token's output = routing-weighted sum
of its experts' down-projection rows) is checked on sampled tokens of the
chain, and on its own at full size on seeded synthetic expert outputs and on
edge shapes, against the oracle's fp64 sum: the device's fp32 FMA chain over
k slots is within k * 2^-24 * sum_j |w_j y_j| of it, plus half a bf16 ulp for
bf16 output.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16, host, verify

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

HID, INTER, E = 2048, 768, 128


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def moe():
    _say("generating the MoE layer inputs (seed 3)")
    d = inputs.qwen3_30b_a3b_moe(3)
    d["routing_skewed"] = inputs.qwen3_30b_a3b_moe(3, skewed=True, weights=False)["routing"]
    _say("done")
    return d


def _sample_groups(offsets, seed, n_groups=8):
    """Sampled non-empty groups (always the first and last non-empty ones and
    the largest) with sampled local rows and columns of each."""
    rng = np.random.default_rng(seed)
    sizes = np.diff(offsets)
    ne = np.flatnonzero(sizes > 0)
    pick = set([int(ne[0]), int(ne[-1]), int(ne[np.argmax(sizes[ne])])])
    pick |= set(int(g) for g in rng.choice(ne, size=min(n_groups, ne.size), replace=False))
    return sorted(pick)


def _sample_rc(n_rows, n_cols, rng):
    rows = np.unique(np.concatenate([[0, 1], [n_rows - 2, n_rows - 1], rng.integers(0, n_rows, 8)]))
    rows = rows[(rows >= 0) & (rows < n_rows)]
    cols = np.unique(np.concatenate([np.arange(0, n_cols, 256), np.arange(255, n_cols, 256),
                                     rng.integers(0, n_cols, 64)]))
    mi = np.repeat(rows, cols.size)
    ni = np.tile(cols, rows.size)
    return rows, cols, mi, ni


def _check_grouped(offsets, groups, seed, c16, c32, operands, mx=False, record=None):
    """Verify sampled outputs of the grouped GEMM.  operands(g, r0, r1) gives
    the host (qa, sa, qb, sb) of group g's rows [r0, r1)."""
    rng = np.random.default_rng(seed)
    for g in groups:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        N = c32.shape[1]
        rows, cols, mi, ni = _sample_rc(r1 - r0, N, rng)
        qa, sa, qb, sb = operands(g, r0, r1)
        y32 = np.zeros((r1 - r0, N), np.float32)
        y16 = np.zeros((r1 - r0, N), np.uint16)
        y32[rows] = host(c32[r0 + torch.from_numpy(rows).cuda()])
        y16[rows] = host(c16[r0 + torch.from_numpy(rows).cuda()])
        _say("group %d: %d rows" % (g, r1 - r0))
        verify(qa, sa, qb, sb, y32, y16, mi=mi, ni=ni, mx=mx,
               record=None if record is None else "%s_group%d" % (record, g))


def _check_rows_quant_1x128(x_bits, q, s, rows):
    qr, sr = oracle.quant_1x128(x_bits[rows])
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(q[idx]), qr)
    assert np.array_equal(host(s[idx].contiguous()).view(np.uint32), sr.view(np.uint32))


def _check_rows_mx(x_bits, q, s, rows):
    qr, sr = oracle.mx_quant_1x32(x_bits[rows])
    idx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(q[idx]), qr)
    assert np.array_equal(host(s[idx]), sr)


def _check_h(gate_up, h, qh, sh, rows, mx):
    """h = bf16(silu(g) * u) bit-exact against the oracle's fp64 evaluation,
    and the requantization of h bit-exact against the oracle's quantization
    of the oracle's h (the whole chain after the gate/up GEMM)."""
    idx = torch.from_numpy(rows).cuda()
    gu = host(gate_up[idx])
    hg = host(h[idx])
    hr = oracle.silu_mul(gu)
    assert np.array_equal(hg, hr), "h differs from the oracle at %s" % (np.argwhere(hg != hr)[:5],)
    if mx:
        qr, sr = oracle.mx_quant_1x32(hr)
        assert np.array_equal(host(qh[idx]), qr)
        assert np.array_equal(host(sh[idx]), sr)
    else:
        qr, sr = oracle.quant_1x128(hr)
        assert np.array_equal(host(qh[idx]), qr)
        assert np.array_equal(host(sh[idx].contiguous()).view(np.uint32), sr.view(np.uint32))


def _check_combine(y_bits, pos, w, out32, out16):
    """y_bits: host bf16 rows, pos/w: host [T, k]; out32 / out16: host device
    results for those T tokens."""
    ref = oracle.moe_combine(y_bits, pos, w)
    mag = oracle.moe_combine(y_bits & np.uint16(0x7FFF), pos, np.abs(w))
    k = pos.shape[1]
    chain = k * 2.0 ** -24 * mag + 1e-30
    if out32 is not None:
        err = np.abs(out32.astype(np.float64) - ref)
        assert np.all(err <= chain), "fp32 combine: worst ratio %.3g" % np.max(err / chain)
    if out16 is not None:
        y = oracle.bf16_to_f32(out16).astype(np.float64)
        half = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(ref), np.abs(y)), 2.0 ** -126))) - 7)
        err = np.abs(y - ref)
        assert np.all(err <= chain + half), "bf16 combine: worst ratio %.3g" % np.max(err / (chain + half))


def _grouped(rows, N, K, G, offs, a_rows, a_count, a, sa, b, sb, out_dtype):
    c = torch.empty((rows, N), dtype=out_dtype, device="cuda")
    ops.fp8_grouped_gemm(rows, N, K, G, offs, a_rows, a_count, a, a.stride(0), sa, sa.stride(0), sa.stride(1),
                         b, b.stride(1), b.stride(0), sb, sb.stride(0), sb.stride(1), sb.stride(2), c, c.stride(0),
                         ops.OUT_FP32 if out_dtype == torch.float32 else ops.OUT_BF16)
    return c


def _blockwise_weights(d):
    wgu = dev_bf16(d["w_gu"])
    qgu, sgu, _ = ops.quant_block2d(wgu)
    del wgu
    wd = dev_bf16(d["w_d"])
    qd, sd, qdt = ops.quant_block2d(wd, transposed=True)
    del wd
    torch.cuda.synchronize()
    for e in (0, 77, E - 1):
        qr, sr = oracle.quant_128x128(d["w_gu"][e])
        assert np.array_equal(host(qgu[e]), qr) and np.array_equal(host(sgu[e]), sr), "W_gu expert %d" % e
        qr, sr = oracle.quant_128x128(d["w_d"][e])
        assert np.array_equal(host(qd[e]), qr) and np.array_equal(host(sd[e]), sr), "W_d expert %d" % e
        assert np.array_equal(host(qdt[e]), qr.T), "W_d transposed copy, expert %d" % e
    # down GEMM operand: B[n = hidden, k = inter] = W_d[e]^T codes, scales read transposed
    return qgu, sgu, qdt, sd.transpose(1, 2)


def _blockwise_chain(d, routing, seed, check_down=True, weights=None, name=None):
    r = routing
    rows, G = r.row_token.size, r.offsets.size - 1
    offs = dev(r.offsets)
    x = dev_bf16(d["x"])
    qx, sx = ops.quant_rowblock(x, ops.AXIS_ROW, "m_major")
    torch.cuda.synchronize()
    _check_rows_quant_1x128(d["x"], qx, sx, np.random.default_rng(seed).integers(0, x.shape[0], 64))
    qgu, sgu, qdt, sdt = weights
    a_rows = dev(r.row_token)
    _say("gate_up: %d rows, G=%d" % (rows, G))
    gu16 = _grouped(rows, 2 * INTER, HID, G, offs, a_rows, x.shape[0], qx, sx, qgu, sgu, torch.bfloat16)
    gu32 = _grouped(rows, 2 * INTER, HID, G, offs, a_rows, x.shape[0], qx, sx, qgu, sgu, torch.float32)
    torch.cuda.synchronize()
    groups = _sample_groups(r.offsets, seed)
    qx_h, sx_h = host(qx), host(sx)
    _check_grouped(r.offsets, groups, seed + 1, gu16, gu32,
                   lambda g, r0, r1: (qx_h[r.row_token[r0:r1]], sx_h[r.row_token[r0:r1]], host(qgu[g]), host(sgu[g])),
                   record=name and name + "_gate_up")
    del gu32
    if not check_down:
        return
    qh = torch.empty((rows, INTER), dtype=torch.uint8, device="cuda")
    shb = torch.empty((INTER // 128, rows), dtype=torch.float32, device="cuda")
    sh = shb.t()
    h = torch.empty((rows, INTER), dtype=torch.bfloat16, device="cuda")
    ops.fp8_silu_mul_quant(gu16, rows, INTER, 2 * INTER, 0, qh, INTER, sh, 1, rows, h, INTER)
    torch.cuda.synchronize()
    _check_h(gu16, h, qh, sh, np.random.default_rng(seed + 2).integers(0, rows, 256), mx=False)
    _fused_gate_up_matches(rows, G, offs, a_rows, x.shape[0], qx, sx, qgu, sgu, qh, shb)
    _say("down")
    dn16 = _grouped(rows, HID, INTER, G, offs, None, rows, qh, sh, qdt, sdt, torch.bfloat16)
    dn32 = _grouped(rows, HID, INTER, G, offs, None, rows, qh, sh, qdt, sdt, torch.float32)
    torch.cuda.synchronize()
    qh_h, sh_h = host(qh), host(sh)
    _check_grouped(r.offsets, groups, seed + 3, dn16, dn32,
                   lambda g, r0, r1: (qh_h[r0:r1], sh_h[r0:r1], host(qdt[g]), host(sdt[g])),
                   record=name and name + "_down")
    del dn32
    _say("combine")
    T = r.token_rows.shape[0]
    pos_d, w_d = dev(r.token_rows), dev(r.weights)
    out16 = ops.moe_combine(dn16, pos_d, w_d, torch.bfloat16)
    out32 = ops.moe_combine(dn16, pos_d, w_d, torch.float32)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(seed + 4).integers(0, T, 256)]))
    pos = r.token_rows[toks]
    yrows = host(dn16[torch.from_numpy(pos.reshape(-1).astype(np.int64)).cuda()])
    local = np.arange(pos.size, dtype=np.int32).reshape(pos.shape)
    tidx = torch.from_numpy(toks).cuda()
    _check_combine(yrows, local, r.weights[toks], host(out32[tidx]), host(out16[tidx]))


def _fused_gate_up_matches(rows, G, offs, a_rows, a_count, qx, sx, qgu, sgu, qh, shb):
    """The gate/up GEMM with SiLU*mul and the 1x128 quantization of h in its
    epilogue: codes and (M-major) scales byte-identical to the bf16 grouped
    GEMM followed by fp8_silu_mul_quant; every row, including the last rows
    of every group."""
    I, K = qgu.shape[1] // 2, qgu.shape[2]
    _say("gate_up with SiLU*mul and 1x128 quantization in the epilogue: %d rows, G=%d" % (rows, G))
    qhf = torch.full((rows, I), 0xAA, dtype=torch.uint8, device="cuda")
    shf = torch.full((I // 128, rows), -1.0, dtype=torch.float32, device="cuda")
    ops.fp8_grouped_gemm_swiglu_quant(rows, I, K, G, offs, a_rows, a_count, qx, qx.stride(0), sx, sx.stride(0),
                                      sx.stride(1), qgu, qgu.stride(1), qgu.stride(0), sgu, sgu.stride(0),
                                      sgu.stride(1), sgu.stride(2), qhf, I, shf, 1, rows)
    torch.cuda.synchronize()
    bad = torch.nonzero(qhf != qh)
    assert bad.numel() == 0, "fused h codes differ at %s" % bad[:5].tolist()
    assert torch.equal(shf.view(torch.int32), shb.view(torch.int32)), "fused h scales differ"


def _fused_mx_gate_up_matches(rows, G, offs, a_rows, a_count, qx, sx, qgu, sgu, qh, sh):
    """The MXFP8 gate/up GEMM with SiLU*mul and the 1x32 quantization of h in
    its epilogue: codes and UE8M0 scales byte-identical to the bf16 grouped
    MXFP8 GEMM followed by fp8_silu_mul_quant(mx = 1), every row."""
    E_, N2, K = qgu.shape
    I = N2 // 2
    _say("MXFP8 gate_up with SiLU*mul and 1x32 quantization in the epilogue: %d rows, G=%d" % (rows, G))
    qhf = torch.full((rows, I), 0xAA, dtype=torch.uint8, device="cuda")
    shf = torch.full((rows, I // 32), 0xAA, dtype=torch.uint8, device="cuda")
    ops.mxfp8_grouped_gemm_swiglu_quant(rows, I, K, G, offs, a_rows, a_count, qx, K, sx, K // 32, qgu, K, N2 * K,
                                        sgu, K // 32, N2 * (K // 32), qhf, I, shf, I // 32, 1)
    torch.cuda.synchronize()
    bad = torch.nonzero(qhf != qh)
    assert bad.numel() == 0, "fused MX h codes differ at %s" % bad[:5].tolist()
    assert torch.equal(shf, sh), "fused MX h scales differ"


def test_mx_gate_up_swiglu_quant_small_moe():
    """The MXFP8 fused gate/up epilogue on the scaled-down MoE layer with
    empty experts and the dispatch gather."""
    d = inputs.small_moe()
    r = d["routing"]
    rows, G = r.row_token.size, r.offsets.size - 1
    E_, N2, K = d["w_gu"].shape
    I = N2 // 2
    qx, sx = ops.mx_quant(dev_bf16(d["x"]))
    qgu, sgu = ops.mx_quant(dev_bf16(d["w_gu"]).view(E_ * N2, K))
    offs, a_rows = dev(r.offsets), dev(r.row_token)
    gu16 = torch.empty((rows, N2), dtype=torch.bfloat16, device="cuda")
    ops.mxfp8_gemm(rows, N2, K, G, offs, a_rows, qx.shape[0], qx, K, sx, K // 32, qgu, K, N2 * K, sgu, K // 32,
                   N2 * (K // 32), gu16, N2, ops.OUT_BF16)
    qh = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    sh = torch.empty((rows, I // 32), dtype=torch.uint8, device="cuda")
    ops.fp8_silu_mul_quant(gu16, rows, I, N2, 1, qh, I, sh, I // 32, 1, None, 0)
    torch.cuda.synchronize()
    _fused_mx_gate_up_matches(rows, G, offs, a_rows, qx.shape[0], qx, sx, qgu.view(E_, N2, K),
                              sgu.view(E_, N2, K // 32), qh, sh)


@pytest.mark.parametrize("gather", [True, False])
def test_gate_up_swiglu_quant_small_moe(gather):
    """The fused gate/up epilogue on the scaled-down MoE layer with empty
    experts, with the dispatch gather of X rows and with pre-gathered rows."""
    d = inputs.small_moe()
    r = d["routing"]
    rows, G = r.row_token.size, r.offsets.size - 1
    assert np.any(np.diff(r.offsets) == 0)
    qx, sx = ops.quant_rowblock(dev_bf16(d["x"]), ops.AXIS_ROW, "m_major")
    qgu, sgu, _ = ops.quant_block2d(dev_bf16(d["w_gu"]))
    offs = dev(r.offsets)
    I = qgu.shape[1] // 2
    if gather:
        a, sa, a_rows, a_count = qx, sx, dev(r.row_token), qx.shape[0]
    else:
        idx = torch.from_numpy(r.row_token.astype(np.int64)).cuda()
        a, sa, a_rows, a_count = qx[idx].contiguous(), sx[idx].t().contiguous().t(), None, rows
    gu16 = _grouped(rows, 2 * I, qgu.shape[2], G, offs, a_rows, a_count, a, sa, qgu, sgu, torch.bfloat16)
    qh = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
    shb = torch.empty((I // 128, rows), dtype=torch.float32, device="cuda")
    ops.fp8_silu_mul_quant(gu16, rows, I, 2 * I, 0, qh, I, shb.t(), 1, rows, None, 0)
    torch.cuda.synchronize()
    _fused_gate_up_matches(rows, G, offs, a_rows, a_count, a, sa, qgu, sgu, qh, shb)


@pytest.fixture(scope="module")
def blockwise_weights(moe):
    return _blockwise_weights(moe)


def test_moe_blockwise_chain_full_size(moe, blockwise_weights):
    r = moe["routing"]
    assert r.row_token.size == 16384 * 8
    _blockwise_chain(moe, r, 30, weights=blockwise_weights, name="moe_blockwise")


def test_moe_blockwise_chain_skewed_routing(moe, blockwise_weights):
    """The parity-only skewed routing: 8 empty experts and group sizes from
    tens to thousands, not multiples of 128."""
    r = moe["routing_skewed"]
    sizes = np.diff(r.offsets)
    assert np.sum(sizes == 0) == 8 and np.any(sizes % 128 != 0)
    _blockwise_chain(moe, r, 40, check_down=True, weights=blockwise_weights, name="moe_blockwise_skewed")


@pytest.fixture(scope="module")
def mx_weights(moe):
    """The MoE layer's expert weights in 1x32 MX blocks along K (gate/up by
    rows of W_gu, down through its transpose), rows of the first and last
    expert checked bit-exact."""
    d = moe
    wgu = dev_bf16(d["w_gu"])
    qgu, sgu = ops.mx_quant(wgu.view(E * 2 * INTER, HID))
    del wgu
    wdt = dev_bf16(d["w_d"]).transpose(1, 2).contiguous()          # [E, hidden, inter]
    qdt, sdt = ops.mx_quant(wdt.view(E * HID, INTER))
    torch.cuda.synchronize()
    for e in (0, E - 1):
        _check_rows_mx(d["w_gu"].reshape(E * 2 * INTER, HID), qgu, sgu, np.arange(e * 2 * INTER, (e + 1) * 2 * INTER))
        _check_rows_mx(np.ascontiguousarray(d["w_d"][e].T), qdt[e * HID:(e + 1) * HID], sdt[e * HID:(e + 1) * HID],
                       np.arange(HID))
    del wdt
    return {"qgu": qgu, "sgu": sgu, "qdt": qdt, "sdt": sdt}


def _mx_chain(d, r, mxw, seed, name):
    rows, G = r.row_token.size, r.offsets.size - 1
    offs = dev(r.offsets)
    qgu, sgu, qdt, sdt = mxw["qgu"], mxw["sgu"], mxw["qdt"], mxw["sdt"]
    x = dev_bf16(d["x"])
    qx, sx = ops.mx_quant(x)
    torch.cuda.synchronize()
    _check_rows_mx(d["x"], qx, sx, np.random.default_rng(seed).integers(0, x.shape[0], 64))

    def mx_grouped(N, K, a_rows, a_count, a, sa, b, sb, out_dtype):
        c = torch.empty((rows, N), dtype=out_dtype, device="cuda")
        ops.mxfp8_gemm(rows, N, K, G, offs, a_rows, a_count, a, K, sa, K // 32, b, K, N * K, sb, K // 32,
                       N * (K // 32), c, N, ops.OUT_FP32 if out_dtype == torch.float32 else ops.OUT_BF16)
        return c

    a_rows = dev(r.row_token)
    gu16 = mx_grouped(2 * INTER, HID, a_rows, x.shape[0], qx, sx, qgu, sgu, torch.bfloat16)
    gu32 = mx_grouped(2 * INTER, HID, a_rows, x.shape[0], qx, sx, qgu, sgu, torch.float32)
    torch.cuda.synchronize()
    groups = _sample_groups(r.offsets, seed + 1)
    qx_h, sx_h = host(qx), host(sx)
    n_gu = 2 * INTER
    _check_grouped(r.offsets, groups, seed + 2, gu16, gu32,
                   lambda g, r0, r1: (qx_h[r.row_token[r0:r1]], sx_h[r.row_token[r0:r1]],
                                      host(qgu[g * n_gu:(g + 1) * n_gu]), host(sgu[g * n_gu:(g + 1) * n_gu])),
                   mx=True, record=name + "_gate_up")
    del gu32
    qh = torch.empty((rows, INTER), dtype=torch.uint8, device="cuda")
    sh = torch.empty((rows, INTER // 32), dtype=torch.uint8, device="cuda")
    h = torch.empty((rows, INTER), dtype=torch.bfloat16, device="cuda")
    ops.fp8_silu_mul_quant(gu16, rows, INTER, 2 * INTER, 1, qh, INTER, sh, INTER // 32, 1, h, INTER)
    torch.cuda.synchronize()
    _check_h(gu16, h, qh, sh, np.random.default_rng(seed + 3).integers(0, rows, 256), mx=True)
    _fused_mx_gate_up_matches(rows, G, offs, a_rows, x.shape[0], qx, sx, qgu.view(E, 2 * INTER, HID),
                              sgu.view(E, 2 * INTER, HID // 32), qh, sh)
    dn16 = mx_grouped(HID, INTER, None, rows, qh, sh, qdt, sdt, torch.bfloat16)
    dn32 = mx_grouped(HID, INTER, None, rows, qh, sh, qdt, sdt, torch.float32)
    torch.cuda.synchronize()
    qh_h, sh_h = host(qh), host(sh)
    _check_grouped(r.offsets, groups, seed + 4, dn16, dn32,
                   lambda g, r0, r1: (qh_h[r0:r1], sh_h[r0:r1], host(qdt[g * HID:(g + 1) * HID]),
                                      host(sdt[g * HID:(g + 1) * HID])),
                   mx=True, record=name + "_down")


def test_moe_mxfp8_chain_full_size(moe, mx_weights):
    _mx_chain(moe, moe["routing"], mx_weights, 50, "moe_mxfp8")


def test_moe_mxfp8_chain_skewed_routing(moe, mx_weights):
    """The MXFP8 chain on the parity-only skewed routing (8 empty experts,
    group sizes from tens to thousands, not multiples of 128)."""
    r = moe["routing_skewed"]
    sizes = np.diff(r.offsets)
    assert np.sum(sizes == 0) == 8 and np.any(sizes % 128 != 0)
    _mx_chain(moe, r, mx_weights, 60, "moe_mxfp8_skewed")


# ------------------------------------------------------------------ combine
def test_moe_combine_full_size_synthetic(moe):
    """The full-size combine (16384 tokens x 2048, top-8 over 131072 grouped
    rows) on seeded synthetic expert outputs, every output."""
    r = moe["routing"]
    rows, (T, k) = r.row_token.size, r.token_rows.shape
    _say("synthetic expert outputs %d x %d" % (rows, HID))
    y = inputs.normal_bf16(np.random.default_rng(50), (rows, HID), 0.05, 0.001, 20.0)
    yd = dev_bf16(y)
    pos_d, w_d = dev(r.token_rows), dev(r.weights)
    out16 = ops.moe_combine(yd, pos_d, w_d, torch.bfloat16)
    out32 = ops.moe_combine(yd, pos_d, w_d, torch.float32)
    torch.cuda.synchronize()
    _say("checking")
    _check_combine(y, r.token_rows, r.weights, host(out32), host(out16))


@pytest.mark.parametrize("T,k,H,rows", [(1, 1, 8, 1), (5, 3, 264, 9), (37, 9, 128, 50), (64, 16, 2048, 300),
                                        (300, 8, 776, 2400)])
def test_moe_combine_shapes(T, k, H, rows):
    """k below, at and above the 8-slot load batch; H not a multiple of the
    workgroup's 256 chunks; repeated rows; negative weights; a row stride
    larger than H."""
    _say("combine", T, k, H, rows)
    rng = np.random.default_rng(T + k + H)
    ld = H + 16
    y = inputs.normal_bf16(rng, (rows, ld), 1.0)
    pos = rng.integers(0, rows, (T, k)).astype(np.int32)
    w = rng.standard_normal((T, k)).astype(np.float32)
    yd = dev_bf16(y)
    out32 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out16 = torch.empty((T, H + 8), dtype=torch.bfloat16, device="cuda")
    ops.fp8_moe_combine(yd, rows, H, ld, dev(pos), dev(w), T, k, out32, H, ops.OUT_FP32)
    ops.fp8_moe_combine(yd, rows, H, ld, dev(pos), dev(w), T, k, out16, H + 8, ops.OUT_BF16)
    torch.cuda.synchronize()
    _check_combine(np.ascontiguousarray(y[:, :H]), pos, w, host(out32), host(out16)[:, :H])


def test_moe_combine_clamps_positions_and_rejects_bad_shapes():
    rng = np.random.default_rng(7)
    y = inputs.normal_bf16(rng, (10, 64), 1.0)
    pos = np.array([[-5, 3], [12, 9]], np.int32)
    w = np.array([[0.5, 0.25], [1.0, -2.0]], np.float32)
    out = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    ops.fp8_moe_combine(dev_bf16(y), 10, 64, 64, dev(pos), dev(w), 2, 2, out, 64, ops.OUT_FP32)
    torch.cuda.synchronize()
    _check_combine(y, np.clip(pos, 0, 9), w, host(out), None)
    empty = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    ops.fp8_moe_combine(dev_bf16(y), 10, 64, 64, None, None, 0, 2, empty, 64, ops.OUT_FP32)
    for args in ((10, 60, 64), (0, 64, 64), (10, 64, 56)):          # H % 8, no rows, ld_y < H
        with pytest.raises(ops.Fp8bsError):
            ops.fp8_moe_combine(dev_bf16(y), args[0], args[1], args[2], dev(pos), dev(w), 2, 2, out, 64,
                                ops.OUT_FP32)
