"""GPU parity of the block-scaled FP8 GEMMs against the fp64 oracle.

GEMM definition: C = sum over 128-wide K slices of the slice's scale product
times the FP32 partial of the slice ("Low Precision RL", sections "Unified
training recipe" and "2. Unified block-wise FP8 (DeepSeek-style)"), and the
MXFP8 variant with 1x32 UE8M0 scales (section "3. Unified MXFP8
(Blackwell)").  Tolerances: relative Frobenius error <= 1e-5 on FP32 outputs
and elementwise |y - yref| <= 1e-4 * sum_k |a_k b_k| (+ half an output ulp);
operands built from small integers and power-of-two scales are exact in any
summation order and must match bit for bit.  Every call goes through the C ABI.

gfx950's FP8 matrix instructions truncate, inside each aligned run of 8
products, every product to 13 bits below the run's largest one (measured;
see gpu_util.run_truncation).  Each result is therefore checked twice: against
the oracle within the stated tolerance plus that truncation bound, and against
the truncation model within the stated tolerance alone.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16, host, sample_indices, verify

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed, sigma=1.0, frac=0.0, mult=1.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def _linear_operands(x, w):
    """Quantize X (1x128, M-major scales) and W (128x128) on the GPU."""
    qa, sa = ops.quant_rowblock(dev_bf16(x), ops.AXIS_ROW, "m_major")
    qb, sb, _ = ops.quant_block2d(dev_bf16(w))
    return qa, sa, qb, sb


def _run_both(qa, sa, qb, sb, bscale=ops.BSCALE_BLOCK128):
    y16 = ops.gemm(qa, sa, qb, sb, bscale, torch.bfloat16)
    y32 = ops.gemm(qa, sa, qb, sb, bscale, torch.float32)
    torch.cuda.synchronize()
    return host(y16), host(y32)


def test_tiny_linear_forward():
    """256 tokens x 512 -> 512 with outliers: every output."""
    d = inputs.tiny_linear(0)
    qa, sa, qb, sb = _linear_operands(d["x"], d["w"])
    y16, y32 = _run_both(qa, sa, qb, sb)
    verify(host(qa), host(sa), host(qb), host(sb), y32, y16, record="tiny_linear")


@pytest.mark.parametrize("M,N,K", [(300, 384, 1024), (1, 128, 128), (513, 640, 384), (64, 256, 2048)])
def test_ragged_shapes(M, N, K):
    _say("ragged", M, N, K)
    x = _bits((M, K), 10 + M, 1.0, 0.01, 30.0)
    w = _bits((N, K), 20 + N, 0.02)
    qa, sa, qb, sb = _linear_operands(x, w)
    y16, y32 = _run_both(qa, sa, qb, sb)
    verify(host(qa), host(sa), host(qb), host(sb), y32, y16)


def _exact_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    ia = rng.integers(-8, 9, size=(M, K))
    ib = rng.integers(-8, 9, size=(N, K))
    ja = rng.integers(-1, 2, size=(M, K // 128))
    jb = rng.integers(-1, 2, size=(N // 128, K // 128))
    qa = oracle.e4m3_encode(ia.astype(np.float32))
    qb = oracle.e4m3_encode(ib.astype(np.float32))
    return qa, np.exp2(ja).astype(np.float32), qb, np.exp2(jb).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(300, 384, 1024), (256, 512, 8192)])
def test_exact_integer_case_bit_exact(M, N, K):
    qa, sa, qb, sb = _exact_case(M, N, K, M + K)
    yref, _ = oracle.gemm_blockscaled(qa, sa, qb, sb, with_abs=False)
    y16, y32 = _run_both(dev(qa), dev(sa), dev(qb), dev(sb))
    assert np.array_equal(y32.astype(np.float64), yref)
    assert np.array_equal(y16, oracle.f64_to_bf16(yref))


def _plan(M, N, K):
    (w1, n1), second, split = ops.fp8_blockscaled_gemm_plan(M, N, K)
    return ((w1, n1), second, split)


# Every tiling the dense planner chooses (the 256 x 256 tile serves grouped
# problems only), each on a shape that the planner routes to it: M not a
# multiple of the tile's rows, N not a multiple of its columns where the
# tiling allows, and the two-region plans.
PLAN_CASES = [
    ((1000, 10368, 384), ((4, 128), None, 10368)),
    ((1000, 8448, 384), ((8, 160), None, 8448)),
    ((1000, 6272, 384), ((4, 256), None, 6272)),
    ((130, 128, 384), ((4, 192), None, 128)),
    ((3200, 10112, 2048), ((4, 256), (4, 128), 5120)),
    ((2816, 9344, 4096), ((4, 128), (8, 160), 5760)),
    ((1664, 14464, 4096), ((8, 160), (4, 128), 5120)),
    ((4000, 2432, 6912), ((4, 160), None, 2432)),
]


@pytest.mark.parametrize("shape,plan", PLAN_CASES)
def test_exact_integer_case_every_tiling(shape, plan):
    """Sampled outputs plus every output in the last rows, the last columns and
    the columns around a region boundary, bit-exact."""
    M, N, K = shape
    assert _plan(M, N, K) == plan
    _say("tiling", shape, plan)
    qa, sa, qb, sb = _exact_case(M, N, K, M + N)
    y16, y32 = _run_both(dev(qa), dev(sa), dev(qb), dev(sb))
    mi, ni = sample_indices(M, N, 4000, 3)
    edge_cols = np.unique(np.concatenate([np.arange(N - 48, N), np.arange(max(plan[2] - 48, 0), min(plan[2] + 48, N))]))
    mi = np.concatenate([mi, np.repeat(np.arange(M - 4, M), N), np.repeat(np.arange(0, M, 7), edge_cols.size)])
    ni = np.concatenate([ni, np.tile(np.arange(N), 4), np.tile(edge_cols, (M + 6) // 7)])
    yref, _ = oracle.gemm_blockscaled_sampled(qa, sa, qb, sb, mi, ni)
    assert np.array_equal(y32[mi, ni].astype(np.float64), yref)
    assert np.array_equal(y16[mi, ni], oracle.f64_to_bf16(yref))


@pytest.mark.parametrize("shape,plan", PLAN_CASES)
def test_row_scale_modes_exact_every_tiling(shape, plan):
    """The modes with per-row weight scales on every planned tiling: ROW128
    (FP32 scales per weight row and 128-K slice, the wgrad GEMM) and dense
    MXFP8 (UE8M0 per row and 32-K block).  Power-of-two scales and small
    integer codes make every sum exact: sampled outputs, the last rows and
    columns and the columns around a region boundary, bit for bit."""
    M, N, K = shape
    _say("row-scale modes", shape, plan)
    rng = np.random.default_rng(M + 2 * N)
    qa = oracle.e4m3_encode(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    qb = oracle.e4m3_encode(rng.integers(-8, 9, size=(N, K)).astype(np.float32))
    sa = np.exp2(rng.integers(-1, 2, size=(M, K // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-1, 2, size=(N, K // 128))).astype(np.float32)
    ea = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    y_row = ops.gemm(dev(qa), dev(sa), dev(qb), dev(sb), ops.BSCALE_ROW128, torch.float32)
    y_mx = ops.mx_gemm(dev(qa), dev(ea), dev(qb), dev(eb))
    torch.cuda.synchronize()
    mi, ni = sample_indices(M, N, 4000, 4)
    edge_cols = np.unique(np.concatenate([np.arange(N - 48, N), np.arange(max(plan[2] - 48, 0), min(plan[2] + 48, N))]))
    mi = np.concatenate([mi, np.repeat(np.arange(M - 4, M), N), np.repeat(np.arange(0, M, 7), edge_cols.size)])
    ni = np.concatenate([ni, np.tile(np.arange(N), 4), np.tile(edge_cols, (M + 6) // 7)])
    yref, _ = oracle.gemm_blockscaled_sampled(qa, sa, qb, sb, mi, ni, oracle.BSCALE_ROW128)
    assert np.array_equal(host(y_row)[mi, ni].astype(np.float64), yref)
    yref, _ = oracle.gemm_mx_sampled(qa, ea, qb, eb, mi, ni)
    assert np.array_equal(host(y_mx)[mi, ni].astype(np.float64), yref)


@pytest.mark.parametrize("M,N,K", [(3000, 2688, 384), (1000, 1408, 384)])
def test_other_tilings_real_data(M, N, K):
    """Quantized N(0,1) activations with outliers and N(0, 0.02) weights on the
    160- and 192-row tilings: every output within tolerance."""
    _say("tiling real data", M, N, K, _plan(M, N, K))
    x = _bits((M, K), 50 + M, 1.0, 0.001, 100.0)
    w = _bits((N, K), 51 + N, 0.02)
    qa, sa, qb, sb = _linear_operands(x, w)
    y16, y32 = _run_both(qa, sa, qb, sb)
    verify(host(qa), host(sa), host(qb), host(sb), y32, y16)


def test_dgrad_through_transposed_weight_copy():
    """dX = dY W: dY [512, 1024] 1x128, W [1024 out, 384 in] 128x128; B is the
    transposed code copy with W's block scales read transposed."""
    dy = _bits((512, 1024), 30, 1e-3)
    w = _bits((1024, 384), 31, 0.02)
    qa, sa = ops.quant_rowblock(dev_bf16(dy), ops.AXIS_ROW, "m_major")
    qw, sw, qwt = ops.quant_block2d(dev_bf16(w), transposed=True)
    swt = sw.t()                                   # [in/128, out/128] view, strides swapped
    y32 = ops.gemm(qa, sa, qwt, swt, ops.BSCALE_BLOCK128, torch.float32)
    torch.cuda.synchronize()
    verify(host(qa), host(sa), np.ascontiguousarray(host(qw).T), np.ascontiguousarray(host(sw).T), host(y32))


def test_wgrad_row128():
    """dW = dY^T X with both operands re-quantized 128x1 along tokens."""
    T, O, I = 512, 256, 384
    dy = _bits((T, O), 40, 1e-3)
    x = _bits((T, I), 41, 1.0, 0.01, 30.0)
    qa, sa = ops.quant_rowblock(dev_bf16(dy), ops.AXIS_COL, "m_major")
    qb, sb = ops.quant_rowblock(dev_bf16(x), ops.AXIS_COL, "m_major")
    y32 = ops.gemm(qa, sa, qb, sb, ops.BSCALE_ROW128, torch.float32)
    torch.cuda.synchronize()
    verify(host(qa), host(sa), host(qb), host(sb), host(y32), bscale_row=True)


@pytest.mark.parametrize("part", ["up", "down"])
def test_qwen3_4b_mlp_full_size_sampled(part):
    d = inputs.qwen3_4b_mlp(1, parts=(part,))
    x, w = d["x_" + part], d["w_" + part]
    _say("full size", part, x.shape, w.shape)
    qa, sa, qb, sb = _linear_operands(x, w)
    y16, y32 = _run_both(qa, sa, qb, sb)
    M, N = y32.shape
    mi, ni = sample_indices(M, N, 3000, 7)
    verify(host(qa), host(sa), host(qb), host(sb), y32, y16, mi=mi, ni=ni, record="qwen3_4b_mlp_" + part)


def test_qwen3_4b_backward_full_size_sampled():
    """Backward GEMMs of the MLP up-projection at full size, FP32 outputs:
    dgrad dX = dY W (dY 1x128, W's transposed codes with its 128x128 block
    scales read transposed, no requantization) and wgrad dW = dY^T X (both
    requantized 128x1 along tokens from the bf16 originals)."""
    d = inputs.qwen3_4b_mlp_backward(2)
    dy, x, w = d["dy"], d["x"], d["w"]
    qdy, sdy = ops.quant_rowblock(dev_bf16(dy), ops.AXIS_ROW, "m_major")
    qw, sw, qwt = ops.quant_block2d(dev_bf16(w), transposed=True)
    dx = ops.gemm(qdy, sdy, qwt, sw.t(), ops.BSCALE_BLOCK128, torch.float32)
    torch.cuda.synchronize()
    _say("dgrad", tuple(dx.shape))
    mi, ni = sample_indices(dx.shape[0], dx.shape[1], 3000, 21)
    verify(host(qdy), host(sdy), np.ascontiguousarray(host(qw).T), np.ascontiguousarray(host(sw).T), host(dx),
           mi=mi, ni=ni, record="qwen3_4b_dgrad")
    del dx
    qa, sa = ops.quant_rowblock(dev_bf16(dy), ops.AXIS_COL, "m_major")
    qb, sb = ops.quant_rowblock(dev_bf16(x), ops.AXIS_COL, "m_major")
    dw = ops.gemm(qa, sa, qb, sb, ops.BSCALE_ROW128, torch.float32)
    torch.cuda.synchronize()
    _say("wgrad", tuple(dw.shape))
    mi, ni = sample_indices(dw.shape[0], dw.shape[1], 3000, 22)
    verify(host(qa), host(sa), host(qb), host(sb), host(dw), bscale_row=True, mi=mi, ni=ni, record="qwen3_4b_wgrad")


# ---------------------------------------------------------------- grouped
def _moe_operands(moe, part="gu"):
    r = moe["routing"]
    G = r.offsets.size - 1
    qx, sx = ops.quant_rowblock(dev_bf16(moe["x"]), ops.AXIS_ROW, "m_major")
    w = moe["w_gu"]
    qw, sw, _ = ops.quant_block2d(dev_bf16(w))
    return r, G, qx, sx, qw, sw


@pytest.mark.parametrize("gather", [True, False])
def test_grouped_small_moe_with_empty_groups(gather):
    moe = inputs.small_moe()
    r, G, qx, sx, qw, sw = _moe_operands(moe)
    assert np.any(np.diff(r.offsets) == 0)
    rows = r.row_token.size
    N, K = qw.shape[1], qw.shape[2]
    offs = dev(r.offsets)
    if gather:
        a, sa, a_rows, a_count = qx, sx, dev(r.row_token), qx.shape[0]
    else:
        idx = torch.from_numpy(r.row_token.astype(np.int64)).cuda()
        a, sa, a_rows, a_count = qx[idx].contiguous(), sx[idx].t().contiguous().t(), None, rows
    for out_dtype in (torch.float32, torch.bfloat16):
        c = torch.full((rows, N), float("nan"), dtype=out_dtype, device="cuda")
        ops.fp8_grouped_gemm(rows, N, K, G, offs, a_rows, a_count, a, a.stride(0), sa, sa.stride(0), sa.stride(1),
                             qw, qw.stride(1), qw.stride(0), sw, sw.stride(0), sw.stride(1), sw.stride(2), c,
                             c.stride(0), ops.OUT_FP32 if out_dtype == torch.float32 else ops.OUT_BF16)
        torch.cuda.synchronize()
        qa_h = host(qx)[r.row_token]
        sa_h = host(sx)[r.row_token]
        ch = host(c)
        for g in range(G):
            r0, r1 = int(r.offsets[g]), int(r.offsets[g + 1])
            if r1 > r0:
                if out_dtype == torch.float32:
                    verify(qa_h[r0:r1], sa_h[r0:r1], host(qw)[g], host(sw)[g], ch[r0:r1])
                else:
                    verify(qa_h[r0:r1], sa_h[r0:r1], host(qw)[g], host(sw)[g], None, ch[r0:r1])


def test_grouped_exact_integer_case():
    """Grouped GEMM on exact operands with ragged and empty groups: bit-exact."""
    rng = np.random.default_rng(8)
    counts = np.array([0, 300, 1, 0, 256, 513, 0, 40])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows, G, N, K = int(offsets[-1]), counts.size, 384, 512
    qa, sa, _, _ = _exact_case(rows, 128, K, 9)
    qbs, sbs = [], []
    for g in range(G):
        _, _, qb, sb = _exact_case(128, N, K, 100 + g)
        qbs.append(qb)
        sbs.append(sb)
    qb, sb = np.stack(qbs), np.stack(sbs)
    yref, _ = oracle.grouped_gemm_blockscaled(qa, sa, offsets, qb, sb)
    c = torch.zeros((rows, N), dtype=torch.float32, device="cuda")
    dqb, dsb = dev(qb), dev(sb)
    dsa = dev(sa)
    ops.fp8_grouped_gemm(rows, N, K, G, dev(offsets), None, rows, dev(qa), K, dsa, dsa.stride(0), dsa.stride(1),
                         dqb, K, N * K, dsb, dsb.stride(0), dsb.stride(1), dsb.stride(2), c, N, ops.OUT_FP32)
    torch.cuda.synchronize()
    assert np.array_equal(host(c).astype(np.float64), yref)


def test_grouped_exact_integer_case_many_groups():
    """More than 128 groups (the work-item lookup then walks the offsets in
    chunks of 128 groups), many of them empty: bit-exact."""
    rng = np.random.default_rng(12)
    G, N, K = 300, 256, 256
    counts = np.where(rng.random(G) < 0.3, 0, rng.integers(1, 300, G))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    qa, sa, _, _ = _exact_case(rows, 128, K, 13)
    qbs, sbs = [], []
    for g in range(G):
        _, _, qb, sb = _exact_case(128, N, K, 1000 + g)
        qbs.append(qb)
        sbs.append(sb)
    qb, sb = np.stack(qbs), np.stack(sbs)
    yref, _ = oracle.grouped_gemm_blockscaled(qa, sa, offsets, qb, sb)
    _say("grouped, %d groups, %d rows" % (G, rows))
    c = torch.zeros((rows, N), dtype=torch.float32, device="cuda")
    dsa, dqb, dsb = dev(sa), dev(qb), dev(sb)
    ops.fp8_grouped_gemm(rows, N, K, G, dev(offsets), None, rows, dev(qa), K, dsa, dsa.stride(0), dsa.stride(1),
                         dqb, K, N * K, dsb, dsb.stride(0), dsb.stride(1), dsb.stride(2), c, N, ops.OUT_FP32)
    torch.cuda.synchronize()
    assert np.array_equal(host(c).astype(np.float64), yref)


def _group_samples(offsets, N, seed, per_group=20):
    """Per non-empty group: its first and last 3 rows and `per_group` random
    rows, every column; returns {g: (local rows, local cols)}."""
    rng = np.random.default_rng(seed)
    out = {}
    for g in range(offsets.size - 1):
        n = int(offsets[g + 1] - offsets[g])
        if n == 0:
            continue
        rows = np.unique(np.concatenate([np.arange(min(3, n)), np.arange(max(0, n - 3), n),
                                         rng.integers(0, n, per_group)]))
        mi = np.repeat(rows, N)
        ni = np.tile(np.arange(N), rows.size)
        out[g] = (mi, ni)
    return out


GROUP_COUNTS_LARGE = np.array([0, 1500, 1, 0, 2300, 1777, 0, 2501])   # 256 x 256 tiles


def test_grouped_exact_integer_case_256x256_tiles():
    """Grouped GEMM large enough for the 256 x 256 tile configuration, ragged
    and empty groups, exact operands: sampled outputs bit-exact."""
    offsets = np.concatenate([[0], np.cumsum(GROUP_COUNTS_LARGE)]).astype(np.int32)
    rows, G, N, K = int(offsets[-1]), GROUP_COUNTS_LARGE.size, 1024, 256
    qa, sa, _, _ = _exact_case(rows, 128, K, 11)
    qbs, sbs = zip(*[_exact_case(128, N, K, 200 + g)[2:] for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    dqa, dsa, dqb, dsb, doffs = dev(qa), dev(sa), dev(qb), dev(sb), dev(offsets)

    def run(out):
        dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
        c = torch.full((rows, N), float("nan"), dtype=dt, device="cuda")
        ops.fp8_grouped_gemm(rows, N, K, G, doffs, None, rows, dqa, K, dsa, dsa.stride(0), dsa.stride(1),
                             dqb, K, N * K, dsb, dsb.stride(0), dsb.stride(1), dsb.stride(2), c, N, out)
        return c

    ch, ch16 = _twice_bitwise(run)
    for g, (mi, ni) in _group_samples(offsets, N, 12).items():
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        yref, _ = oracle.gemm_blockscaled_sampled(qa[r0:r1], sa[r0:r1], qb[g], sb[g], mi, ni)
        assert np.array_equal(ch[r0:r1][mi, ni].astype(np.float64), yref), "group %d" % g
    # bf16 output (staged through the two-region epilogue) equals the RNE
    # rounding of the exact fp32 output (single-region staging), everywhere
    assert np.array_equal(ch16, oracle.f64_to_bf16(ch.astype(np.float64)))


def test_grouped_exact_integer_case_256x256_tiles_many_groups():
    """The 256 x 256 persistent configuration with 200 groups (the work-item
    lookup walks the offsets in chunks of 128 groups), 30% of them empty and
    the rest ragged (each group's last row tile runs with its empty waves
    idle): sampled outputs of every group bit-exact, launches repeatable."""
    rng = np.random.default_rng(21)
    G, N, K = 200, 1024, 256
    counts = np.where(rng.random(G) < 0.3, 0, rng.integers(1, 600, G))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    qa, sa, _, _ = _exact_case(rows, 128, K, 22)
    qbs, sbs = zip(*[_exact_case(128, N, K, 3000 + g)[2:] for g in range(G)])
    qb, sb = np.stack(qbs), np.stack(sbs)
    dqa, dsa, dqb, dsb, doffs = dev(qa), dev(sa), dev(qb), dev(sb), dev(offsets)
    _say("grouped 256x256, %d groups, %d rows" % (G, rows))

    def run(out):
        dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
        c = torch.full((rows, N), float("nan"), dtype=dt, device="cuda")
        ops.fp8_grouped_gemm(rows, N, K, G, doffs, None, rows, dqa, K, dsa, dsa.stride(0), dsa.stride(1),
                             dqb, K, N * K, dsb, dsb.stride(0), dsb.stride(1), dsb.stride(2), c, N, out)
        return c

    ch, ch16 = _twice_bitwise(run)
    for g, (mi, ni) in _group_samples(offsets, N, 23, per_group=6).items():
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        yref, _ = oracle.gemm_blockscaled_sampled(qa[r0:r1], sa[r0:r1], qb[g], sb[g], mi, ni)
        assert np.array_equal(ch[r0:r1][mi, ni].astype(np.float64), yref), "group %d" % g
    assert np.array_equal(ch16, oracle.f64_to_bf16(ch.astype(np.float64)))


def _twice_bitwise(run):
    """Run a GEMM launcher twice per output type on the same inputs; the two
    results must be identical bytes (an LDS-pipeline race shows up as a
    difference).  Returns the host fp32 and bf16 results."""
    res = []
    for out in (ops.OUT_FP32, ops.OUT_BF16):
        c1 = run(out)
        c2 = run(out)
        torch.cuda.synchronize()
        h1, h2 = host(c1), host(c2)
        assert h1.tobytes() == h2.tobytes(), "second launch differs (%s)" % out
        res.append(h1)
    return res


def test_mx_grouped_exact_integer_case_256x256_tiles():
    """The same for the MX grouped GEMM: integer codes, UE8M0 scale codes
    126..128, sampled outputs bit-exact."""
    offsets = np.concatenate([[0], np.cumsum(GROUP_COUNTS_LARGE)]).astype(np.int32)
    rows, G, N, K = int(offsets[-1]), GROUP_COUNTS_LARGE.size, 1024, 256
    rng = np.random.default_rng(13)
    qa = oracle.e4m3_encode(rng.integers(-8, 9, size=(rows, K)).astype(np.float32))
    ea = rng.integers(126, 129, size=(rows, K // 32)).astype(np.uint8)
    qb = oracle.e4m3_encode(rng.integers(-8, 9, size=(G, N, K)).astype(np.float32))
    eb = rng.integers(126, 129, size=(G, N, K // 32)).astype(np.uint8)
    dqa, dea, dqb, deb, doffs = dev(qa), dev(ea), dev(qb), dev(eb), dev(offsets)

    def run(out):
        dt = torch.float32 if out == ops.OUT_FP32 else torch.bfloat16
        c = torch.full((rows, N), float("nan"), dtype=dt, device="cuda")
        ops.mxfp8_gemm(rows, N, K, G, doffs, None, rows, dqa, K, dea, K // 32, dqb, K, N * K,
                       deb, K // 32, N * (K // 32), c, N, out)
        return c

    ch, ch16 = _twice_bitwise(run)
    for g, (mi, ni) in _group_samples(offsets, N, 14).items():
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        yref, _ = oracle.gemm_mx_sampled(qa[r0:r1], ea[r0:r1], qb[g], eb[g], mi, ni)
        assert np.array_equal(ch[r0:r1][mi, ni].astype(np.float64), yref), "group %d" % g
    assert np.array_equal(ch16, oracle.f64_to_bf16(ch.astype(np.float64)))


# ---------------------------------------------------------------------- MX
def test_mx_dense_and_exact():
    M, N, K = 300, 384, 1024
    x = _bits((M, K), 50, 1.0, 0.02, 40.0)
    w = _bits((N, K), 51, 0.02)
    qa, sa = ops.mx_quant(dev_bf16(x))
    qb, sb = ops.mx_quant(dev_bf16(w))
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.mxfp8_gemm(M, N, K, 0, None, None, M, qa, K, sa, K // 32, qb, K, 0, sb, K // 32, 0, c, N, ops.OUT_FP32)
    torch.cuda.synchronize()
    verify(host(qa), host(sa), host(qb), host(sb), host(c), mx=True)
    # exact: integer codes and UE8M0 codes 126..128
    rng = np.random.default_rng(52)
    ia = oracle.e4m3_encode(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    ib = oracle.e4m3_encode(rng.integers(-8, 9, size=(N, K)).astype(np.float32))
    ea = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    yref, _ = oracle.gemm_mx(ia, ea, ib, eb)
    ops.mxfp8_gemm(M, N, K, 0, None, None, M, dev(ia), K, dev(ea), K // 32, dev(ib), K, 0, dev(eb), K // 32, 0,
                   c, N, ops.OUT_FP32)
    torch.cuda.synchronize()
    assert np.array_equal(host(c).astype(np.float64), yref)


def test_mx_grouped_small_moe():
    moe = inputs.small_moe()
    r = moe["routing"]
    G = r.offsets.size - 1
    rows = r.row_token.size
    qx, sx = ops.mx_quant(dev_bf16(moe["x"]))
    w = moe["w_gu"]
    Gw, N, K = w.shape
    qw, sw = ops.mx_quant(dev_bf16(w.reshape(Gw * N, K)))
    c = torch.empty((rows, N), dtype=torch.float32, device="cuda")
    ops.mxfp8_gemm(rows, N, K, G, dev(r.offsets), dev(r.row_token), qx.shape[0], qx, K, sx, K // 32, qw, K, N * K,
                   sw, K // 32, N * (K // 32), c, N, ops.OUT_FP32)
    torch.cuda.synchronize()
    qa_h, sa_h = host(qx)[r.row_token], host(sx)[r.row_token]
    qw_h, sw_h = host(qw).reshape(Gw, N, K), host(sw).reshape(Gw, N, K // 32)
    ch = host(c)
    for g in range(G):
        r0, r1 = int(r.offsets[g]), int(r.offsets[g + 1])
        if r1 > r0:
            verify(qa_h[r0:r1], sa_h[r0:r1], qw_h[g], sw_h[g], ch[r0:r1], mx=True)


# ------------------------------------------------------- MXFP8 backward
@pytest.mark.parametrize("shape", [(256, 512), (96, 264), (32, 8), (4096, 2560), (9728, 2560), (4192, 4040)])
def test_mx_quant_t_bit_exact(shape):
    """32x1 MX blocks down each column, written transposed: codes and scale
    bytes equal the oracle's 1x32 quantization of the transpose (partial
    128-row and 64-column tiles included; (9728, 2560) and (4192, 4040) take
    the register kernel, the others the LDS kernel)."""
    _say("mx_quant_t", shape)
    x = _bits(shape, 60, 1.0, 0.01, 50.0)
    if shape[0] >= 64 and shape[1] >= 3:
        x[:32, 0] = 0                                   # an all-zero block
        x[32:64, 1] = inputs.to_bf16_bits(np.full(32, 3e38, np.float32))
        x[:32, 2] = inputs.to_bf16_bits((np.arange(32) * 1e-39).astype(np.float32))
    qt, s = ops.mx_quant_t(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr = oracle.mx_quant_32x1_t(x)
    assert np.array_equal(host(qt), qr)
    assert np.array_equal(host(s), sr)


def test_mx_backward_full_size_sampled():
    """MXFP8 backward of the MLP up-projection at full size, FP32 outputs:
    dgrad dX = dY W with dY 1x32 along O and W re-quantized 32x1 along O;
    wgrad dW = dY^T X with both re-quantized 32x1 along tokens."""
    d = inputs.qwen3_4b_mlp_backward(2)
    dy, x, w = d["dy"], d["x"], d["w"]
    qdy, sdy = ops.mx_quant(dev_bf16(dy))
    qwt, swt = ops.mx_quant_t(dev_bf16(w))
    dx = ops.mx_gemm(qdy, sdy, qwt, swt)
    torch.cuda.synchronize()
    rows = np.random.default_rng(23).integers(0, w.shape[1], 64)
    qr, sr = oracle.mx_quant_1x32(np.ascontiguousarray(w.T[rows]))
    assert np.array_equal(host(qwt)[rows], qr) and np.array_equal(host(swt)[rows], sr)
    _say("mx dgrad", tuple(dx.shape))
    mi, ni = sample_indices(dx.shape[0], dx.shape[1], 3000, 24)
    verify(host(qdy), host(sdy), host(qwt), host(swt), host(dx), mi=mi, ni=ni, mx=True, record="qwen3_4b_mx_dgrad")
    del dx
    qa, sa = ops.mx_quant_t(dev_bf16(dy))
    qb, sb = ops.mx_quant_t(dev_bf16(x))
    dw = ops.mx_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rows = np.random.default_rng(25).integers(0, dy.shape[1], 64)
    qr, sr = oracle.mx_quant_1x32(np.ascontiguousarray(dy.T[rows]))
    assert np.array_equal(host(qa)[rows], qr) and np.array_equal(host(sa)[rows], sr)
    _say("mx wgrad", tuple(dw.shape))
    mi, ni = sample_indices(dw.shape[0], dw.shape[1], 3000, 26)
    verify(host(qa), host(sa), host(qb), host(sb), host(dw), mi=mi, ni=ni, mx=True, record="qwen3_4b_mx_wgrad")


def test_mx_quant_t_rejects_bad_shapes():
    x = dev_bf16(_bits((48, 64), 61))
    qt = torch.empty((64, 48), dtype=torch.uint8, device="cuda")
    s = torch.empty((64, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.Fp8bsError):
        ops.mxfp8_quant_t(x, 48, 64, 64, qt, 48, s, 2, 1)       # rows % 32
    with pytest.raises(ops.Fp8bsError):
        ops.mxfp8_quant_t(x, 32, 64, 64, qt, 40, s, 2, 1)       # ld_qt % 16
