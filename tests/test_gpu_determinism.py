"""Run-to-run determinism of the GEMMs (a race in the LDS pipeline, the
persistent work loop or the staged epilogue would show up as two launches on
identical inputs giving different bytes).  Each planned dense tiling, the
per-row and K-invariant scale modes, power-of-two and MXFP8, the persistent
grouped GEMMs and both fused SiLU*mul epilogues run twice on the same
operands; the outputs must be byte-identical.  The operands are ordinary
quantized random data (not exact cases), so every output bit depends on the
order of the accumulation; both launches must take the same one.  The
K-invariant ("scales constant along K") reading and everything else about the
results are covered by the parity tests."""
import numpy as np
import pytest
import torch

from fp8_block_scaled_x128_amd import inputs, ops
from gpu_util import dev, dev_bf16
from test_gpu_gemm import PLAN_CASES

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(shape, seed, sigma=1.0, frac=0.0, mult=1.0):
    return inputs.normal_bf16(np.random.default_rng(seed), shape, sigma, frac, mult)


def _same_twice(run, what):
    a = run()
    b = run()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "%s: second launch differs" % what


def _dense_operands(M, N, K, seed):
    x = dev_bf16(_bits((M, K), seed, 1.0, 0.01, 30.0))
    w = dev_bf16(_bits((N, K), seed + 1, 0.02))
    qa, sa = ops.quant_rowblock(x, ops.AXIS_ROW, "m_major")
    qb, sb, _ = ops.quant_block2d(w)
    return x, w, qa, sa, qb, sb


@pytest.mark.parametrize("shape,plan", PLAN_CASES)
def test_dense_tilings_deterministic(shape, plan):
    M, N, K = shape
    _say("determinism, tiling", shape, plan)
    x, w, qa, sa, qb, sb = _dense_operands(M, N, K, M + N)
    for dt in (torch.bfloat16, torch.float32):
        _same_twice(lambda: ops.gemm(qa, sa, qb, sb, ops.BSCALE_BLOCK128, dt), "BLOCK128 %s" % dt)


def test_dense_other_modes_deterministic():
    M, N, K = 1000, 8448, 384          # the 160-row tiling with its two-block weight scales
    x, w, qa, sa, qb, sb = _dense_operands(M, N, K, 5)
    _say("determinism, ROW128 / K-invariant / pow2 / MX")
    qbt, sbt = ops.quant_rowblock(w.t().contiguous(), ops.AXIS_COL, "m_major")      # per-row B scales
    _same_twice(lambda: ops.gemm(qa, sa, qbt, sbt, ops.BSCALE_ROW128, torch.float32), "ROW128")
    qr, sr = ops.quant_rowwise(x)
    qwr, swr = ops.quant_rowwise(w)
    _same_twice(lambda: ops.gemm_rowscaled(qr, sr, qwr, swr), "K-invariant")
    qp, sp = ops.quant_pow2(x, 1)
    qwp, swp = ops.quant_pow2(w, 128)
    _same_twice(lambda: ops.gemm_pow2(qp, sp, qwp, swp), "pow2")
    qm, sm = ops.mx_quant(x)
    qwm, swm = ops.mx_quant(w)
    _same_twice(lambda: ops.mx_gemm(qm, sm, qwm, swm, torch.bfloat16), "MX")


def _moe_case():
    """A grouped problem big enough for the persistent 8-wave 256 x 256
    configuration (several work items per workgroup), with ragged and empty
    groups and the dispatch gather."""
    rng = np.random.default_rng(77)
    G, T, H, I = 32, 4096, 512, 256
    counts = np.where(rng.random(G) < 0.15, 0, rng.integers(100, 1600, G))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    row_token = rng.integers(0, T, rows).astype(np.int32)
    x = dev_bf16(_bits((T, H), 78))
    wgu = dev_bf16(_bits((G, 2 * I, H), 79, 0.02))
    return G, T, H, I, offsets, rows, row_token, x, wgu


def test_grouped_and_fused_epilogues_deterministic():
    G, T, H, I, offsets, rows, row_token, x, wgu = _moe_case()
    _say("determinism, grouped: %d rows, %d groups" % (rows, G))
    offs, a_rows = dev(offsets), dev(row_token)
    qx, sx = ops.quant_rowblock(x, ops.AXIS_ROW, "m_major")
    qgu, sgu, _ = ops.quant_block2d(wgu)

    def grouped(dt):
        c = torch.empty((rows, 2 * I), dtype=dt, device="cuda")
        ops.fp8_grouped_gemm(rows, 2 * I, H, G, offs, a_rows, T, qx, H, sx, 1, T, qgu, H, 2 * I * H, sgu,
                             sgu.stride(0), sgu.stride(1), sgu.stride(2), c, 2 * I,
                             ops.OUT_FP32 if dt == torch.float32 else ops.OUT_BF16)
        return c

    for dt in (torch.bfloat16, torch.float32):
        _same_twice(lambda: grouped(dt), "grouped %s" % dt)

    def fused():
        qh = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
        sh = torch.empty((I // 128, rows), dtype=torch.float32, device="cuda")
        ops.fp8_grouped_gemm_swiglu_quant(rows, I, H, G, offs, a_rows, T, qx, H, sx, 1, T, qgu, H, 2 * I * H, sgu,
                                          sgu.stride(0), sgu.stride(1), sgu.stride(2), qh, I, sh, 1, rows)
        return torch.cat([qh.view(-1), sh.view(torch.uint8).view(-1)])

    _same_twice(fused, "fused SiLU*mul epilogue (1x128)")

    qmx, smx = ops.mx_quant(x)
    qgm, sgm = ops.mx_quant(wgu.view(G * 2 * I, H))

    def mx_grouped(dt):
        c = torch.empty((rows, 2 * I), dtype=dt, device="cuda")
        ops.mxfp8_gemm(rows, 2 * I, H, G, offs, a_rows, T, qmx, H, smx, H // 32, qgm, H, 2 * I * H, sgm, H // 32,
                       2 * I * (H // 32), c, 2 * I, ops.OUT_FP32 if dt == torch.float32 else ops.OUT_BF16)
        return c

    for dt in (torch.bfloat16, torch.float32):
        _same_twice(lambda: mx_grouped(dt), "MX grouped %s" % dt)

    def mx_fused():
        qh = torch.empty((rows, I), dtype=torch.uint8, device="cuda")
        sh = torch.empty((rows, I // 32), dtype=torch.uint8, device="cuda")
        ops.mxfp8_grouped_gemm_swiglu_quant(rows, I, H, G, offs, a_rows, T, qmx, H, smx, H // 32, qgm, H, 2 * I * H,
                                            sgm, H // 32, 2 * I * (H // 32), qh, I, sh, I // 32, 1)
        return torch.cat([qh.view(-1), sh.view(-1)])

    _same_twice(mx_fused, "fused SiLU*mul epilogue (1x32)")


def test_concurrent_threads_and_streams():
    """Two host threads, each on its own stream, quantize a linear layer's
    operands and run the block-scaled and MXFP8 GEMMs on different inputs at
    the same time (ctypes releases the GIL, so the calls and the kernels
    overlap).  Every result equals the same work run alone, byte for byte:
    the library keeps no state between calls, so the streams share nothing."""
    import threading

    jobs = [(dev_bf16(_bits((2048, 2560), 60 + 2 * i, 1.0, 0.01, 30.0)), dev_bf16(_bits((4096, 2560), 61 + 2 * i, 0.02)))
            for i in range(2)]

    def work(x, w):
        qx, sx, qw, sw = ops.quant_linear(x, w)
        y = ops.gemm(qx, sx, qw, sw)
        mqx, msx = ops.mx_quant(x)
        mqw, msw = ops.mx_quant(w)
        ym = ops.mx_gemm(mqx, msx, mqw, msw)
        return [qx, sx.contiguous(), qw, sw, y, mqx, msx, mqw, msw, ym]

    serial = [work(*j) for j in jobs]
    torch.cuda.synchronize()
    results, errors = [None, None], []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    r = work(*jobs[i])
                s.synchronize()
            results[i] = r
        except Exception as e:     # re-raised on the main thread below
            errors.append(e)

    _say("two threads, two streams")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for k, (a, b) in enumerate(zip(serial[i], results[i])):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
                "thread %d, result %d differs from the serial run" % (i, k)
