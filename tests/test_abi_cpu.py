"""The C-ABI library loads, exports every function include/fp8bs.h declares,
and rejects invalid arguments on the host before touching a device.  No
computation is launched here (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from fp8_block_scaled_x128_amd import ops
    if not os.path.exists(ops.library_path()):
        pytest.fail("libfp8bs.so is not built; run __graft_entry__.build()")
    return ops.load()


# The boundary the problem statement fixes: the quantizers (S = max|X| / 448,
# Q = round(x / S): "Unified FP8: Beyond Mixed Precision...", section "FP8
# Quantization"), the block-scaled, grouped and MXFP8 GEMMs and the SiLU*mul
# step between the MoE GEMMs, the grouped GEMM's workspace query and the two
# status helpers.
BOUNDARY = ["fp8_quant_rowblock", "fp8_quant_block2d", "fp8_blockscaled_gemm", "fp8_grouped_gemm",
            "fp8_grouped_gemm_ws_size", "fp8_silu_mul_quant", "mxfp8_quant", "mxfp8_gemm",
            "fp8bs_status_string", "fp8bs_last_error_detail"]
BOUNDARY_ENUMS = ["fp8bs_status", "fp8bs_axis", "fp8bs_out", "fp8bs_bscale"]


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in BOUNDARY + ["fp8bs_e4m3_encode"]:
        assert n in names, n
    text = open(HEADER).read()
    for e in BOUNDARY_ENUMS:
        assert re.search(r"}\s*%s\s*;" % e, text), e


def test_boundary_exported(lib):
    for n in BOUNDARY:
        assert hasattr(lib, n), "missing export %s" % n


def test_grouped_gemm_needs_no_workspace(lib):
    from fp8_block_scaled_x128_amd import ops
    assert ops.fp8_grouped_gemm_ws_size(131072, 128, 2048) == 0
    assert ops.fp8_grouped_gemm_ws_size(0, 1, 0) == 0
    assert ops.fp8_grouped_gemm_ws_size(-1, 128, 2048, raise_on_error=False) is None
    assert ops.fp8_grouped_gemm_ws_size(16, 0, 128, raise_on_error=False) is None
    assert lib.fp8_grouped_gemm_ws_size(16, 4, 128, None) == 1      # FP8BS_ERR_NULL


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), "missing export %s" % n


def test_status_strings(lib):
    assert lib.fp8bs_status_string(0) == b"FP8BS_OK"
    assert lib.fp8bs_status_string(2) == b"FP8BS_ERR_SHAPE"
    assert lib.fp8bs_status_string(99) == b"FP8BS_UNKNOWN_STATUS"


def test_host_validation_rejects_before_launch(lib):
    from fp8_block_scaled_x128_amd import ops
    fake = 1 << 20     # never dereferenced: validation fails first
    # negative size
    assert ops.fp8_quant_rowblock(fake, -1, 128, 128, 0, fake, 128, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 2
    # cols not a multiple of 8
    assert ops.fp8_quant_rowblock(fake, 4, 100, 104, 0, fake, 104, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 2
    # ld_x < cols
    assert ops.fp8_quant_rowblock(fake, 4, 128, 64, 0, fake, 128, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 3
    # misaligned x
    assert ops.fp8_quant_rowblock(fake + 2, 4, 128, 128, 0, fake, 128, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 4
    # bad axis
    assert ops.fp8_quant_rowblock(fake, 4, 128, 128, 7, fake, 128, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 5
    # NULL input
    assert ops.fp8_quant_rowblock(None, 4, 128, 128, 0, fake, 128, fake, 1, 1, stream=0,
                                  raise_on_error=False) == 1
    detail = lib.fp8bs_last_error_detail()
    assert b"required" in detail
    # GEMM: K % 128, N % 128, bad bscale, bad out
    g = lambda M, N, K, bs=0, out=0: ops.fp8_blockscaled_gemm(M, N, K, fake, K, fake, 1, 1, fake, K, fake, 1, 1,
                                                              bs, fake, N, out, stream=0, raise_on_error=False)
    assert g(128, 128, 100) == 2
    assert g(128, 100, 128) == 2
    assert g(128, 128, 128, bs=3) == 5
    assert g(128, 128, 128, out=9) == 5
    # grouped: G < 1
    assert ops.fp8_grouped_gemm(128, 128, 128, 0, fake, None, 0, fake, 128, fake, 1, 1, fake, 128, 0, fake, 0, 1, 1,
                                fake, 128, 0, stream=0, raise_on_error=False) == 2
    # MX: cols % 32
    assert ops.mxfp8_quant(fake, 4, 48, 48, fake, 48, fake, 1, 1, stream=0, raise_on_error=False) == 2
    # silu: I % 128 for the FP32-scale mode
    assert ops.fp8_silu_mul_quant(fake, 4, 96, 192, 0, fake, 96, fake, 1, 1, None, 0, stream=0,
                                  raise_on_error=False) == 2
    # empty inputs are a successful no-op
    assert ops.fp8_quant_rowblock(None, 0, 128, 128, 0, None, 128, None, 1, 1, stream=0,
                                  raise_on_error=False) == 0
    # both operands of a linear layer in one launch: each operand checked as
    # its own call would check it; an empty operand's pointers are not read
    lin = lambda x, rows, cols, ld_x, w, w_rows, ld_w, sx=fake, sw=fake: ops.fp8_quant_linear(
        x, rows, cols, ld_x, fake, cols, sx, 1, max(rows, 1), w, w_rows, ld_w, fake, cols, sw, stream=0,
        raise_on_error=False)
    assert lin(fake, 4, 100, 100, fake, 128, 100) == 2          # cols % 8
    assert lin(fake, 4, 128, 64, fake, 128, 128) == 3           # ld_x < cols
    assert lin(fake, 4, 128, 128, fake, 128, 64) == 3           # ld_w < cols
    assert lin(fake + 2, 4, 128, 128, fake, 128, 128) == 4      # misaligned x
    assert lin(fake, 4, 128, 128, fake + 2, 128, 128) == 4      # misaligned w
    assert lin(None, 4, 128, 128, fake, 128, 128) == 1          # NULL x
    assert lin(fake, 4, 128, 128, fake, 128, 128, sw=None) == 1  # NULL weight scales
    assert lin(fake, -1, 128, 128, fake, 128, 128) == 2
    assert lin(None, 0, 128, 128, None, 0, 128, sx=None, sw=None) == 0
    # grouped gate/up GEMM with SiLU*mul and 1x128 quantization of h
    swi = lambda rows, I, K, G=2, hq=fake, ld_hq=None, hs=fake, ldb=None: ops.fp8_grouped_gemm_swiglu_quant(
        rows, I, K, G, fake, None, rows, fake, K, fake, 1, 1, fake, K if ldb is None else ldb, 2 * I * K, fake, 1,
        1, 1, hq, I if ld_hq is None else ld_hq, hs, 1, max(rows, 1), stream=0, raise_on_error=False)
    assert swi(256, 96, 256) == 2                 # I % 128
    assert swi(256, 128, 200) == 2                # K % 128
    assert swi(256, 128, 256, G=0) == 2           # G < 1
    assert swi(256, 128, 256, hq=None) == 1       # NULL h codes
    assert swi(256, 128, 256, hs=None) == 1       # NULL h scales
    assert swi(256, 128, 256, ld_hq=64) == 3      # ld_hq < I
    assert swi(256, 128, 256, hq=fake + 4) == 4   # h codes not 8-byte aligned
    assert swi(256, 128, 256, ldb=64) == 3        # ldb < K
    assert swi(0, 128, 256) == 0                  # no rows: a successful no-op
    # its MXFP8 counterpart
    mxs = lambda rows, I, K, G=2, lds=None, hs=fake: ops.mxfp8_grouped_gemm_swiglu_quant(
        rows, I, K, G, fake, None, rows, fake, K, fake, K // 32 if lds is None else lds, fake, K, 2 * I * K, fake,
        K // 32 if lds is None else lds, 2 * I * (K // 32), fake, I, hs, I // 32, 1, stream=0, raise_on_error=False)
    assert mxs(256, 96, 256) == 2                 # I % 128
    assert mxs(256, 128, 256, G=0) == 2           # G < 1
    assert mxs(256, 128, 256, lds=4) == 3         # scale leading dimension < K/32
    assert mxs(256, 128, 256, lds=10) == 4        # scale leading dimension % 4
    assert mxs(256, 128, 256, hs=None) == 1       # NULL h scales
    assert mxs(0, 128, 256) == 0
    # 128x128 blocks: the row-major codes may be skipped only when the
    # transposed copy is written
    b2 = lambda q, qt: ops.fp8_quant_block2d(fake, 1, 128, 128, 128, q, 128, qt, 128, fake, stream=0,
                                             raise_on_error=False)
    assert b2(None, None) == 1
    assert b2(None, fake + 8) == 4                # q_t must be 16-byte aligned
    # both operands with power-of-two scales
    lp = lambda rows, w_rows, cols, ld_sx=None, ld_sw=None, sx=fake, sw=fake: ops.fp8_quant_linear_pow2(
        fake, rows, cols, cols, fake, cols, sx, (cols + 127) // 128 if ld_sx is None else ld_sx, fake, w_rows, cols,
        fake, cols, sw, (cols + 127) // 128 if ld_sw is None else ld_sw, stream=0, raise_on_error=False)
    assert lp(4, 128, 100) == 2                   # cols % 8
    assert lp(4, 128, 512, ld_sx=3) == 3          # ld_sx < ceil(cols / 128)
    assert lp(4, 128, 512, ld_sw=3) == 3
    assert lp(4, 128, 512, sw=None) == 1
    assert lp(0, 128, 512, sx=None) != 1          # an empty X's pointers are not checked (no NULL error)
    assert lp(0, 0, 512, sx=None, sw=None) == 0
    # transposed copy of codes
    tr = lambda rows, cols, q=fake, qt=fake, ld_q=None, ld_qt=None, batch=1: ops.fp8_transpose_codes(
        q, batch, rows, cols, cols if ld_q is None else ld_q, qt, rows if ld_qt is None else ld_qt, stream=0,
        raise_on_error=False)
    assert tr(128, 120) == 2                      # cols % 16
    assert tr(120, 128) == 2                      # rows % 16
    assert tr(128, 128, batch=0) == 2
    assert tr(128, 128, ld_qt=112) == 3           # ld_qt < rows
    assert tr(128, 128, q=fake + 8) == 4          # q not 16-byte aligned
    assert tr(128, 128, ld_qt=136) == 4           # ld_qt % 16
    assert tr(128, 128, qt=None) == 1
    assert tr(0, 128, q=None, qt=None) == 0
    # both axes of one tensor from one read
    dual = lambda rows, cols, mx=0, x=fake, ld_x=None, q=fake, qt=fake, ld_qt=None, st=fake: ops.fp8_quant_dual_axis(
        x, rows, cols, cols if ld_x is None else ld_x, mx, q, cols, fake, 1, 1, qt, rows if ld_qt is None else ld_qt,
        st, 1, 1, stream=0, raise_on_error=False)
    assert dual(128, 128, mx=2) == 5              # bad mx
    assert dual(120, 128) == 2                    # rows % 16
    assert dual(128, 100) == 2                    # cols % 8
    assert dual(80, 128, mx=1) == 2               # MX rows % 32
    assert dual(128, 64 * 1024 * 128, ld_x=None) == 2   # more than 65535 column tiles
    assert dual(128, 128, ld_x=64) == 3           # ld_x < cols
    assert dual(128, 128, ld_qt=64) == 3          # ld_qt < rows
    assert dual(128, 128, x=fake + 2) == 4        # misaligned x
    assert dual(128, 128, qt=fake + 4) == 4       # qt not 8-byte aligned
    assert dual(128, 128, st=fake + 2) == 4       # fp32 column scales not 4-byte aligned
    assert dual(128, 128, q=None) == 1            # NULL row codes
    assert dual(0, 128, x=None, q=None, qt=None, st=None) == 0


def test_splitk_plan(lib):
    """The K-split query (host only): no split for the MLP shapes at 4096
    tokens, a split for decode-sized ones, the workspace it needs, and the
    shape errors of the GEMM."""
    from fp8_block_scaled_x128_amd import ops
    for M, N, K in [(4096, 9728, 2560), (4096, 2560, 9728), (9728, 2560, 4096), (0, 2560, 9728), (128, 0, 9728)]:
        assert ops.fp8_blockscaled_gemm_splitk_plan(M, N, K, ops.OUT_BF16) == (1, 0)
    for M, N, K in [(128, 2560, 9728), (512, 2560, 9728), (128, 9728, 2560)]:
        for out in (ops.OUT_BF16, ops.OUT_FP32):
            s, wb = ops.fp8_blockscaled_gemm_splitk_plan(M, N, K, out)
            assert 1 < s <= min(32, K // 128) and wb == s * M * N * 4
    sp, wb = ctypes.c_int32(0), ctypes.c_size_t(0)
    assert lib.fp8_blockscaled_gemm_splitk_plan(128, 100, 128, 0, ctypes.byref(sp), ctypes.byref(wb)) == 2
    assert lib.fp8_blockscaled_gemm_splitk_plan(128, 128, 100, 0, ctypes.byref(sp), ctypes.byref(wb)) == 2
    assert lib.fp8_blockscaled_gemm_splitk_plan(128, 128, 128, 7, ctypes.byref(sp), ctypes.byref(wb)) == 5
    assert lib.fp8_blockscaled_gemm_splitk_plan(128, 128, 128, 0, None, ctypes.byref(wb)) == 1


def test_dense_tile_plan(lib):
    """The tiling query (host only): regions cover N on a 128-column boundary,
    every region's tiling is one the library builds, and the MLP shapes get
    tilings that fill whole rounds of 256 compute units."""
    from fp8_block_scaled_x128_amd import ops
    tilings = {(8, 256), (4, 256), (8, 160), (4, 192), (4, 128), (4, 160)}
    for M in (1, 130, 1000, 4096, 4100, 16384):
        for N in (128, 640, 1408, 2560, 4096, 9728):
            for K in (128, 2560, 9728):
                first, second, split = ops.fp8_blockscaled_gemm_plan(M, N, K)
                assert first in tilings
                if second is None:
                    assert split == N
                else:
                    assert second in tilings and second != first
                    assert 0 < split < N and split % 128 == 0 and split % first[1] == 0
    # down projection (and dgrad): 32 x 16 tiles of 160 x 128, two per
    # compute unit (one round); up projection and wgrad: 128 x 256 tiles, two
    # per compute unit; K 4096 at the down projection's M and N: 160 x 256
    assert ops.fp8_blockscaled_gemm_plan(4096, 2560, 9728) == ((4, 160), None, 2560)
    assert ops.fp8_blockscaled_gemm_plan(4096, 2560, 4096) == ((8, 160), None, 2560)
    assert ops.fp8_blockscaled_gemm_plan(4096, 9728, 2560) == ((4, 128), None, 9728)
    assert ops.fp8_blockscaled_gemm_plan(9728, 2560, 4096) == ((4, 128), None, 2560)
    assert lib.fp8_blockscaled_gemm_plan(128, 100, 128, ctypes.c_void_p(1 << 20)) == 2
    assert lib.fp8_blockscaled_gemm_plan(128, 128, 128, None) == 1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with a message before any
    device work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
