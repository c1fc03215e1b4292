"""Thin ctypes binding of libfp8bs.so (include/fp8bs.h).

The functions carry the C names and only marshal arguments: tensor -> device
pointer, sizes, strides, and the current torch stream as the HIP stream.
Every step of the computation runs in the HIP library; if the library is not
built or cannot be loaded, every call raises.  PyTorch provides device memory
and streams only.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8bs.so")
_lock = threading.Lock()
_lib = None

STATUS = {0: "FP8BS_OK", 1: "FP8BS_ERR_NULL", 2: "FP8BS_ERR_SHAPE", 3: "FP8BS_ERR_STRIDE",
          4: "FP8BS_ERR_ALIGN", 5: "FP8BS_ERR_UNSUPPORTED", 6: "FP8BS_ERR_DEVICE"}
AXIS_ROW, AXIS_COL = 0, 1
OUT_BF16, OUT_FP32 = 0, 1
BSCALE_BLOCK128, BSCALE_ROW128 = 0, 1

EXPORTS = ["fp8_quant_rowblock", "fp8_quant_block2d", "fp8_quant_linear", "fp8_quant_rowwise", "fp8_quant_tensorwise", "fp8_blockscaled_gemm", "fp8_blockscaled_gemm_plan",
           "fp8_blockscaled_gemm_splitk", "fp8_blockscaled_gemm_splitk_noalloc", "fp8_blockscaled_gemm_splitk_plan",
           "fp8_grouped_gemm", "fp8_grouped_gemm_ws_size", "fp8_grouped_gemm_swiglu_quant", "mxfp8_grouped_gemm_swiglu_quant",
           "fp8_silu_mul_quant", "fp8_moe_combine", "mxfp8_quant", "mxfp8_quant_t",
           "fp8_quant_dual_axis", "fp8_transpose_codes", "fp8_quant_linear_pow2",
           "fp8_quant_pow2", "fp8_blockscaled_gemm_pow2", "mxfp8_gemm", "fp8bs_e4m3_encode",
           "fp8bs_status_string", "fp8bs_last_error_detail"]


class Fp8bsError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), detail))
        self.status = status
        self.detail = detail


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libfp8bs.so (raises if it is missing: there is no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libfp8bs.so is not built (%s); run `python -m fp8_block_scaled_x128_amd.build`"
                               % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        sig = {
            "fp8_quant_rowblock": [P, I64, I64, I64, INT, P, I64, P, I64, I64, P],
            "fp8_quant_block2d": [P, I64, I64, I64, I64, P, I64, P, I64, P, P],
            "fp8_quant_linear": [P, I64, I64, I64, P, I64, P, I64, I64, P, I64, I64, P, I64, P, P],
            "fp8_quant_rowwise": [P, I64, I64, I64, P, I64, P, P],
            "fp8_quant_tensorwise": [P, I64, I64, I64, P, I64, P, P],
            "fp8_blockscaled_gemm": [I64, I64, I64, P, I64, P, I64, I64, P, I64, P, I64, I64, INT, P, I64, INT, P],
            "fp8_blockscaled_gemm_plan": [I64, I64, I64, P],
            "fp8_blockscaled_gemm_splitk": [I64, I64, I64, P, I64, P, I64, I64, P, I64, P, I64, I64, INT, P, I64,
                                            INT, I32, P, ctypes.c_size_t, P],
            "fp8_blockscaled_gemm_splitk_plan": [I64, I64, I64, INT, P, P],
            "fp8_blockscaled_gemm_splitk_noalloc": [I64, I64, I64, P, I64, P, I64, I64, P, I64, P, I64, I64, INT, P,
                                                    I64, INT, I32, P],
            "fp8_grouped_gemm": [I64, I64, I64, I32, P, P, I64, P, I64, P, I64, I64, P, I64, I64, P, I64, I64, I64,
                                 P, I64, INT, P],
            "fp8_grouped_gemm_ws_size": [I64, I32, I64, P],
            "fp8_grouped_gemm_swiglu_quant": [I64, I64, I64, I32, P, P, I64, P, I64, P, I64, I64, P, I64, I64, P,
                                              I64, I64, I64, P, I64, P, I64, I64, P],
            "mxfp8_grouped_gemm_swiglu_quant": [I64, I64, I64, I32, P, P, I64, P, I64, P, I64, P, I64, I64, P, I64,
                                                I64, P, I64, P, I64, I64, P],
            "fp8_silu_mul_quant": [P, I64, I64, I64, INT, P, I64, P, I64, I64, P, I64, P],
            "fp8_moe_combine": [P, I64, I64, I64, P, P, I64, I32, P, I64, INT, P],
            "mxfp8_quant": [P, I64, I64, I64, P, I64, P, I64, I64, P],
            "mxfp8_quant_t": [P, I64, I64, I64, P, I64, P, I64, I64, P],
            "fp8_quant_dual_axis": [P, I64, I64, I64, I32, P, I64, P, I64, I64, P, I64, P, I64, I64, P],
            "fp8_transpose_codes": [P, I64, I64, I64, I64, P, I64, P],
            "fp8_quant_linear_pow2": [P, I64, I64, I64, P, I64, P, I64, P, I64, I64, P, I64, P, I64, P],
            "fp8_quant_pow2": [P, I64, I64, I64, I32, P, I64, P, I64, P],
            "fp8_blockscaled_gemm_pow2": [I64, I64, I64, P, I64, P, I64, P, I64, P, I64, P, I64, INT, P],
            "mxfp8_gemm": [I64, I64, I64, I32, P, P, I64, P, I64, P, I64, P, I64, I64, P, I64, I64, P, I64, INT, P],
            "fp8bs_e4m3_encode": [P, P, I64, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.fp8bs_status_string.argtypes = [ctypes.c_int]
        lib.fp8bs_status_string.restype = ctypes.c_char_p
        lib.fp8bs_last_error_detail.argtypes = []
        lib.fp8bs_last_error_detail.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name, status, raise_on_error=True):
    if status != 0 and raise_on_error:
        detail = load().fp8bs_last_error_detail().decode()
        raise Fp8bsError(name, status, detail)
    return status


# ---------------------------------------------------------------- raw C calls
def fp8_quant_rowblock(x, rows, cols, ld_x, axis, q, ld_q, s, s_stride_row, s_stride_group, stream=None,
                       raise_on_error=True):
    st = load().fp8_quant_rowblock(_p(x), rows, cols, ld_x, axis, _p(q), ld_q, _p(s), s_stride_row,
                                   s_stride_group, _stream(stream))
    return _check("fp8_quant_rowblock", st, raise_on_error)


def fp8_quant_block2d(w, batch, rows, cols, ld_w, q, ld_q, q_t, ld_qt, s, stream=None, raise_on_error=True):
    st = load().fp8_quant_block2d(_p(w), batch, rows, cols, ld_w, _p(q), ld_q, _p(q_t), ld_qt, _p(s),
                                  _stream(stream))
    return _check("fp8_quant_block2d", st, raise_on_error)


def fp8_quant_linear(x, rows, cols, ld_x, qx, ld_qx, sx, sx_stride_row, sx_stride_group, w, w_rows, ld_w, qw, ld_qw,
                     sw, stream=None, raise_on_error=True):
    st = load().fp8_quant_linear(_p(x), rows, cols, ld_x, _p(qx), ld_qx, _p(sx), sx_stride_row, sx_stride_group,
                                 _p(w), w_rows, ld_w, _p(qw), ld_qw, _p(sw), _stream(stream))
    return _check("fp8_quant_linear", st, raise_on_error)


def fp8_quant_rowwise(x, rows, cols, ld_x, q, ld_q, s, stream=None, raise_on_error=True):
    st = load().fp8_quant_rowwise(_p(x), rows, cols, ld_x, _p(q), ld_q, _p(s), _stream(stream))
    return _check("fp8_quant_rowwise", st, raise_on_error)


def fp8_quant_tensorwise(x, rows, cols, ld_x, q, ld_q, s, stream=None, raise_on_error=True):
    st = load().fp8_quant_tensorwise(_p(x), rows, cols, ld_x, _p(q), ld_q, _p(s), _stream(stream))
    return _check("fp8_quant_tensorwise", st, raise_on_error)


def fp8_blockscaled_gemm(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n, sb_stride_k,
                         bscale, c, ldc, out, stream=None, raise_on_error=True):
    st = load().fp8_blockscaled_gemm(M, N, K, _p(a), lda, _p(sa), sa_stride_m, sa_stride_k, _p(b), ldb, _p(sb),
                                     sb_stride_n, sb_stride_k, bscale, _p(c), ldc, out, _stream(stream))
    return _check("fp8_blockscaled_gemm", st, raise_on_error)


def fp8_blockscaled_gemm_plan(M, N, K):
    """Tiling of a BLOCK128 problem: ((waves, weight rows per tile) for columns
    [0, split), (waves, rows) for [split, N) or None, split).  Host only."""
    out = (ctypes.c_int32 * 5)()
    _check("fp8_blockscaled_gemm_plan", load().fp8_blockscaled_gemm_plan(M, N, K, ctypes.cast(out, ctypes.c_void_p)))
    return (out[0], out[1]), ((out[2], out[3]) if out[2] else None), out[4]


def fp8_blockscaled_gemm_splitk(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n,
                                sb_stride_k, bscale, c, ldc, out, splits, ws, ws_bytes, stream=None,
                                raise_on_error=True):
    st = load().fp8_blockscaled_gemm_splitk(M, N, K, _p(a), lda, _p(sa), sa_stride_m, sa_stride_k, _p(b), ldb,
                                            _p(sb), sb_stride_n, sb_stride_k, bscale, _p(c), ldc, out, splits,
                                            _p(ws), ws_bytes, _stream(stream))
    return _check("fp8_blockscaled_gemm_splitk", st, raise_on_error)


def fp8_blockscaled_gemm_splitk_noalloc(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n,
                                        sb_stride_k, bscale, c, ldc, out, splits, stream=None, raise_on_error=True):
    st = load().fp8_blockscaled_gemm_splitk_noalloc(M, N, K, _p(a), lda, _p(sa), sa_stride_m, sa_stride_k, _p(b),
                                                    ldb, _p(sb), sb_stride_n, sb_stride_k, bscale, _p(c), ldc, out,
                                                    splits, _stream(stream))
    return _check("fp8_blockscaled_gemm_splitk_noalloc", st, raise_on_error)


def fp8_blockscaled_gemm_splitk_plan(M, N, K, out):
    """(splits, workspace bytes) the K-split GEMM chooses.  Host only."""
    sp, wb = ctypes.c_int32(0), ctypes.c_size_t(0)
    _check("fp8_blockscaled_gemm_splitk_plan",
           load().fp8_blockscaled_gemm_splitk_plan(M, N, K, out, ctypes.byref(sp), ctypes.byref(wb)))
    return sp.value, wb.value


def fp8_grouped_gemm_ws_size(max_total_rows, G, N, raise_on_error=True):
    """Workspace bytes of the grouped GEMMs (host only); always 0."""
    out = ctypes.c_size_t(0)
    st = load().fp8_grouped_gemm_ws_size(max_total_rows, G, N, ctypes.byref(out))
    if _check("fp8_grouped_gemm_ws_size", st, raise_on_error) != 0:
        return None
    return out.value


def fp8_grouped_gemm_swiglu_quant(total_rows, I, K, G, offsets, a_rows, a_count, a, lda, sa, sa_stride_m, sa_stride_k,
                                  b, ldb, b_stride_g, sb, sb_stride_g, sb_stride_n, sb_stride_k, hq, ld_hq, hs,
                                  hs_stride_row, hs_stride_group, stream=None, raise_on_error=True):
    st = load().fp8_grouped_gemm_swiglu_quant(total_rows, I, K, G, _p(offsets), _p(a_rows), a_count, _p(a), lda, _p(sa),
                                              sa_stride_m, sa_stride_k, _p(b), ldb, b_stride_g, _p(sb), sb_stride_g,
                                              sb_stride_n, sb_stride_k, _p(hq), ld_hq, _p(hs), hs_stride_row,
                                              hs_stride_group, _stream(stream))
    return _check("fp8_grouped_gemm_swiglu_quant", st, raise_on_error)


def mxfp8_grouped_gemm_swiglu_quant(total_rows, I, K, G, offsets, a_rows, a_count, a, lda, sa, lds_a, b, ldb,
                                    b_stride_g, sb, lds_b, sb_stride_g, hq, ld_hq, hs, hs_stride_row,
                                    hs_stride_group, stream=None, raise_on_error=True):
    st = load().mxfp8_grouped_gemm_swiglu_quant(total_rows, I, K, G, _p(offsets), _p(a_rows), a_count, _p(a), lda,
                                                _p(sa), lds_a, _p(b), ldb, b_stride_g, _p(sb), lds_b, sb_stride_g,
                                                _p(hq), ld_hq, _p(hs), hs_stride_row, hs_stride_group,
                                                _stream(stream))
    return _check("mxfp8_grouped_gemm_swiglu_quant", st, raise_on_error)


def fp8_grouped_gemm(total_rows, N, K, G, offsets, a_rows, a_count, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb,
                     b_stride_g, sb, sb_stride_g, sb_stride_n, sb_stride_k, c, ldc, out, stream=None,
                     raise_on_error=True):
    st = load().fp8_grouped_gemm(total_rows, N, K, G, _p(offsets), _p(a_rows), a_count, _p(a), lda, _p(sa),
                                 sa_stride_m, sa_stride_k, _p(b), ldb, b_stride_g, _p(sb), sb_stride_g, sb_stride_n,
                                 sb_stride_k, _p(c), ldc, out, _stream(stream))
    return _check("fp8_grouped_gemm", st, raise_on_error)


def fp8_silu_mul_quant(gate_up, rows, I, ld_in, mx, q, ld_q, s, s_stride_row, s_stride_group, h_out, ld_h,
                       stream=None, raise_on_error=True):
    st = load().fp8_silu_mul_quant(_p(gate_up), rows, I, ld_in, mx, _p(q), ld_q, _p(s), s_stride_row,
                                   s_stride_group, _p(h_out), ld_h, _stream(stream))
    return _check("fp8_silu_mul_quant", st, raise_on_error)


def fp8_moe_combine(y, rows, H, ld_y, token_rows, weights, T, k, out, ld_out, out_type, stream=None,
                    raise_on_error=True):
    st = load().fp8_moe_combine(_p(y), rows, H, ld_y, _p(token_rows), _p(weights), T, k, _p(out), ld_out,
                                out_type, _stream(stream))
    return _check("fp8_moe_combine", st, raise_on_error)


def mxfp8_quant(x, rows, cols, ld_x, q, ld_q, s, s_stride_row, s_stride_group, stream=None, raise_on_error=True):
    st = load().mxfp8_quant(_p(x), rows, cols, ld_x, _p(q), ld_q, _p(s), s_stride_row, s_stride_group,
                            _stream(stream))
    return _check("mxfp8_quant", st, raise_on_error)


def mxfp8_quant_t(x, rows, cols, ld_x, qt, ld_qt, s, s_stride_row, s_stride_group, stream=None,
                  raise_on_error=True):
    st = load().mxfp8_quant_t(_p(x), rows, cols, ld_x, _p(qt), ld_qt, _p(s), s_stride_row, s_stride_group,
                              _stream(stream))
    return _check("mxfp8_quant_t", st, raise_on_error)


def fp8_quant_dual_axis(x, rows, cols, ld_x, mx, q, ld_q, s, s_stride_row, s_stride_group, qt, ld_qt, st,
                        st_stride_row, st_stride_group, stream=None, raise_on_error=True):
    r = load().fp8_quant_dual_axis(_p(x), rows, cols, ld_x, mx, _p(q), ld_q, _p(s), s_stride_row, s_stride_group,
                                   _p(qt), ld_qt, _p(st), st_stride_row, st_stride_group, _stream(stream))
    return _check("fp8_quant_dual_axis", r, raise_on_error)


def fp8_quant_linear_pow2(x, rows, cols, ld_x, qx, ld_qx, sx, ld_sx, w, w_rows, ld_w, qw, ld_qw, sw, ld_sw,
                          stream=None, raise_on_error=True):
    r = load().fp8_quant_linear_pow2(_p(x), rows, cols, ld_x, _p(qx), ld_qx, _p(sx), ld_sx, _p(w), w_rows, ld_w,
                                     _p(qw), ld_qw, _p(sw), ld_sw, _stream(stream))
    return _check("fp8_quant_linear_pow2", r, raise_on_error)


def fp8_transpose_codes(q, batch, rows, cols, ld_q, q_t, ld_qt, stream=None, raise_on_error=True):
    r = load().fp8_transpose_codes(_p(q), batch, rows, cols, ld_q, _p(q_t), ld_qt, _stream(stream))
    return _check("fp8_transpose_codes", r, raise_on_error)


def fp8_quant_pow2(x, rows, cols, ld_x, block_rows, q, ld_q, s, ld_s, stream=None, raise_on_error=True):
    st = load().fp8_quant_pow2(_p(x), rows, cols, ld_x, block_rows, _p(q), ld_q, _p(s), ld_s, _stream(stream))
    return _check("fp8_quant_pow2", st, raise_on_error)


def fp8_blockscaled_gemm_pow2(M, N, K, a, lda, sa, lds_a, b, ldb, sb, lds_b, c, ldc, out, stream=None,
                              raise_on_error=True):
    st = load().fp8_blockscaled_gemm_pow2(M, N, K, _p(a), lda, _p(sa), lds_a, _p(b), ldb, _p(sb), lds_b, _p(c), ldc,
                                          out, _stream(stream))
    return _check("fp8_blockscaled_gemm_pow2", st, raise_on_error)


def mxfp8_gemm(rows, N, K, G, offsets, a_rows, a_count, a, lda, sa, lds_a, b, ldb, b_stride_g, sb, lds_b,
               sb_stride_g, c, ldc, out, stream=None, raise_on_error=True):
    st = load().mxfp8_gemm(rows, N, K, G, _p(offsets), _p(a_rows), a_count, _p(a), lda, _p(sa), lds_a, _p(b), ldb,
                           b_stride_g, _p(sb), lds_b, sb_stride_g, _p(c), ldc, out, _stream(stream))
    return _check("mxfp8_gemm", st, raise_on_error)


def fp8bs_e4m3_encode(inp, out, n, stream=None, raise_on_error=True):
    st = load().fp8bs_e4m3_encode(_p(inp), _p(out), n, _stream(stream))
    return _check("fp8bs_e4m3_encode", st, raise_on_error)


# ------------------------------------------------------- tensor conveniences
def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


def quant_rowblock(x: torch.Tensor, axis: int = AXIS_ROW, scale_layout: str = "m_major"):
    """Quantize a bf16 [rows, cols] tensor.  Returns (q, s) with s logically
    [rows, groups] (AXIS_ROW) or [cols, groups] (AXIS_COL).  scale_layout
    'm_major' stores s as a [groups, rows] buffer (stride_row 1) and returns a
    [rows, groups] view of it; 'row_major' stores [rows, groups]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if axis == AXIS_ROW:
        q = _u8((rows, cols), x.device)
        lead, ng = rows, (cols + 127) // 128
        ld_q = cols
    else:
        q = _u8((cols, rows), x.device)
        lead, ng = cols, (rows + 127) // 128
        ld_q = rows
    if scale_layout == "m_major":
        sbuf = torch.empty((ng, lead), dtype=torch.float32, device=x.device)
        s, ssr, ssg = sbuf.t(), 1, lead
    else:
        s = torch.empty((lead, ng), dtype=torch.float32, device=x.device)
        ssr, ssg = ng, 1
    fp8_quant_rowblock(x, rows, cols, x.stride(0), axis, q, ld_q, s, ssr, ssg)
    return q, s


def quant_dual_axis(x: torch.Tensor, mx: bool = False):
    """Row groups and column groups of a bf16 [rows, cols] tensor from one
    read: (q [rows, cols], s, qt [cols, rows], st).  FP32 scales (mx False):
    s is a [rows, cols/128] view of a [cols/128, rows] buffer and st a
    [cols, rows/128] view of a [rows/128, cols] buffer (the M-major layouts
    the GEMMs read); MX: uint8 s [rows, cols/32] and st [cols, rows/32],
    row-major."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    q, qt = _u8((rows, cols), x.device), _u8((cols, rows), x.device)
    if mx:
        s, st = _u8((rows, cols // 32), x.device), _u8((cols, rows // 32), x.device)
        fp8_quant_dual_axis(x, rows, cols, x.stride(0), 1, q, cols, s, cols // 32, 1, qt, rows, st, rows // 32, 1)
        return q, s, qt, st
    ng, ngt = (cols + 127) // 128, (rows + 127) // 128
    sbuf = torch.empty((ng, rows), dtype=torch.float32, device=x.device)
    stbuf = torch.empty((ngt, cols), dtype=torch.float32, device=x.device)
    fp8_quant_dual_axis(x, rows, cols, x.stride(0), 0, q, cols, sbuf, 1, rows, qt, rows, stbuf, 1, cols)
    return q, sbuf.t(), qt, stbuf.t()


def quant_linear(x: torch.Tensor, w: torch.Tensor):
    """Both operands of a linear layer in one launch: X [rows, cols] in 1x128
    groups (M-major scales, returned as a [rows, groups] view) and W
    [w_rows, cols] in 128x128 blocks.  Returns (qx, sx, qw, sw)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.is_contiguous() and w.shape[1] == x.shape[1]
    rows, cols = x.shape
    w_rows = w.shape[0]
    ng = (cols + 127) // 128
    qx, qw = _u8((rows, cols), x.device), _u8((w_rows, cols), x.device)
    sbuf = torch.empty((ng, rows), dtype=torch.float32, device=x.device)
    sw = torch.empty(((w_rows + 127) // 128, ng), dtype=torch.float32, device=x.device)
    fp8_quant_linear(x, rows, cols, cols, qx, cols, sbuf, 1, rows, w, w_rows, cols, qw, cols, sw)
    return qx, sbuf.t(), qw, sw


def quant_block2d(w: torch.Tensor, transposed: bool = False):
    """128x128 block quantization of a bf16 [rows, cols] or [batch, rows, cols]
    tensor.  Returns (q, s, q_t or None)."""
    assert w.dtype == torch.bfloat16 and w.is_contiguous()
    batched = w.dim() == 3
    ww = w if batched else w.unsqueeze(0)
    batch, rows, cols = ww.shape
    q = _u8(ww.shape, w.device)
    qt = _u8((batch, cols, rows), w.device) if transposed else None
    s = torch.empty((batch, (rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=w.device)
    fp8_quant_block2d(ww, batch, rows, cols, cols, q, cols, qt, rows, s)
    if not batched:
        q, s = q[0], s[0]
        qt = qt[0] if qt is not None else None
    return q, s, qt


def quant_rowwise(x: torch.Tensor):
    """One scale per row of a bf16 [rows, cols] tensor -> (q, s [rows])."""
    rows, cols = x.shape
    q = _u8((rows, cols), x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    fp8_quant_rowwise(x, rows, cols, x.stride(0), q, cols, s)
    return q, s


def quant_tensorwise(x: torch.Tensor):
    """One scale for a whole bf16 [rows, cols] tensor -> (q, s [1])."""
    rows, cols = x.shape
    q = _u8((rows, cols), x.device)
    s = torch.empty((1,), dtype=torch.float32, device=x.device)
    fp8_quant_tensorwise(x, rows, cols, x.stride(0), q, cols, s)
    return q, s


def gemm_rowscaled(a, sa, b, sb, out_dtype=torch.bfloat16):
    """C = diag(sa) (A B^T) diag(sb) for codes a [M, K], b [N, K] and scales
    sa [M] or [1], sb [N] or [1] (rowwise or tensorwise): the block-scaled GEMM
    with scale views of K stride 0."""
    M, K = a.shape
    N = b.shape[0]
    sa_v = sa.view(-1, 1).expand(M, K // 128)
    sb_v = sb.view(-1, 1).expand(N, K // 128)
    return gemm(a, sa_v, b, sb_v, bscale=BSCALE_ROW128, out_dtype=out_dtype)


def gemm(a, sa, b, sb, bscale=BSCALE_BLOCK128, out_dtype=torch.bfloat16):
    """C = A B^T for codes a [M, K], b [N, K] and logical scale views
    sa [M, K/128], sb [N/128 or N, K/128] (any strides)."""
    M, K = a.shape
    N = b.shape[0]
    c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    fp8_blockscaled_gemm(M, N, K, a, a.stride(0), sa, sa.stride(0), sa.stride(1), b, b.stride(0), sb, sb.stride(0),
                         sb.stride(1), bscale, c, c.stride(0), OUT_FP32 if out_dtype == torch.float32 else OUT_BF16)
    return c


def linear_forward(x: torch.Tensor, w: torch.Tensor, out_dtype=torch.bfloat16):
    """Y = X W^T of the block-wise FP8 linear layer: X [T, in] in 1x128 groups
    and W [out, in] in 128x128 blocks (one launch), then the block-scaled GEMM.
    Returns (y, saved); saved = (qw, sw, x) is what linear_backward reads: the
    weight's codes and scales (dgrad's operand is their transpose) and the
    bf16 activation (quantized along tokens for wgrad)."""
    qx, sx, qw, sw = quant_linear(x, w)
    return gemm(qx, sx, qw, sw, BSCALE_BLOCK128, out_dtype), (qw, sw, x)


def linear_backward(dy: torch.Tensor, saved):
    """dX = dY W and dW = dY^T X, both fp32, of the layer linear_forward ran:
    dY [T, out] in 1x128 groups (dgrad) and 128x1 groups along tokens (wgrad)
    from one read, X in 128x1 groups along tokens, and W^T as the transposed
    copy of the forward's codes with W's 128x128 scales read transposed."""
    qw, sw, x = saved
    assert dy.dtype == torch.bfloat16 and dy.dim() == 2 and dy.is_contiguous()
    T, O = dy.shape
    I = x.shape[1]
    qdy, sdy, qdyt, sdyt = quant_dual_axis(dy)
    qxt, sxt = quant_rowblock(x, AXIS_COL, "m_major")
    qwt = _u8((I, O), dy.device)
    fp8_transpose_codes(qw, 1, O, I, qw.stride(0), qwt, O)
    dx = gemm(qdy, sdy, qwt, sw.t(), BSCALE_BLOCK128, torch.float32)
    dw = gemm(qdyt, sdyt, qxt, sxt, BSCALE_ROW128, torch.float32)
    return dx, dw


def moe_forward(x, qgu, sgu, qdt, sdt, offsets, row_token, token_rows, weights, out_dtype=torch.bfloat16):
    """One block-wise FP8 MoE layer forward: X [T, H] in 1x128 groups; the
    grouped gate/up GEMM over the experts' rows (gathered by row_token), with
    SiLU*mul and the 1x128 requantization of h in its epilogue; the grouped
    down GEMM; the routing-weighted combine.  Weights come quantized:
    qgu [G, 2I, H] codes with sgu [G, 2I/128, H/128] (gate rows [0, I), up
    rows [I, 2I)), qdt [G, H, I] codes of the down weights ([out][in]) with
    sdt [G, I/128, H/128] (the blocks of the [in][out] stack, read transposed).
    offsets int32 [G + 1] (device), row_token int32 [rows], token_rows int32
    [T, k] (grouped row of each token's slot), weights fp32 [T, k]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    T, H = x.shape
    G, N2, _ = qgu.shape
    I = N2 // 2
    rows = row_token.numel()
    qx, sx = quant_rowblock(x, AXIS_ROW, "m_major")
    qh = _u8((rows, I), x.device)
    shb = torch.empty((I // 128, rows), dtype=torch.float32, device=x.device)
    fp8_grouped_gemm_swiglu_quant(rows, I, H, G, offsets, row_token, T, qx, H, sx, sx.stride(0), sx.stride(1), qgu, H,
                                  N2 * H, sgu, sgu.stride(0), sgu.stride(1), sgu.stride(2), qh, I, shb, 1, rows)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=x.device)
    fp8_grouped_gemm(rows, H, I, G, offsets, None, rows, qh, I, shb, 1, rows, qdt, I, H * I, sdt, sdt.stride(0),
                     sdt.stride(2), sdt.stride(1), y, H, OUT_BF16)
    k = token_rows.shape[1]
    out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    fp8_moe_combine(y, rows, H, H, token_rows.contiguous(), weights.contiguous(), T, k, out, H,
                    OUT_FP32 if out_dtype == torch.float32 else OUT_BF16)
    return out


def gemm_splitk(a, sa, b, sb, bscale=BSCALE_BLOCK128, out_dtype=torch.bfloat16, splits=0):
    """gemm() with the K slices split among grid rows (splits 0: the
    planner's count); the fp32 workspace is allocated here with torch."""
    M, K = a.shape
    N = b.shape[0]
    out = OUT_FP32 if out_dtype == torch.float32 else OUT_BF16
    if splits == 0:
        splits, _ = fp8_blockscaled_gemm_splitk_plan(M, N, K, out)
    ws = torch.empty(max(splits, 1) * M * N if splits > 1 else 4, dtype=torch.float32, device=a.device)
    c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    fp8_blockscaled_gemm_splitk(M, N, K, a, a.stride(0), sa, sa.stride(0), sa.stride(1), b, b.stride(0), sb,
                                sb.stride(0), sb.stride(1), bscale, c, c.stride(0), out, splits, ws,
                                ws.numel() * 4)
    return c


def mx_quant(x: torch.Tensor):
    """MXFP8 1x32 quantization of bf16 [rows, cols] -> (q, s [rows, cols/32] uint8)."""
    rows, cols = x.shape
    q = _u8((rows, cols), x.device)
    s = _u8((rows, cols // 32), x.device)
    mxfp8_quant(x, rows, cols, x.stride(0), q, cols, s, cols // 32, 1)
    return q, s


def moe_combine(y: torch.Tensor, token_rows: torch.Tensor, weights: torch.Tensor, out_dtype=torch.bfloat16):
    """out[t] = sum_j weights[t, j] * y[token_rows[t, j]] for y bf16 [rows, H],
    token_rows int32 [T, k], weights fp32 [T, k]."""
    rows, H = y.shape
    T, k = token_rows.shape
    out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    fp8_moe_combine(y, rows, H, y.stride(0), token_rows.contiguous(), weights.contiguous(), T, k, out, H,
                    OUT_FP32 if out_dtype == torch.float32 else OUT_BF16)
    return out


def mx_quant_t(x: torch.Tensor):
    """MXFP8 32x1 quantization along the rows of bf16 [rows, cols], written
    transposed -> (qt [cols, rows], s [cols, rows/32] uint8)."""
    rows, cols = x.shape
    qt = _u8((cols, rows), x.device)
    s = _u8((cols, rows // 32), x.device)
    mxfp8_quant_t(x, rows, cols, x.stride(0), qt, rows, s, rows // 32, 1)
    return qt, s


def mx_gemm(a, sa, b, sb, out_dtype=torch.float32):
    """Dense MXFP8 GEMM C = A B^T: a [M, K], b [N, K] codes, sa [M, K/32],
    sb [N, K/32] UE8M0 bytes (row-major)."""
    M, K = a.shape
    N = b.shape[0]
    c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    mxfp8_gemm(M, N, K, 0, None, None, M, a, a.stride(0), sa, sa.stride(0), b, b.stride(0), 0, sb, sb.stride(0), 0,
               c, N, OUT_FP32 if out_dtype == torch.float32 else OUT_BF16)
    return c


def quant_pow2(x: torch.Tensor, block_rows: int):
    """Power-of-two-scale quantization of bf16 [rows, cols] in 1x128
    (block_rows 1) or 128x128 (128) groups -> (q, s) with s a
    [row groups, ld_s] uint8 buffer, ld_s = 4 * ceil(cols / 512) (the GEMM's
    layout); s[:, :ceil(cols/128)] holds the bytes."""
    rows, cols = x.shape
    q = _u8((rows, cols), x.device)
    ld_s = 4 * ((cols + 511) // 512)
    s = torch.zeros(((rows + block_rows - 1) // block_rows, ld_s), dtype=torch.uint8, device=x.device)
    fp8_quant_pow2(x, rows, cols, x.stride(0), block_rows, q, cols, s, ld_s)
    return q, s


def gemm_pow2(a, sa, b, sb, out_dtype=torch.bfloat16):
    """C = A B^T with power-of-two scale bytes sa [M, lds_a], sb [N/128, lds_b]."""
    M, K = a.shape
    N = b.shape[0]
    c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    fp8_blockscaled_gemm_pow2(M, N, K, a, a.stride(0), sa, sa.stride(0), b, b.stride(0), sb, sb.stride(0), c, N,
                              OUT_FP32 if out_dtype == torch.float32 else OUT_BF16)
    return c


def e4m3_encode(v: torch.Tensor):
    out = _u8(v.shape, v.device)
    fp8bs_e4m3_encode(v.contiguous(), out, v.numel())
    return out
