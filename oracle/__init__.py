"""CPU oracle for the block-wise FP8 linear layer (test infrastructure only).

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library never loads it,
and it shares no code with the HIP path.

The arithmetic lives in ``fp8_oracle.c`` (plain scalar C, fp64 where the
method leaves the precision open).  This module only builds that file with
gcc, loads it with ctypes and marshals numpy arrays.  Every function names
the passage of the pages it follows:

* quantizer S = max|X| / V_max, Q(x) = round(x / S): "Unified FP8: Beyond Mixed
  Precision..." (winzheng.com), section "FP8 Quantization", Steps 1 and 2;
* E4M3 element format, FP32 scales: same page, sections "FP8 Format" and
  "FP8 Scale Selection";
* 128x128 blocks with FP32 scales, and 1x32 MXFP8 blocks with UE8M0 scales:
  "Low Precision RL" (miles.radixark.com), table "Choose a precision",
  sections "2. Unified block-wise FP8 (DeepSeek-style)" and
  "3. Unified MXFP8 (Blackwell)".

Parity pins (tests/test_oracle_*.py) tie each function to closed forms,
invariants, brute force and an independent library cast; no function here is
left "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
GCC_FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-Wall", "-shared", "-fPIC"]
# FP8_ORACLE_SANITIZE=1 selects a second build of the same source with
# AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the
# process must preload the ASan runtime, see tests/test_oracle_sanitized.py).
SANITIZE = os.environ.get("FP8_ORACLE_SANITIZE", "") == "1"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
_LIB_PATH = os.path.join(_HERE, "libfp8_oracle_san.so" if SANITIZE else "libfp8_oracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile fp8_oracle.c into libfp8_oracle.so with gcc (no HIP)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, *(SANITIZE_FLAGS if SANITIZE else []), _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.or_e4m3_decode.restype = ctypes.c_double
        lib.or_e4m3_encode.argtypes = [ctypes.c_float]
        lib.or_e4m3_encode.restype = ctypes.c_uint8
        lib.or_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.or_f32_to_bf16.restype = ctypes.c_uint16
        lib.or_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.or_f64_to_bf16.restype = ctypes.c_uint16
        lib.or_mx_exponent.argtypes = [ctypes.c_float]
        lib.or_mx_exponent.restype = ctypes.c_int
        lib.or_ue8m0_decode.argtypes = [ctypes.c_uint8]
        lib.or_ue8m0_decode.restype = ctypes.c_double
        for name in ("or_quant_1x128", "or_quant_128x1_t", "or_quant_128x128", "or_mx_quant_1x32"):
            getattr(lib, name).argtypes = [P, I64, I64, I64, P, P]
            getattr(lib, name).restype = None
        lib.or_gemm_blockscaled.argtypes = [I64, I64, I64, P, I64, P, I64, I64,
                                            P, I64, P, I64, I64, ctypes.c_int, P, P]
        lib.or_gemm_blockscaled.restype = None
        lib.or_gemm_blockscaled_sampled.argtypes = [I64, P, I64, P, I64, I64, P, I64, P, I64, I64,
                                                    ctypes.c_int, P, P, I64, P, P]
        lib.or_gemm_blockscaled_sampled.restype = None
        lib.or_gemm_mx_sampled.argtypes = [I64, P, I64, P, I64, P, I64, P, I64, P, P, I64, P, P]
        lib.or_gemm_mx_sampled.restype = None
        lib.or_silu_mul.argtypes = [P, I64, I64, I64, P]
        lib.or_silu_mul.restype = None
        lib.or_quant_pow2.argtypes = [P, I64, I64, I64, I64, P, P, I64]
        lib.or_quant_pow2.restype = None
        lib.or_moe_combine.argtypes = [P, I64, I64, P, P, I64, I64, P]
        lib.or_moe_combine.restype = None
        lib.or_num_threads.argtypes = []
        lib.or_num_threads.restype = ctypes.c_int
        lib.or_set_num_threads.argtypes = [ctypes.c_int]
        lib.or_set_num_threads.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _bf16_view(x) -> np.ndarray:
    """Accept a uint16 array (bf16 bit patterns) and return it C-contiguous."""
    x = np.asarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % x.dtype)
    return np.ascontiguousarray(x)


def num_threads() -> int:
    return _load().or_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (results are independent of it)."""
    _load().or_set_num_threads(int(n))


# ---------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3FN decode of uint8 codes to float64 (NaN for 0x7F/0xFF)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.or_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def e4m3_encode(values) -> np.ndarray:
    """E4M3 encode of float32 values: RNE, saturating to +-448, NaN -> 0x7F|s."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32)
    flat = v.reshape(-1)
    out = np.fromiter((lib.or_e4m3_encode(float(x)) for x in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(v.shape)


def ue8m0_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.or_ue8m0_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def mx_exponent(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e, clamped to [-127, 127] (-127 for 0)."""
    return _load().or_mx_exponent(float(np.float32(amax)))


def f64_to_bf16(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.fromiter((lib.or_f64_to_bf16(float(x)) for x in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(v.shape)


def bf16_to_f32(x) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    x = np.asarray(x, dtype=np.uint16)
    return (x.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- quantizers
def quant_1x128(x):
    """Per-token 1x128 groups along the contiguous axis.  x: [rows, cols] bf16
    bits -> (q [rows, cols] uint8, s [rows, ceil(cols/128)] float32)."""
    x = _bf16_view(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, (cols + 127) // 128), np.float32)
    _load().or_quant_1x128(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s))
    return q, s


def quant_128x1_t(x):
    """128x1 groups along the row (token) axis, transposed output.
    x: [rows, cols] -> (qt [cols, rows], s [cols, ceil(rows/128)])."""
    x = _bf16_view(x)
    rows, cols = x.shape
    qt = np.empty((cols, rows), np.uint8)
    s = np.empty((cols, (rows + 127) // 128), np.float32)
    _load().or_quant_128x1_t(_ptr(x), rows, cols, cols, _ptr(qt), _ptr(s))
    return qt, s


def quant_128x128(x):
    """128x128 blocks.  x: [rows, cols] -> (q [rows, cols],
    s [ceil(rows/128), ceil(cols/128)])."""
    x = _bf16_view(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(((rows + 127) // 128, (cols + 127) // 128), np.float32)
    _load().or_quant_128x128(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s))
    return q, s


def quant_rowwise(x):
    """One group per row (rowwise scaling; the tensorwise/rowwise comparison
    of "Towards Full Pipeline FP8 Reinforcement Learning for LLMs").
    x: [rows, cols] -> (q [rows, cols], s [rows] float32)."""
    x = _bf16_view(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows,), np.float32)
    _load().or_quant_rowwise(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s))
    return q, s


def quant_tensorwise(x):
    """One group for the whole tensor ("per-tensor", "Unified FP8...",
    section "FP8 Quantization").  x: [rows, cols] -> (q [rows, cols],
    s [1] float32)."""
    x = _bf16_view(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((1,), np.float32)
    _load().or_quant_tensorwise(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s))
    return q, s


def mx_quant_1x32(x):
    """MXFP8: 1x32 blocks along the contiguous axis, UE8M0 codes.
    x: [rows, cols] -> (q [rows, cols], s [rows, ceil(cols/32)] uint8)."""
    x = _bf16_view(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, (cols + 31) // 32), np.uint8)
    _load().or_mx_quant_1x32(_ptr(x), rows, cols, cols, _ptr(q), _ptr(s))
    return q, s


# ---------------------------------------------------------------- GEMMs
BSCALE_BLOCK128 = 0   # sb[n // 128, k // 128]
BSCALE_ROW128 = 1     # sb[n, k // 128]


def _quant_pow2(x, block_rows):
    x = _bf16_view(x)
    rows, cols = x.shape
    ngr, ngc = (rows + block_rows - 1) // block_rows, (cols + 127) // 128
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((ngr, ngc), np.uint8)
    _load().or_quant_pow2(_ptr(x), rows, cols, cols, block_rows, _ptr(q), _ptr(s), ngc)
    return q, s


def quant_1x128_pow2(x):
    """1x128 groups with power-of-two scales: the group's scale is rounded up
    to a power of two (the MX exponent rule on the 128-element group), kept
    as a UE8M0 byte; "Low Precision RL", section "2. Unified block-wise FP8
    (DeepSeek-style)": the block-wise recipe with power-of-two scales, as
    TransformerEngine runs it on Blackwell through MXFP8.  x: [rows, cols] ->
    (q [rows, cols], s [rows, ceil(cols/128)] uint8)."""
    return _quant_pow2(x, 1)


def quant_128x128_pow2(x):
    """128x128 blocks with power-of-two UE8M0 scales (see quant_1x128_pow2).
    x: [rows, cols] -> (q, s [ceil(rows/128), ceil(cols/128)] uint8)."""
    return _quant_pow2(x, 128)


def pow2_scales(s):
    """UE8M0 scale bytes -> their float32 values 2^(c - 127) (exact)."""
    return ue8m0_decode(np.asarray(s, np.uint8)).astype(np.float32)


def mx_quant_32x1_t(x):
    """MXFP8 blocks of 32 consecutive values down each column, written
    transposed: the 1x32 quantization of the transpose (the operand layout of
    the MXFP8 weight- and data-gradient GEMMs, "Low Precision RL", section
    "3. Unified MXFP8 (Blackwell)").  x: [rows, cols] -> (qt [cols, rows],
    s [cols, rows/32] uint8)."""
    return mx_quant_1x32(np.ascontiguousarray(_bf16_view(x).T))


def _f32c(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def gemm_blockscaled(qa, sa, qb, sb, bmode=BSCALE_BLOCK128, with_abs=True):
    """Reference Y = A~ . B~^T in fp64 on dequantized operands.

    qa [M, K] codes, sa [M, K/128]; qb [N, K] codes, sb [N/128, K/128] (bmode
    BLOCK128) or [N, K/128] (ROW128).  Returns (Y [M, N] f64, Babs or None)
    where Babs = sum_k |A~ B~|."""
    qa = np.ascontiguousarray(qa, np.uint8)
    qb = np.ascontiguousarray(qb, np.uint8)
    sa = _f32c(sa)
    sb = _f32c(sb)
    M, K = qa.shape
    N = qb.shape[0]
    assert qb.shape[1] == K and sa.shape == (M, (K + 127) // 128)
    y = np.empty((M, N), np.float64)
    yabs = np.empty((M, N), np.float64) if with_abs else None
    _load().or_gemm_blockscaled(M, N, K, _ptr(qa), K, _ptr(sa), sa.shape[1], 1,
                                _ptr(qb), K, _ptr(sb), sb.shape[1], 1, int(bmode),
                                _ptr(y), _ptr(yabs) if with_abs else None)
    return y, yabs


def gemm_blockscaled_sampled(qa, sa, qb, sb, mi, ni, bmode=BSCALE_BLOCK128):
    """The same reference on selected outputs (mi[i], ni[i]) only."""
    qa = np.ascontiguousarray(qa, np.uint8)
    qb = np.ascontiguousarray(qb, np.uint8)
    sa = _f32c(sa)
    sb = _f32c(sb)
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    K = qa.shape[1]
    y = np.empty(mi.size, np.float64)
    yabs = np.empty(mi.size, np.float64)
    _load().or_gemm_blockscaled_sampled(K, _ptr(qa), K, _ptr(sa), sa.shape[1], 1,
                                        _ptr(qb), K, _ptr(sb), sb.shape[1], 1, int(bmode),
                                        _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(yabs))
    return y, yabs


def expand_rowscales(sa, sb, M, N, K):
    """Scales constant along K (rowwise: sa [M], sb [N]; tensorwise: one value
    each) written out per 128-wide K slice, as the block-scaled GEMM takes
    them: (sa [M, K/128], sb [N, K/128]) for BSCALE_ROW128."""
    nk = K // 128
    sa = np.broadcast_to(np.asarray(sa, np.float32).reshape(-1, 1), (M, nk))
    sb = np.broadcast_to(np.asarray(sb, np.float32).reshape(-1, 1), (N, nk))
    return np.ascontiguousarray(sa), np.ascontiguousarray(sb)


def gemm_rowscaled(qa, sa, qb, sb, with_abs=True):
    """GEMM with scales constant along K: Y[m,n] = sa[m] sb[n] sum_k
    dec(qa[m,k]) dec(qb[n,k]) (sa, sb of length M and N, or 1 for a
    tensorwise scale).  It is the block-scaled GEMM whose per-slice scales are
    the same in every slice."""
    M, K = qa.shape
    N = qb.shape[0]
    sae, sbe = expand_rowscales(sa, sb, M, N, K)
    return gemm_blockscaled(qa, sae, qb, sbe, BSCALE_ROW128, with_abs)


def gemm_mx_sampled(qa, sa, qb, sb, mi, ni):
    """MXFP8 reference on selected outputs.  sa [M, K/32], sb [N, K/32] UE8M0."""
    qa = np.ascontiguousarray(qa, np.uint8)
    qb = np.ascontiguousarray(qb, np.uint8)
    sa = np.ascontiguousarray(sa, np.uint8)
    sb = np.ascontiguousarray(sb, np.uint8)
    mi = np.ascontiguousarray(mi, np.int64)
    ni = np.ascontiguousarray(ni, np.int64)
    K = qa.shape[1]
    y = np.empty(mi.size, np.float64)
    yabs = np.empty(mi.size, np.float64)
    _load().or_gemm_mx_sampled(K, _ptr(qa), K, _ptr(sa), sa.shape[1], _ptr(qb), K, _ptr(sb),
                               sb.shape[1], _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(yabs))
    return y, yabs


def gemm_mx(qa, sa, qb, sb):
    """Full MXFP8 reference GEMM (small shapes): returns (Y, Babs)."""
    M, N = qa.shape[0], qb.shape[0]
    mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, yabs = gemm_mx_sampled(qa, sa, qb, sb, mi.reshape(-1), ni.reshape(-1))
    return y.reshape(M, N), yabs.reshape(M, N)


# ---------------------------------------------------------------- MoE pieces
def silu_mul(gate_up):
    """h = bf16(silu(g) * u) with g = columns [0, I), u = columns [I, 2I)."""
    gu = _bf16_view(gate_up)
    rows, two_i = gu.shape
    I = two_i // 2
    h = np.empty((rows, I), np.uint16)
    _load().or_silu_mul(_ptr(gu), rows, I, two_i, _ptr(h))
    return h


def grouped_gemm_blockscaled(qa, sa, offsets, qb, sb):
    """Grouped (MoE) reference: rows offsets[g]:offsets[g+1] of A times expert
    g's B [N, K] with 128x128 scales sb[g].  Each group is the dense reference
    above; empty groups contribute nothing.  Returns (Y [rows, N], Babs)."""
    rows, K = qa.shape
    G, N, _ = qb.shape
    y = np.zeros((rows, N), np.float64)
    yabs = np.zeros((rows, N), np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            y[r0:r1], yabs[r0:r1] = gemm_blockscaled(qa[r0:r1], sa[r0:r1], qb[g], sb[g])
    return y, yabs


def moe_combine(y, pos, w):
    """MoE combine: out[t] = sum_j w[t, j] * y[pos[t, j]] in fp64 (the
    weighted sum of a token's expert outputs that closes the MoE layer whose
    grouped GEMMs "Low Precision RL" runs in FP8, section "2. Unified
    block-wise FP8 (DeepSeek-style)", Qwen3-30B-A3B).  y: [rows, H] bf16 bit
    patterns in grouped order; pos: [T, k] int grouped rows; w: [T, k] fp32.
    Returns [T, H] float64."""
    y = _bf16_view(y)
    pos = np.ascontiguousarray(pos, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, k = pos.shape
    assert w.shape == (T, k) and y.ndim == 2
    assert pos.size == 0 or (pos.min() >= 0 and pos.max() < y.shape[0])
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    _load().or_moe_combine(_ptr(y), H, H, _ptr(pos), _ptr(w), T, k, _ptr(out))
    return out
