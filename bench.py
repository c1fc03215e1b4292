"""Benchmark of the block-wise FP8 linear layer on one MI355X.

Headline step: the Qwen3-4B MLP forward with the block-wise FP8 recipe,
every part on the GPU through the C ABI:
    quantize X_up [4096 x 2560] per token (1x128) and W_up [9728 x 2560] in
    128x128 blocks (one fp8_quant_linear launch), GEMM up (bf16 out),
    quantize X_down [4096 x 9728] and W_down [2560 x 9728] (one launch),
    GEMM down (bf16 out).
Inputs are seeded synthetic tensors (see fp8_block_scaled_x128_amd.inputs),
resident in HBM before timing; activations rotate over several copies so
that the 256 MB last-level cache cannot serve them.

The other workloads of the path are timed after it (median of --reps
repetitions, each kernel bracketed by HIP events on the launch stream):
    tiny_linear      X [256 x 512], W [512 x 512] (quantizers, GEMM bf16/fp32)
    mlp_backward     dY [4096 x 9728]: 1x128 and 128x1 quantization in one pass, X 128x1,
                     the transposed copy of the forward's W codes, dgrad and wgrad
                     GEMMs (fp32 out)
    moe_blockwise    Qwen3-30B-A3B MoE layer (16384 tokens, 128 experts, top 8):
                     X 1x128, W_gu / W_d 128x128, grouped gate_up GEMM, SiLU*mul
                     + 1x128 requantization, grouped down GEMM, combine
    moe_blockwise_fused  the same layer with SiLU*mul and the requantization
                     in the gate_up GEMM's epilogue
    moe_mxfp8        the layer in MXFP8 (1x32 UE8M0 blocks)
    moe_mxfp8_fused  the MXFP8 layer with the fused gate_up epilogue

Prints ONE JSON line: value = GEMM FLOPs of the headline step / step time
(TFLOP/s); per-kernel times with TFLOP/s or GB/s against MI355X's peaks (GB/s
figures also against a timed 512 MiB device copy, copy_context); a roofline
object for the dominant kernel (the block-scaled GEMM); a CPU-oracle baseline
on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5030.0     # 256 CUs x 2.4 GHz x 8192 dense FP8 flop/clk/CU
PEAK_HBM_GBS = 8000.0
M_TOK, HID, INTER = 4096, 2560, 9728
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic.json")
WORKLOADS = ("tiny_linear", "mlp_backward", "mlp_backward_mxfp8", "moe_blockwise", "moe_blockwise_fused", "moe_mxfp8",
             "moe_mxfp8_fused", "up_proj_rowwise",
             "up_proj_pow2")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the shader clock takes tens of milliseconds of sustained load to settle
    # (GEMM time falls by 10-20% over the first ~10 ms): 200 untimed steps
    # (about 70 ms) come first
    ap.add_argument("--warmup", type=int, default=200)
    # before the counted warm-up steps, step passes run for at least this long
    # so that a short --warmup still times the settled clock
    ap.add_argument("--settle-ms", type=float, default=300.0)
    ap.add_argument("--batch", type=int, default=10,
                    help="back-to-back launches per event pair in the per-kernel pass")
    ap.add_argument("--copies", type=int, default=4, help="activation copies rotated across steps")
    ap.add_argument("--reps", type=int, default=10, help="repetitions per kernel of the other workloads")
    ap.add_argument("--warm-ms", type=float, default=60.0, help="warm-up of each other workload (ms)")
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="other workloads to time after the headline step (comma list, or 'none')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=288, help="token rows in the CPU-oracle sample")
    ap.add_argument("--cpu-rows-1t", type=int, default=24, help="token rows in the one-thread CPU-oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB 3 times (counter calibration)")
    return ap.parse_args()


def qbytes_row(rows, cols, group=128, scale_bytes=4):
    """Quantizer algorithmic bytes: bf16 in, one code byte out, one scale per group."""
    return rows * cols * 3 + rows * ((cols + group - 1) // group) * scale_bytes


def qbytes_dual(rows, cols, group=128, scale_bytes=4):
    """Both axes from one read: bf16 in once, codes and scales of the row
    groups and of the column groups out."""
    return rows * cols * 4 + (rows * ((cols + group - 1) // group) + cols * ((rows + group - 1) // group)) * scale_bytes


def qbytes_block2d(batch, rows, cols, transposed=False):
    return batch * (rows * cols * (4 if transposed else 3) + ((rows + 127) // 128) * ((cols + 127) // 128) * 4)


def combine_bytes(rows, H, T, k):
    """MoE combine: every grouped row read once (bf16), one bf16 row written
    per token, and the token's k positions and weights."""
    return rows * H * 2 + T * H * 2 + T * k * 8


def rate(unit, amount, ms):
    if unit == "TFLOP/s":
        r = amount / (ms * 1e-3) / 1e12
        return r, r / PEAK_FP8_TFLOPS
    r = amount / (ms * 1e-3) / 1e9
    return r, r / PEAK_HBM_GBS


def kernel_entry(unit, amount, ms, p10=None, p90=None):
    """Median time with its rate and fraction of peak; p10 and p90 of the
    timed repetitions beside it."""
    r, f = rate(unit, amount, ms)
    e = {"ms": round(ms, 5), unit: round(r, 2), "frac_of_peak": round(f, 4)}
    if p10 is not None:
        e["ms_p10"], e["ms_p90"] = round(p10, 5), round(p90, 5)
    return e


def spread(times):
    """(median, p10, p90) of a list of durations."""
    t = np.asarray(times, dtype=np.float64)
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def time_sequence(torch, stream, launches, reps, warmup, warm_ms=60.0):
    """Run the list of launches at least `warmup` times and for at least
    `warm_ms` of wall time (the shader clock settles under sustained load),
    then `reps` times with each launch bracketed by events; returns the
    per-launch (median, p10, p90) ms."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        for fn in launches:
            fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(reps)]
    for i in range(reps):
        for k, fn in enumerate(launches):
            ev[i][k].record(stream)
            fn(i)
        ev[i][len(launches)].record(stream)
    torch.cuda.synchronize()
    return [spread([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(reps)]) for k in range(len(launches))]


class ClockSampler:
    """Samples the GPU shader clock (the current DPM level of the sclk table
    in sysfs, MHz) from a host thread while the GPU runs.  A sample is the
    clock the power manager set; under a matrix-heavy load it drops below the
    2.4 GHz the peak figures assume.  source is None where no readable sysfs
    clock exists (then sclk_mhz_timed_region is null)."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.period = period_s
        self.samples = []
        self.mark_at = 0
        self.source = None
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            if self._read(f) is not None:
                self.source = f
                break
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split()[0].lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read(self.source)
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def start(self):
        if self.source:
            self._thr.start()

    def mark(self):
        self.mark_at = len(self.samples)

    def since_mark(self):
        s = self.samples[self.mark_at:]
        return round(float(np.median(s)), 1) if s else None

    def stop(self):
        self._stop.set()
        if self._thr.is_alive():
            self._thr.join()


# ------------------------------------------------------------- workloads
def wl_tiny_linear(torch, ops, inputs, to_dev, R):
    d = inputs.tiny_linear(0)
    M, K = d["x"].shape
    N = d["w"].shape[0]
    xs = [to_dev(d["x"]) for _ in range(R)]
    w = to_dev(d["w"])
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    gemm = lambda c, out: ops.fp8_blockscaled_gemm(M, N, K, qx, K, sx, 1, M, qw, K, sw, K // 128, 1,
                                                   ops.BSCALE_BLOCK128, c, N, out)
    return [
        ("quant_x_1x128", lambda i: ops.fp8_quant_rowblock(xs[i % R], M, K, K, ops.AXIS_ROW, qx, K, sx, 1, M),
         ("GB/s", qbytes_row(M, K))),
        ("quant_w_128x128", lambda i: ops.fp8_quant_block2d(w, 1, N, K, K, qw, K, None, 0, sw),
         ("GB/s", qbytes_block2d(1, N, K))),
        ("gemm_bf16", lambda i: gemm(y16, ops.OUT_BF16), ("TFLOP/s", 2.0 * M * N * K)),
        ("gemm_fp32", lambda i: gemm(y32, ops.OUT_FP32), ("TFLOP/s", 2.0 * M * N * K)),
    ], {"workload": "tiny_linear", "tokens": M, "in": K, "out": N, "seed": 0}


def wl_mlp_backward(torch, ops, inputs, to_dev, R):
    d = inputs.qwen3_4b_mlp_backward(2)
    T, O = d["dy"].shape
    I = d["x"].shape[1]
    dys = [to_dev(d["dy"]) for _ in range(R)]
    xs = [to_dev(d["x"]) for _ in range(R)]
    w = to_dev(d["w"])
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    qdy, sdy = u8(T, O), f32(O // 128, T)                  # 1x128, M-major scales
    qdyt, sdyt = u8(O, T), f32(T // 128, O)                # 128x1 along tokens, transposed codes
    qxt, sxt = u8(I, T), f32(T // 128, I)
    qwt, sw = u8(I, O), f32(O // 128, I // 128)
    # W's 128x128 codes and scales as the forward step leaves them (its
    # fp8_quant_linear); the backward needs their transposed copy
    qw = u8(O, I)
    ops.fp8_quant_block2d(w, 1, O, I, I, qw, I, None, 0, sw)
    dx = torch.empty((T, I), dtype=torch.float32, device="cuda")
    dw = torch.empty((O, I), dtype=torch.float32, device="cuda")
    return [
        # dY in 1x128 groups (dgrad) and 128x1 groups along tokens (wgrad) from one read
        ("quant_dy_dual_axis", lambda i: ops.fp8_quant_dual_axis(dys[i % R], T, O, O, 0, qdy, O, sdy, 1, T, qdyt, T,
                                                                 sdyt, 1, O),
         ("GB/s", qbytes_dual(T, O))),
        ("quant_x_128x1", lambda i: ops.fp8_quant_rowblock(xs[i % R], T, I, I, ops.AXIS_COL, qxt, T, sxt, 1, I),
         ("GB/s", qbytes_row(I, T))),
        # dgrad reads W through the transposed copy of the forward's codes (128x128 blocks are
        # transpose-invariant: the same scales, read with swapped strides)
        ("transpose_w_codes", lambda i: ops.fp8_transpose_codes(qw, 1, O, I, I, qwt, O), ("GB/s", 2 * O * I)),
        # dX [T, I] = dY [T, O] W [O, I]: B = W^T codes [I, O], scales sw read transposed
        ("gemm_dgrad_fp32", lambda i: ops.fp8_blockscaled_gemm(T, I, O, qdy, O, sdy, 1, T, qwt, O, sw, 1, I // 128,
                                                              ops.BSCALE_BLOCK128, dx, I, ops.OUT_FP32),
         ("TFLOP/s", 2.0 * T * I * O)),
        # dW [O, I] = dY^T [O, T] X [T, I]: both 128x1 along tokens, per-row B scales
        ("gemm_wgrad_fp32", lambda i: ops.fp8_blockscaled_gemm(O, I, T, qdyt, T, sdyt, 1, O, qxt, T, sxt, 1, I,
                                                              ops.BSCALE_ROW128, dw, I, ops.OUT_FP32),
         ("TFLOP/s", 2.0 * O * I * T)),
    ], {"workload": "mlp_backward", "tokens": T, "hidden": I, "intermediate": O, "seeds": [1, 2]}


def wl_up_proj_rowwise(torch, ops, inputs, to_dev, R):
    """The up projection of the headline step with rowwise and tensorwise
    scales instead of 1x128 / 128x128 blocks."""
    d = inputs.qwen3_4b_mlp(1)
    M, K, N = M_TOK, HID, INTER
    xs = [to_dev(d["x_up"]) for _ in range(R)]
    w = to_dev(d["w_up"])
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    qx, sx, qw, sw, st = u8(M, K), f32(M), u8(N, K), f32(N), f32(1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    return [
        ("quant_x_rowwise", lambda i: ops.fp8_quant_rowwise(xs[i % R], M, K, K, qx, K, sx),
         ("GB/s", qbytes_row(M, K, group=K))),
        ("quant_x_tensorwise", lambda i: ops.fp8_quant_tensorwise(xs[i % R], M, K, K, qx, K, st),
         ("GB/s", M * K * 3 + 4)),
        ("quant_w_rowwise", lambda i: ops.fp8_quant_rowwise(w, N, K, K, qw, K, sw),
         ("GB/s", qbytes_row(N, K, group=K))),
        # scales constant along K: views of K stride 0
        ("gemm_rowscaled_bf16", lambda i: ops.fp8_blockscaled_gemm(M, N, K, qx, K, sx, 1, 0, qw, K, sw, 1, 0,
                                                                  ops.BSCALE_ROW128, y, N, ops.OUT_BF16),
         ("TFLOP/s", 2.0 * M * N * K)),
    ], {"workload": "up_proj_rowwise", "tokens": M, "in": K, "out": N, "seed": 1}


def wl_mlp_backward_mxfp8(torch, ops, inputs, to_dev, R):
    """The backward GEMMs of mlp_backward in MXFP8: dY 1x32 along O for
    dgrad and 32x1 along tokens (transposed) for wgrad, in one pass; W
    re-quantized 32x1 along O (transposed) and X 32x1 along tokens."""
    d = inputs.qwen3_4b_mlp_backward(2)
    T, O = d["dy"].shape
    I = d["x"].shape[1]
    dys = [to_dev(d["dy"]) for _ in range(R)]
    xs = [to_dev(d["x"]) for _ in range(R)]
    w = to_dev(d["w"])
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    qdy, sdy = u8(T, O), u8(T, O // 32)
    qdyt, sdyt = u8(O, T), u8(O, T // 32)
    qxt, sxt = u8(I, T), u8(I, T // 32)
    qwt, swt = u8(I, O), u8(I, O // 32)
    dx = torch.empty((T, I), dtype=torch.float32, device="cuda")
    dw = torch.empty((O, I), dtype=torch.float32, device="cuda")
    return [
        ("mx_quant_dy_dual_axis", lambda i: ops.fp8_quant_dual_axis(dys[i % R], T, O, O, 1, qdy, O, sdy, O // 32, 1,
                                                                    qdyt, T, sdyt, T // 32, 1),
         ("GB/s", qbytes_dual(T, O, 32, 1))),
        ("mx_quant_x_t", lambda i: ops.mxfp8_quant_t(xs[i % R], T, I, I, qxt, T, sxt, T // 32, 1),
         ("GB/s", qbytes_row(I, T, 32, 1))),
        ("mx_quant_w_t", lambda i: ops.mxfp8_quant_t(w, O, I, I, qwt, O, swt, O // 32, 1),
         ("GB/s", qbytes_row(I, O, 32, 1))),
        ("mx_gemm_dgrad_fp32", lambda i: ops.mxfp8_gemm(T, I, O, 0, None, None, T, qdy, O, sdy, O // 32, qwt, O, 0,
                                                       swt, O // 32, 0, dx, I, ops.OUT_FP32),
         ("TFLOP/s", 2.0 * T * I * O)),
        ("mx_gemm_wgrad_fp32", lambda i: ops.mxfp8_gemm(O, I, T, 0, None, None, O, qdyt, T, sdyt, T // 32, qxt, T, 0,
                                                       sxt, T // 32, 0, dw, I, ops.OUT_FP32),
         ("TFLOP/s", 2.0 * O * I * T)),
    ], {"workload": "mlp_backward_mxfp8", "tokens": T, "hidden": I, "intermediate": O, "seeds": [1, 2]}


def wl_up_proj_pow2(torch, ops, inputs, to_dev, R):
    """The up projection of the headline step with power-of-two (UE8M0)
    block scales: 1x128 activation groups, 128x128 weight blocks, the GEMM
    applying the scales inside the scaled matrix instruction."""
    d = inputs.qwen3_4b_mlp(1, parts=("up",))
    M, K, N = M_TOK, HID, INTER
    xs = [to_dev(d["x_up"]) for _ in range(R)]
    w = to_dev(d["w_up"])
    lds = 4 * ((K + 511) // 512)
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8, device="cuda")
    qx, sx, qw, sw = u8(M, K), u8(M, lds), u8(N, K), u8(N // 128, lds)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    return [
        # X in 1x128 groups and W in 128x128 blocks, one launch, as fp8_quant_linear with FP32 scales
        ("quant_linear_pow2", lambda i: ops.fp8_quant_linear_pow2(xs[i % R], M, K, K, qx, K, sx, lds, w, N, K, qw, K,
                                                                 sw, lds),
         ("GB/s", qbytes_row(M, K, 128, 1) + N * K * 3 + (N // 128) * (K // 128))),
        ("gemm_pow2_bf16", lambda i: ops.fp8_blockscaled_gemm_pow2(M, N, K, qx, K, sx, lds, qw, K, sw, lds, y, N,
                                                                  ops.OUT_BF16),
         ("TFLOP/s", 2.0 * M * N * K)),
    ], {"workload": "up_proj_pow2", "tokens": M, "in": K, "out": N, "seed": 1}


def _moe_inputs(inputs, cache={}):
    if "d" not in cache:
        cache["d"] = inputs.qwen3_30b_a3b_moe(3)
    return cache["d"]


def wl_moe_blockwise(torch, ops, inputs, to_dev, R, fused=False):
    """The Qwen3-30B-A3B MoE layer with the block-wise recipe.  fused: the
    gate/up GEMM forms h = SiLU(gate) * up and its 1x128 codes in its
    epilogue (fp8_grouped_gemm_swiglu_quant) instead of writing bf16 gate/up
    for the separate SiLU*mul kernel."""
    d = _moe_inputs(inputs)
    r = d["routing"]
    T, H = d["x"].shape
    E, N2, _ = d["w_gu"].shape
    I = N2 // 2
    rows, G = r.row_token.size, r.offsets.size - 1
    xs = [to_dev(d["x"]) for _ in range(R)]
    wgu, wd = to_dev(d["w_gu"]), to_dev(d["w_d"])
    offs = torch.from_numpy(r.offsets).cuda()
    a_rows = torch.from_numpy(r.row_token).cuda()
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    qx, sx = u8(T, H), f32(H // 128, T)
    qgu, sgu = u8(E, N2, H), f32(E, N2 // 128, H // 128)
    qdt, sd = u8(E, H, I), f32(E, I // 128, H // 128)
    gu = None if fused else torch.empty((rows, N2), dtype=torch.bfloat16, device="cuda")
    qh, sh = u8(rows, I), f32(I // 128, rows)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    pos, wts = torch.from_numpy(r.token_rows).cuda(), torch.from_numpy(r.weights).cuda()
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    k = r.token_rows.shape[1]
    n_gu = 2.0 * rows * N2 * H
    n_dn = 2.0 * rows * H * I
    gate_up_steps = [
        ("grouped_gemm_gate_up", lambda i: ops.fp8_grouped_gemm(
            rows, N2, H, G, offs, a_rows, T, qx, H, sx, 1, T, qgu, H, N2 * H, sgu, (N2 // 128) * (H // 128),
            H // 128, 1, gu, N2, ops.OUT_BF16), ("TFLOP/s", n_gu)),
        ("silu_mul_quant_1x128", lambda i: ops.fp8_silu_mul_quant(gu, rows, I, N2, 0, qh, I, sh, 1, rows, None, 0),
         ("GB/s", rows * N2 * 2 + rows * I + rows * (I // 128) * 4)),
    ]
    if fused:
        gate_up_steps = [
            ("grouped_gemm_gate_up_swiglu_quant", lambda i: ops.fp8_grouped_gemm_swiglu_quant(
                rows, I, H, G, offs, a_rows, T, qx, H, sx, 1, T, qgu, H, N2 * H, sgu, (N2 // 128) * (H // 128),
                H // 128, 1, qh, I, sh, 1, rows), ("TFLOP/s", n_gu)),
        ]
    return [
        ("quant_x_1x128", lambda i: ops.fp8_quant_rowblock(xs[i % R], T, H, H, ops.AXIS_ROW, qx, H, sx, 1, T),
         ("GB/s", qbytes_row(T, H))),
        ("quant_w_gate_up_128x128", lambda i: ops.fp8_quant_block2d(wgu, E, N2, H, H, qgu, H, None, 0, sgu),
         ("GB/s", qbytes_block2d(E, N2, H))),
        # W_d is stored [in][out]: the down GEMM reads only its transposed codes
        ("quant_w_down_128x128_transposed", lambda i: ops.fp8_quant_block2d(wd, E, I, H, H, None, 0, qdt, I, sd),
         ("GB/s", qbytes_block2d(E, I, H))),
    ] + gate_up_steps + [
        # B[n = hidden, k = inter] = W_d[e]^T codes; scales sd[e][k/128][n/128] read transposed
        ("grouped_gemm_down", lambda i: ops.fp8_grouped_gemm(
            rows, H, I, G, offs, None, rows, qh, I, sh, 1, rows, qdt, I, H * I, sd, (I // 128) * (H // 128),
            1, H // 128, y, H, ops.OUT_BF16), ("TFLOP/s", n_dn)),
        ("combine", lambda i: ops.fp8_moe_combine(y, rows, H, H, pos, wts, T, k, out, H, ops.OUT_BF16),
         ("GB/s", combine_bytes(rows, H, T, k))),
    ], {"workload": "moe_blockwise_fused" if fused else "moe_blockwise", "tokens": T, "hidden": H, "experts": E,
        "intermediate": I, "top_k": 8,
        "grouped_rows": rows, "seed": 3}


def wl_moe_mxfp8(torch, ops, inputs, to_dev, R, fused=False):
    """The MoE layer in MXFP8.  fused: SiLU*mul and the 1x32 quantization of
    h in the gate/up GEMM's epilogue (mxfp8_grouped_gemm_swiglu_quant)."""
    d = _moe_inputs(inputs)
    r = d["routing"]
    T, H = d["x"].shape
    E, N2, _ = d["w_gu"].shape
    I = N2 // 2
    rows, G = r.row_token.size, r.offsets.size - 1
    xs = [to_dev(d["x"]) for _ in range(R)]
    wgu = to_dev(d["w_gu"]).view(E * N2, H)
    wdt = to_dev(d["w_d"]).transpose(1, 2).contiguous().view(E * H, I)   # contraction axis (inter) contiguous
    offs = torch.from_numpy(r.offsets).cuda()
    a_rows = torch.from_numpy(r.row_token).cuda()
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    qx, sx = u8(T, H), u8(T, H // 32)
    qgu, sgu = u8(E * N2, H), u8(E * N2, H // 32)
    qdt, sdt = u8(E * H, I), u8(E * H, I // 32)
    gu = None if fused else torch.empty((rows, N2), dtype=torch.bfloat16, device="cuda")
    qh, sh = u8(rows, I), u8(rows, I // 32)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    pos, wts = torch.from_numpy(r.token_rows).cuda(), torch.from_numpy(r.weights).cuda()
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    k = r.token_rows.shape[1]
    return [
        ("mx_quant_x", lambda i: ops.mxfp8_quant(xs[i % R], T, H, H, qx, H, sx, H // 32, 1),
         ("GB/s", qbytes_row(T, H, 32, 1))),
        ("mx_quant_w_gate_up", lambda i: ops.mxfp8_quant(wgu, E * N2, H, H, qgu, H, sgu, H // 32, 1),
         ("GB/s", qbytes_row(E * N2, H, 32, 1))),
        ("mx_quant_w_down_t", lambda i: ops.mxfp8_quant(wdt, E * H, I, I, qdt, I, sdt, I // 32, 1),
         ("GB/s", qbytes_row(E * H, I, 32, 1))),
    ] + ([
        ("mx_grouped_gemm_gate_up_swiglu_quant", lambda i: ops.mxfp8_grouped_gemm_swiglu_quant(
            rows, I, H, G, offs, a_rows, T, qx, H, sx, H // 32, qgu, H, N2 * H, sgu, H // 32, N2 * (H // 32),
            qh, I, sh, I // 32, 1), ("TFLOP/s", 2.0 * rows * N2 * H)),
    ] if fused else [
        ("mx_grouped_gemm_gate_up", lambda i: ops.mxfp8_gemm(
            rows, N2, H, G, offs, a_rows, T, qx, H, sx, H // 32, qgu, H, N2 * H, sgu, H // 32, N2 * (H // 32),
            gu, N2, ops.OUT_BF16), ("TFLOP/s", 2.0 * rows * N2 * H)),
        ("silu_mul_quant_mx", lambda i: ops.fp8_silu_mul_quant(gu, rows, I, N2, 1, qh, I, sh, I // 32, 1, None, 0),
         ("GB/s", rows * N2 * 2 + rows * I + rows * (I // 32))),
    ]) + [
        ("mx_grouped_gemm_down", lambda i: ops.mxfp8_gemm(
            rows, H, I, G, offs, None, rows, qh, I, sh, I // 32, qdt, I, H * I, sdt, I // 32, H * (I // 32),
            y, H, ops.OUT_BF16), ("TFLOP/s", 2.0 * rows * H * I)),
        ("combine", lambda i: ops.fp8_moe_combine(y, rows, H, H, pos, wts, T, k, out, H, ops.OUT_BF16),
         ("GB/s", combine_bytes(rows, H, T, k))),
    ], {"workload": "moe_mxfp8_fused" if fused else "moe_mxfp8", "tokens": T, "hidden": H, "experts": E,
        "intermediate": I, "top_k": 8, "grouped_rows": rows, "seed": 3}


# ---------------------------------------------------------- CPU baseline
def _oracle_step_sample(oracle, d, rows):
    """The oracle on the first `rows` tokens of the headline step; returns
    (seconds, GEMM flops)."""
    t0 = time.perf_counter()
    qa, sa = oracle.quant_1x128(d["x_up"][:rows])
    qw, sw = oracle.quant_128x128(d["w_up"])
    mi = np.repeat(np.arange(rows), INTER)
    ni = np.tile(np.arange(INTER), rows)
    oracle.gemm_blockscaled_sampled(qa, sa, qw, sw, mi, ni)
    qa2, sa2 = oracle.quant_1x128(d["x_down"][:rows])
    qw2, sw2 = oracle.quant_128x128(d["w_down"])
    mi2 = np.repeat(np.arange(rows), HID)
    ni2 = np.tile(np.arange(HID), rows)
    oracle.gemm_blockscaled_sampled(qa2, sa2, qw2, sw2, mi2, ni2)
    return time.perf_counter() - t0, 2.0 * rows * INTER * HID * 2


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, rows, rows_1t):
    """Time the CPU oracle on a bounded sample of the headline step: the first
    `rows` tokens of both activations (1x128), both full weights (128x128) and
    both GEMMs for those tokens, on every host thread; then the first
    `rows_1t` tokens on one thread.  Reported in the metric's unit (TFLOP/s of
    GEMM work per second of oracle time)."""
    import oracle
    threads = os.cpu_count() or 1
    oracle.set_num_threads(threads)
    dt, flops = _oracle_step_sample(oracle, d, rows)
    used = oracle.num_threads()
    oracle.set_num_threads(1)
    dt1, flops1 = _oracle_step_sample(oracle, d, rows_1t)
    oracle.set_num_threads(threads)
    sample = ("first %d of 4096 tokens: 1x128 quantization of both activations, 128x128 quantization of both "
              "full weights, fp64 reference GEMMs up and down for those tokens")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": sample % rows + " (%.1f s)" % dt, "cpu_model": cpu_model(), "nproc": threads,
            "single_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": sample % rows_1t + " (%.1f s)" % dt1}}


def traffic_record():
    """HBM bytes per GEMM launch from the committed counter runs, or None if
    the GEMM sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    from fp8_block_scaled_x128_amd.profiling import gemm_sources_hash
    if rec.get("gemm_sources_sha256") != gemm_sources_hash():
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from fp8_block_scaled_x128_amd import inputs, ops

    ops.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    d = inputs.qwen3_4b_mlp(1)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    R = max(1, args.copies)
    xs_up = [to_dev(d["x_up"]) for _ in range(R)]
    xs_dn = [to_dev(d["x_down"]) for _ in range(R)]
    w_up, w_dn = to_dev(d["w_up"]), to_dev(d["w_down"])

    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    qx_up, sx_up = u8(M_TOK, HID), f32(HID // 128, M_TOK)          # M-major activation scales
    qw_up, sw_up = u8(INTER, HID), f32(INTER // 128, HID // 128)
    y_up = torch.empty((M_TOK, INTER), dtype=torch.bfloat16, device=dev)
    qx_dn, sx_dn = u8(M_TOK, INTER), f32(INTER // 128, M_TOK)
    qw_dn, sw_dn = u8(HID, INTER), f32(HID // 128, INTER // 128)
    y_dn = torch.empty((M_TOK, HID), dtype=torch.bfloat16, device=dev)

    names = ["quant_up", "gemm_up", "quant_down", "gemm_down"]
    # each launch takes (activation copy index, raw HIP stream handle); each
    # projection's activation (1x128) and weight (128x128) are quantized by
    # one fp8_quant_linear launch
    launches = [
        lambda i, st: ops.fp8_quant_linear(xs_up[i], M_TOK, HID, HID, qx_up, HID, sx_up, 1, M_TOK,
                                           w_up, INTER, HID, qw_up, HID, sw_up, stream=st),
        lambda i, st: ops.fp8_blockscaled_gemm(M_TOK, INTER, HID, qx_up, HID, sx_up, 1, M_TOK, qw_up, HID, sw_up,
                                               HID // 128, 1, ops.BSCALE_BLOCK128, y_up, INTER, ops.OUT_BF16,
                                               stream=st),
        lambda i, st: ops.fp8_quant_linear(xs_dn[i], M_TOK, INTER, INTER, qx_dn, INTER, sx_dn, 1, M_TOK,
                                           w_dn, HID, INTER, qw_dn, INTER, sw_dn, stream=st),
        lambda i, st: ops.fp8_blockscaled_gemm(M_TOK, HID, INTER, qx_dn, INTER, sx_dn, 1, M_TOK, qw_dn, INTER, sw_dn,
                                               INTER // 128, 1, ops.BSCALE_BLOCK128, y_dn, HID, ops.OUT_BF16,
                                               stream=st),
    ]
    gemm_flops = 2.0 * M_TOK * INTER * HID
    work = {"quant_up": ("GB/s", qbytes_row(M_TOK, HID) + qbytes_block2d(1, INTER, HID)),
            "gemm_up": ("TFLOP/s", gemm_flops),
            "quant_down": ("GB/s", qbytes_row(M_TOK, INTER) + qbytes_block2d(1, HID, INTER)),
            "gemm_down": ("TFLOP/s", gemm_flops)}

    # The four launches in order on one stream.  The timed loop records no
    # per-kernel events (their host cost paced the GPU: 0.36 instead of 0.29
    # ms per step); the per-kernel times come from a second pass.  Running
    # each weight quantization on a second stream next to the activation
    # quantization was measured slower (0.305 ms per step): the concurrent
    # quantizers share HBM and the cross-stream waits add latency.  So was
    # quantizing W_down on a second stream from the start of GEMM up (it does
    # not depend on it), with X_down alone on this stream: 267-272 against
    # 262-264 us per step with inputs rotated past the last-level cache.
    main_h = stream.cuda_stream

    def step(i, only=None, events=None):
        """One step; with `only` = k, events bracket launch k alone."""
        r = i % R
        for k in range(len(names)):
            if k == only:
                events[0].record(stream)
            launches[k](r, main_h)
            if k == only:
                events[1].record(stream)

    clock = ClockSampler()
    clock.start()
    # the shader clock settles over tens of milliseconds of sustained load:
    # step passes for at least --settle-ms, then the counted warm-up steps
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    clock.mark()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    clock_mhz = clock.since_mark()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # Per-kernel times in the step's schedule: one kernel per pass has events
    # around it (events around every launch paced the GPU).  They include the
    # launch gap before the kernel, 1-3 us.
    kernels = {}
    for k, n in enumerate(names):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, k, evs[i])
        torch.cuda.synchronize()
        kernels[n] = kernel_entry(*work[n], *spread([a.elapsed_time(b) for a, b in evs]))
    # The GEMMs for the roofline: events around a batch of back-to-back
    # launches of the same GEMM on the launch stream (its operands are the
    # codes the step's quantizers wrote, still in the last-level cache as in
    # the step), median over batches: the kernel's average launch duration
    # without the event overhead of a single launch.
    gemm_b2b = {}
    for k, n in enumerate(names):
        if not n.startswith("gemm"):
            continue
        per = []
        for rep in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for j in range(args.batch):
                launches[k](0, main_h)
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / args.batch)
        gemm_b2b[n] = float(np.median(per))
        kernels[n]["ms_back_to_back"] = round(gemm_b2b[n], 5)
    clock.stop()

    gemm_ms = (gemm_b2b["gemm_up"] + gemm_b2b["gemm_down"]) / 2
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    value = 2 * gemm_flops / (ms_step * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(dev)
    trec = traffic_record()
    res = {
        "metric": "block-scaled FP8 GEMM TFLOPS + quant GB/s, % of MI355X FP8/HBM peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": "qwen3_4b_mlp_forward_blockwise_fp8", "tokens": M_TOK, "hidden": HID,
                   "intermediate": INTER, "act_groups": "1x128", "weight_blocks": "128x128",
                   "scales": "fp32", "out": "bf16", "seed": 1, "input_copies": R},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": (round(trec["hbm_bytes_per_launch"]) if trec else None),
                     "kernel": "k_gemm, block-scaled FP8 GEMM (gemm_up and gemm_down of the step)",
                     "per_launch": "2*M*N*K = %.4g FLOP" % gemm_flops,
                     "timing": "HIP events around %d back-to-back launches on the launch stream, median of 5, "
                               "mean of gemm_up and gemm_down" % args.batch},
        "clock": {"sclk_mhz_timed_region": clock_mhz, "source": clock.source,
                  "settle_ms": args.settle_ms},
        "kernels": kernels,
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
    }
    if trec:
        res["roofline"]["traffic_detail"] = {k: trec[k] for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                                                  "algorithmic_min_bytes_per_launch", "source")}
    del xs_up, xs_dn

    # ------------------------------------------------- the other workloads
    wanted = [w for w in args.workloads.split(",") if w and w != "none"]
    table = {"tiny_linear": wl_tiny_linear, "mlp_backward": wl_mlp_backward,
             "mlp_backward_mxfp8": wl_mlp_backward_mxfp8, "up_proj_pow2": wl_up_proj_pow2,
             "moe_blockwise": wl_moe_blockwise, "moe_mxfp8": wl_moe_mxfp8, "up_proj_rowwise": wl_up_proj_rowwise,
             "moe_blockwise_fused": lambda *a: wl_moe_blockwise(*a, fused=True),
             "moe_mxfp8_fused": lambda *a: wl_moe_mxfp8(*a, fused=True)}
    others = {}
    for wname in wanted:
        if wname not in table:
            print("unknown workload %s" % wname, file=sys.stderr)
            sys.exit(2)
        print("timing %s" % wname, file=sys.stderr, flush=True)
        seq, cfg = table[wname](torch, ops, inputs, to_dev, R)
        ms = time_sequence(torch, stream, [fn for _, fn, _ in seq], args.reps, min(10, args.reps), args.warm_ms)
        ks = {n: kernel_entry(*wk, *t) for (n, _, wk), t in zip(seq, ms)}
        others[wname] = {"config": cfg, "ms_per_pass": round(float(sum(t[0] for t in ms)), 5), "kernels": ks}
        del seq
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if others:
        res["workloads"] = others

    # streaming-copy context: a plain 512 MiB device copy, timed like the
    # kernels; every GB/s figure also gets its fraction of this rate
    ccount = (512 << 20) // 4
    ca = torch.ones(ccount, dtype=torch.float32, device=dev)
    cb = torch.empty_like(ca)
    cms = time_sequence(torch, stream, [lambda i: cb.copy_(ca)], 20, 5, 20.0)[0]
    crate = 2.0 * ccount * 4 / (cms[0] * 1e-3) / 1e9
    res["copy_context"] = {"bytes_read": ccount * 4, "bytes_written": ccount * 4, "ms": round(cms[0], 5),
                           "GB/s": round(crate, 1), "frac_of_peak": round(crate / PEAK_HBM_GBS, 4)}
    del ca, cb
    kernel_sets = [res["kernels"]] + [w["kernels"] for w in res.get("workloads", {}).values()]
    for ks in kernel_sets:
        for e in ks.values():
            if "GB/s" in e:
                e["frac_of_copy"] = round(e["GB/s"] / crate, 4)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        res["copy_probe"] = {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_rows, args.cpu_rows_1t)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
