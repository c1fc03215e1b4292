"""Benchmark of the block-wise FP8 linear layer on one MI355X.

One step is the Qwen3-4B MLP forward with the block-wise FP8 recipe, every
part on the GPU through the C ABI:
    quantize X_up [4096 x 2560] per token (1x128), quantize W_up [9728 x 2560]
    in 128x128 blocks, GEMM up (bf16 out), quantize X_down [4096 x 9728],
    quantize W_down [2560 x 9728], GEMM down (bf16 out).
Inputs are seeded synthetic tensors (see fp8_block_scaled_x128_amd.inputs),
resident in HBM before timing; the step rotates over several copies so that
the 256 MB last-level cache cannot serve them.

Prints ONE JSON line: value = GEMM FLOPs of the step / step time (TFLOP/s),
with per-kernel times, TFLOP/s or GB/s against MI355X's peaks, a roofline
object for the dominant kernel (the block-scaled GEMM) and a CPU-oracle
baseline on a bounded sample.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=288, help="token rows in the CPU-oracle sample")
    return ap.parse_args()


def quant_bytes_1x128(rows, cols):
    return rows * cols * 3 + rows * ((cols + 127) // 128) * 4


def quant_bytes_128x128(rows, cols):
    return rows * cols * 3 + ((rows + 127) // 128) * ((cols + 127) // 128) * 4


def cpu_baseline(d, rows):
    """Time the CPU oracle on a bounded sample of the same step: the first
    `rows` tokens of both activations (1x128), both full weights (128x128) and
    both GEMMs for those tokens.  Reported in the metric's unit (TFLOP/s of
    GEMM work per second of oracle time)."""
    import oracle
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
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * INTER * HID * 2
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "first %d of 4096 tokens: 1x128 quantization of both activations, 128x128 quantization "
                      "of both full weights, fp64 reference GEMMs up and down for those tokens (%.1f s)"
                      % (rows, dt)}


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
    d = inputs.qwen3_4b_mlp(1)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    R = max(1, args.copies)
    xs_up = [to_dev(d["x_up"]) for _ in range(R)]
    ws_up = [to_dev(d["w_up"]) for _ in range(R)]
    xs_dn = [to_dev(d["x_down"]) for _ in range(R)]
    ws_dn = [to_dev(d["w_down"]) for _ in range(R)]

    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    qx_up, sx_up = u8(M_TOK, HID), f32(HID // 128, M_TOK)          # M-major activation scales
    qw_up, sw_up = u8(INTER, HID), f32(INTER // 128, HID // 128)
    y_up = torch.empty((M_TOK, INTER), dtype=torch.bfloat16, device=dev)
    qx_dn, sx_dn = u8(M_TOK, INTER), f32(INTER // 128, M_TOK)
    qw_dn, sw_dn = u8(HID, INTER), f32(HID // 128, INTER // 128)
    y_dn = torch.empty((M_TOK, HID), dtype=torch.bfloat16, device=dev)

    names = ["quant_x_up", "quant_w_up", "gemm_up", "quant_x_down", "quant_w_down", "gemm_down"]
    launches = [
        lambda i: ops.fp8_quant_rowblock(xs_up[i], M_TOK, HID, HID, ops.AXIS_ROW, qx_up, HID, sx_up, 1, M_TOK),
        lambda i: ops.fp8_quant_block2d(ws_up[i], 1, INTER, HID, HID, qw_up, HID, None, 0, sw_up),
        lambda i: ops.fp8_blockscaled_gemm(M_TOK, INTER, HID, qx_up, HID, sx_up, 1, M_TOK, qw_up, HID, sw_up,
                                           HID // 128, 1, ops.BSCALE_BLOCK128, y_up, INTER, ops.OUT_BF16),
        lambda i: ops.fp8_quant_rowblock(xs_dn[i], M_TOK, INTER, INTER, ops.AXIS_ROW, qx_dn, INTER, sx_dn, 1, M_TOK),
        lambda i: ops.fp8_quant_block2d(ws_dn[i], 1, HID, INTER, INTER, qw_dn, INTER, None, 0, sw_dn),
        lambda i: ops.fp8_blockscaled_gemm(M_TOK, HID, INTER, qx_dn, INTER, sx_dn, 1, M_TOK, qw_dn, INTER, sw_dn,
                                           INTER // 128, 1, ops.BSCALE_BLOCK128, y_dn, HID, ops.OUT_BF16),
    ]
    gemm_flops = 2.0 * M_TOK * INTER * HID
    work = {"quant_x_up": ("GB/s", quant_bytes_1x128(M_TOK, HID)),
            "quant_w_up": ("GB/s", quant_bytes_128x128(INTER, HID)),
            "gemm_up": ("TFLOP/s", gemm_flops),
            "quant_x_down": ("GB/s", quant_bytes_1x128(M_TOK, INTER)),
            "quant_w_down": ("GB/s", quant_bytes_128x128(HID, INTER)),
            "gemm_down": ("TFLOP/s", gemm_flops)}

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]

    def step(i, events=None):
        for k, fn in enumerate(launches):
            if events is not None:
                events[k].record(stream)
            fn(i % R)
        if events is not None:
            events[len(names)].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i, ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    kernels = {}
    for k, n in enumerate(names):
        ms = float(np.mean([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)]))
        unit, amount = work[n]
        if unit == "TFLOP/s":
            rate = amount / (ms * 1e-3) / 1e12
            frac = rate / PEAK_FP8_TFLOPS
        else:
            rate = amount / (ms * 1e-3) / 1e9
            frac = rate / PEAK_HBM_GBS
        kernels[n] = {"ms": round(ms, 5), unit: round(rate, 2), "frac_of_peak": round(frac, 4)}

    gemm_ms = (kernels["gemm_up"]["ms"] + kernels["gemm_down"]["ms"]) / 2
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    value = 2 * gemm_flops / (ms_step * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(dev)
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
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel": "fp8bs k_gemm (block-scaled FP8 GEMM)",
                     "per_launch": "2*M*N*K = %.4g FLOP" % gemm_flops},
        "kernels": kernels,
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
