"""Build libfp8bs.so (HIP, gfx950 only) in-tree with hipcc.

    python -m fp8_block_scaled_x128_amd.build [--resource-usage]

Every source is compiled for gfx950 with -ffp-contract=off (the kernels place
their FMAs explicitly) and with packed-FP32 code generation disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp8bs.so")
SOURCES = ["quant.hip", "gemm.hip", "moe.hip", "capi.hip"]
# The GEMM promotes MFMA results with VALU FMAs, so the results must land in
# VGPRs (not AGPRs, which would need a v_accvgpr_read per value).
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str, extra):
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return out


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every HIP source and link libfp8bs.so; returns its path."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        outs = list(ex.map(lambda so: _compile(os.path.join(CSRC, so[0]), so[1], extra + EXTRA.get(so[0], [])),
                           zip(SOURCES, objs)))
    if verbose or resource_usage:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv))
