"""Builds libmoe.so (the HIP kernels and the C ABI of include/moe.h) for gfx950.

Each source compiles to an object in _build/ in parallel, then one shared library is
linked next to this file. Flags: -ffp-contract=off, correctly rounded fp32 division
and no denormal flush keep the quantisers' fp32 steps single IEEE operations; packed
fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["quant.hip", "route.hip", "permute.hip", "gemm.hip", "gemm_tile.hip", "gemm_stream.hip", "gemm_mx.hip",
           "gemm_fp8_wide.hip", "gemm_bf16_wide.hip", "combine.hip", "moe_api.hip"]
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops' is not a recognized" not in l)
        if p.returncode != 0:
            failed.append(f"{src}:\n{out}")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("HIP build failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
