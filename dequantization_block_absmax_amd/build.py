"""Builds libbq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python dequantization_block_absmax_amd/build.py

Every translation unit is compiled with -ffp-contract=off (no multiply-add contraction: the
outputs are defined with separately rounded binary32 operations) and without fast-math.
Packed fp32 instructions are disabled (-packed-fp32-ops) for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = ["bq_api.cpp", "bq_table.cpp", "k_quant.hip", "k_dequant.hip", "k_nested.hip", "k_q32.hip",
           "k_linear.hip", "k_gemm.hip", "k_scratch.hip", "k_iq2xs.hip",
           "k_iq1s.hip"]


def _cmd(src: str, obj: str) -> list[str]:
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        return [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj]
    return [HIPCC, *COMMON, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c", path,
            "-o", obj]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmd = _cmd(src, obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("compilation failed: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
