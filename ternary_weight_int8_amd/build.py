"""Build libternary_gemm.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ternary_gemm.hip")
SRCS = [SRC, os.path.join(PKG, "csrc", "prep.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libternary_gemm.so")
# measurement probes for bench.py (a store floor and MFMA-only loops), not
# part of the GEMM library
PROBE_SRC = os.path.join(PKG, "csrc", "roofline.hip")
PROBE_LIB = os.path.join(PKG, "libtgemm_roofline.so")
ARCH = "gfx950"


def hipcc_cmd(out: str, srcs=None) -> list[str]:
    return [
        "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *(srcs or SRCS), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the HIP library and the probe library (always) and atomically
    replace the old ones."""
    for lib, srcs in ((LIB, SRCS), (PROBE_LIB, [PROBE_SRC])):
        tmp = lib + ".tmp"
        r = subprocess.run(hipcc_cmd(tmp, srcs), capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
        if verbose:
            print(r.stderr)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
