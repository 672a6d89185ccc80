"""Build libsgemm.so (HIP, gfx950) in-tree with hipcc.

    python -m dense_fp32_matrix_03_amd.build [--save-temps DIR] [--resource-usage]

Every HIP source is compiled for gfx950 only.  Packed single-precision FMA is
disabled (-packed-fp32-ops): all float arithmetic is issued as scalar VALU or
matrix-core instructions.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsgemm.so")
SOURCES = ["api.hip", "mfma_kernels.hip", "valu_kernels.hip", "vector_add.hip", "bf16x3.hip",
           "ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def build(save_temps: str | None = None, resource_usage: bool = False,
          verbose: bool = False) -> str:
    cmd = [hipcc(), *flags(), "-shared", "-o", LIB + ".tmp"]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += [f"-save-temps={'obj'}"]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = save_temps if save_temps else None
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--save-temps", metavar="DIR", help="keep intermediate files (ISA) in DIR")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/scratch usage")
    a = ap.parse_args(argv)
    build(save_temps=a.save_temps, resource_usage=a.resource_usage, verbose=True)
    print(LIB)
    return 0


if __name__ == "__main__":
    sys.exit(main())
