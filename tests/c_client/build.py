"""Build the plain-C client of libsgemm.so (sgemm_client.c) with gcc.

    python tests/c_client/build.py

Strict C99 with every warning an error, so this also checks that the public
headers under include/ are valid C.  The HIP runtime's C API comes from
/opt/rocm (included as a system header).  The binary finds libsgemm.so
in-tree through its run path.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sgemm_client.c")
BIN = os.path.join(HERE, "sgemm_client")
PKG = os.path.join(ROOT, "dense_fp32_matrix_03_amd")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(rocm, "include"),
           "-I" + os.path.join(ROOT, "include"), SRC, "-o", BIN + ".tmp",
           "-L" + PKG, "-lsgemm", "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../dense_fp32_matrix_03_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
