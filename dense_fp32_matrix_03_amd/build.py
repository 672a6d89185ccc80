"""Build libsgemm.so (HIP, gfx950) in-tree with hipcc.

    python -m dense_fp32_matrix_03_amd.build [--save-temps DIR] [--resource-usage] [-j N]

Every HIP source is compiled for gfx950 only, in two passes that run in
parallel across sources:

* the device pass (``--offload-device-only``) compiles the kernels into a
  bundled code object.  Packed single-precision arithmetic is disabled here
  (``-target-feature -packed-fp32-ops``), so all float arithmetic is issued
  as scalar VALU or matrix-core instructions;
* the host pass (``--offload-host-only``) compiles the host code and embeds
  that code object, the way one-pass hipcc does.

The target feature is a gfx950 feature, so giving it only to the device pass
keeps the host compiler from warning about it.  After the link, every code
object is disassembled and the build fails if any packed single-precision
add, multiply or FMA is found.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsgemm.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "mfma_kernels.hip", "mfma_layout_nn.hip", "mfma_layout_nn_unswizzled.hip",
           "mfma_layout_nt.hip", "mfma_layout_tn.hip", "mfma_layout_tt.hip",
           "mfma_layout_nn_phases.hip", "mfma_layout_nn_serial.hip", "mfma_small.hip",
           "mfma_staged.hip",
           "valu_kernels.hip", "vector_add.hip", "bf16x3.hip", "ceiling.hip", "noalloc.hip"]
ARCH = "gfx950"
BUNDLE_TARGET = f"hipv4-amdgcn-amd-amdhsa--{ARCH}"
# Packed single-precision ops that the device pass must not emit.
PACKED_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    cand = os.path.join(rocm(), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def llvm_tool(name: str) -> str:
    return os.path.join(rocm(), "lib", "llvm", "bin", name)


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def device_flags() -> list[str]:
    return ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _cuid(src: str) -> str:
    # One compilation-unit id for both passes of a source.
    return hashlib.sha256(os.path.basename(src).encode()).hexdigest()[:16]


def _run(cmd: list[str], cwd: str | None, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.stdout:
        print(r.stdout, end="", flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def _compile(src: str, save_temps: str | None, resource_usage: bool, verbose: bool) -> str:
    stem = os.path.splitext(os.path.basename(src))[0]
    fatbin = os.path.join(OBJDIR, stem + ".hipfb")
    obj = os.path.join(OBJDIR, stem + ".o")
    cuid = f"-cuid={_cuid(src)}"
    dev = [hipcc(), *common_flags(), *device_flags(), cuid, "--offload-device-only",
           "--gpu-bundle-output", "-c", src, "-o", fatbin]
    if save_temps:
        dev.append("-save-temps=obj")
    if resource_usage:
        dev.append("-Rpass-analysis=kernel-resource-usage")
    _run(dev, save_temps, verbose)
    host = [hipcc(), *common_flags(), "-fPIC", cuid, "--offload-host-only",
            "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", src, "-o", obj]
    _run(host, None, verbose)
    return obj


def check_no_packed_f32(verbose: bool = False) -> None:
    """Disassemble the device code objects of this build and fail on any
    packed single-precision add, multiply or FMA."""
    for s in SOURCES:
        stem = os.path.splitext(s)[0]
        fatbin = os.path.join(OBJDIR, stem + ".hipfb")
        co = os.path.join(OBJDIR, stem + ".co")
        subprocess.run([llvm_tool("clang-offload-bundler"), "--type=o",
                        f"--targets={BUNDLE_TARGET}", f"--input={fatbin}", f"--output={co}",
                        "--unbundle"], check=True)
        dis = subprocess.run([llvm_tool("llvm-objdump"), "-d", f"--mcpu={ARCH}", co],
                             check=True, stdout=subprocess.PIPE, text=True).stdout
        hits = PACKED_F32.findall(dis)
        if hits:
            raise RuntimeError(f"{s}: {len(hits)} packed single-precision instructions in the "
                               "gfx950 code object")
        if verbose:
            print(f"{s}: no packed single-precision instructions", flush=True)


def build(save_temps: str | None = None, resource_usage: bool = False,
          verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    if jobs is None:
        jobs = int(os.environ.get("MAX_JOBS", "0")) or min(len(SOURCES), os.cpu_count() or 1)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps, resource_usage, verbose), srcs))
    # -z defs: a symbol no object defines fails the link, not the first load.
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-Wl,-z,defs", "-o", LIB + ".tmp", *objs],
         None, verbose)
    check_no_packed_f32(verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--save-temps", metavar="DIR", help="keep intermediate files (ISA) in DIR")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/scratch usage")
    ap.add_argument("-j", "--jobs", type=int, default=None, help="parallel compile jobs")
    a = ap.parse_args(argv)
    build(save_temps=a.save_temps, resource_usage=a.resource_usage, verbose=True, jobs=a.jobs)
    print(LIB)
    return 0


if __name__ == "__main__":
    sys.exit(main())
