"""Build libzero_mi355x.so in-tree with hipcc for gfx950.

    python -m fsdp_sharded_mixed_zero_amd.build

Packed-fp32 instructions are disabled for the device code (``-packed-fp32-ops``),
no fast-math flag is used (division and square root stay correctly rounded,
denormals are kept) and floating-point contraction is off everywhere: only the
fused multiply-adds written out in the source are fused.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libzero_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["layout.cpp", "offload.cpp", "kernels.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libzero_mi355x.so)")


def host_cxx() -> str:
    """ROCm's clang++ in host mode, for the host-only sources."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for cand in (os.path.join(rocm, "lib", "llvm", "bin", "clang++"), "/opt/rocm/lib/llvm/bin/clang++",
                 shutil.which("clang++"), shutil.which("g++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def compile_flags():
    """Device sources (.hip): gfx950, packed-fp32 instructions disabled, and no
    implicit contraction of a*b+c into fused multiply-adds: only the fmaf()
    calls written in the source fuse, so device and host code (ZeRO-Offload)
    run the same operation sequence."""
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC]


def host_flags():
    """Host-only sources (.cpp): plain C++, no device pass. -fno-math-errno lets
    sqrtf and fmaf become (vector) instructions; results are unchanged."""
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "include")
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-math-errno", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
            "-I", INCLUDE, "-I", CSRC, "-I", rocm_inc]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    objs = []
    tmp_dir = os.path.join(HERE, "_build")
    os.makedirs(tmp_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp_dir, src + ".o")
        if src.endswith(".hip"):
            cmd = [cc, *compile_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [host_cxx(), *host_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp_lib = LIB_PATH + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-pthread", "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv[1:]))
