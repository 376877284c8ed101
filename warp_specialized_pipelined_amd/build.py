"""Build libmigemm.so in-tree with hipcc for gfx950.

    python -m warp_specialized_pipelined_amd.build                # build
    python -m warp_specialized_pipelined_amd.build --asm DIR      # also write the AMD assembly to DIR

The library is written next to this file so that it travels with the source
tree; nothing is installed.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmigemm.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "gemm_kernels.hip")]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 arithmetic instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libmigemm.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


def build_c_client(verbose: bool = False) -> str:
    """Compile tests/c_client.c, a plain C program that uses the C ABI with
    its own device memory (no Python), against the in-tree library, into
    tests/_build/c_client.  Needs build() first."""
    root = os.path.dirname(HERE)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    out_dir = os.path.join(root, "tests", "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "c_client")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(root, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(root, "tests", "c_client.c"), "-o", exe + ".tmp",
           "-L", HERE, "-lmigemm", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../warp_specialized_pipelined_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(exe + ".tmp", exe)
    return exe


def dump_asm(out_dir: str) -> str:
    """Write the gfx950 assembly of the kernel translation unit to out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "gemm_kernels.s")
    cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", "-o", out,
           os.path.join(CSRC, "gemm_kernels.hip")]
    subprocess.run(cmd, check=True, cwd=CSRC)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if "--asm" in sys.argv:
        i = sys.argv.index("--asm")
        if i + 1 >= len(sys.argv):
            sys.exit("--asm needs an output directory")
        print(dump_asm(sys.argv[i + 1]))
