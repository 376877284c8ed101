"""Build libmigemm.so in-tree with hipcc for gfx950.

    python -m warp_specialized_pipelined_amd.build                # build
    python -m warp_specialized_pipelined_amd.build --asm DIR      # also write the AMD assembly to DIR

The library is written next to this file so that it travels with the source
tree (objects and the host-sanitizer variant under _build/); nothing is
installed.
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


OBJ_DIR = os.path.join(HERE, "_build")
# The host-side sanitizer build of the C ABI layer (api.cpp): the address
# and undefined-behaviour sanitizers, any report fatal.  Each -fsanitize=
# flag follows -Xarch_host, so no device code is instrumented.
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)


def _obj(name):
    os.makedirs(OBJ_DIR, exist_ok=True)
    return os.path.join(OBJ_DIR, name)


def build(verbose: bool = False, asan: bool = True) -> str:
    """Compile every HIP source into libmigemm.so (always recompiles): the
    kernel translation unit once into an object, the C ABI layer, and the
    link.  With asan, also _build/libmigemm_asan.so: the same kernel object
    with the C ABI layer built under the host AddressSanitizer."""
    kobj, aobj = _obj("gemm_kernels.o"), _obj("api.o")
    _run([hipcc(), *HIPCC_FLAGS, "-c", "-o", kobj, os.path.join(CSRC, "gemm_kernels.hip")], verbose)
    _run([hipcc(), *HIPCC_FLAGS, "-c", "-o", aobj, os.path.join(CSRC, "api.cpp")], verbose)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc(), *HIPCC_FLAGS, "-shared", "-o", tmp, aobj, kobj], verbose)
    os.replace(tmp, LIB)
    if asan:
        sobj, slib = _obj("api_asan.o"), _obj("libmigemm_asan.so")
        _run([hipcc(), *HIPCC_FLAGS, *ASAN_HOST_FLAGS, "-c", "-o", sobj,
              os.path.join(CSRC, "api.cpp")], verbose)
        _run([hipcc(), *HIPCC_FLAGS, *ASAN_HOST_FLAGS, "-shared", "-o", slib + ".tmp", sobj, kobj],
             verbose)
        os.replace(slib + ".tmp", slib)
    return LIB


def build_c_client(verbose: bool = False) -> list:
    """Compile the C programs of the tests into tests/_build: c_client (the
    C ABI used from plain C with its own device memory, no Python) against
    the in-tree library; and, when build() made _build/libmigemm_asan.so,
    c_client_asan and c_validate_extremes against it, under the host
    address and undefined-behaviour sanitizers.  Needs build() first."""
    root = os.path.dirname(HERE)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    out_dir = os.path.join(root, "tests", "_build")
    os.makedirs(out_dir, exist_ok=True)
    common = ["-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(root, "include"), "-I", os.path.join(rocm, "include")]
    hip = ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    built = []
    variants = [("c_client", "gcc", [], HERE, "migemm",
                 "$ORIGIN/../../warp_specialized_pipelined_amd")]
    if os.path.exists(os.path.join(OBJ_DIR, "libmigemm_asan.so")):
        # The sanitized library comes from hipcc's clang, so these programs
        # are built by ROCm's clang too: one sanitizer runtime, clang's.
        clang = os.path.join(rocm, "llvm", "bin", "clang")
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer"]
        rp = "$ORIGIN/../../warp_specialized_pipelined_amd/_build"
        variants.append(("c_client_asan", clang, san, OBJ_DIR, "migemm_asan", rp))
        variants.append(("c_validate_extremes", clang, san, OBJ_DIR, "migemm_asan", rp,
                         os.path.join(root, "tests", "c_validate_extremes.c")))
    for v in variants:
        name, cc, extra, libdir, lib, rpath = v[:6]
        src = v[6] if len(v) > 6 else os.path.join(root, "tests", "c_client.c")
        exe = os.path.join(out_dir, name)
        cmd = [cc, *extra, *common, src, "-o", exe + ".tmp", "-L", libdir, "-l" + lib,
               "-Wl,-rpath," + rpath, *hip]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(exe + ".tmp", exe)
        built.append(exe)
    return built


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
