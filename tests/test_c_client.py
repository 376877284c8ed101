"""The C ABI from plain C (GPU): tests/c_client.c, built by the package's
build step, allocates its own device memory with HIP, includes
include/migemm.h and links libmigemm.so -- no Python or PyTorch in the
process.  It runs a ragged bf16 GEMM with beta through gemm_run and a
stream-K plan through gemm_run_no_alloc, compares every output bit for bit
with the closed-form result of its small-integer inputs, and checks that a
destroyed plan is refused with D untouched."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "c_client")


def test_c_client_runs_the_abi_from_c():
    if not os.path.exists(EXE):
        # A one-second gcc compile of a test program (not of the library,
        # which the other tests need built already).
        from warp_specialized_pipelined_amd import build
        build.build_c_client()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "c_client: OK", (r.returncode, r.stdout,
                                                                     r.stderr)
