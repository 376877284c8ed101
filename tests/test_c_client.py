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


ASAN_EXE = os.path.join(os.path.dirname(EXE), "c_client_asan")


def test_c_client_under_host_address_sanitizer():
    # The same program against libmigemm_asan.so: the C ABI layer (plan
    # checks, the set of live plans, plan create/destroy, the runs) built
    # with the host AddressSanitizer -- no device code is instrumented.  Any
    # out-of-bounds or freed-memory access on the host aborts the run with a
    # report.  (Leak checking is off: the HIP runtime keeps allocations
    # until the process ends.)
    if not os.path.exists(ASAN_EXE):
        from warp_specialized_pipelined_amd import build
        build.build_c_client()
    assert os.path.exists(ASAN_EXE), "the sanitized library was not built (build(asan=True))"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([ASAN_EXE], capture_output=True, text=True, timeout=300, env=env)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and r.stdout.strip() == "c_client: OK", (r.returncode, r.stdout,
                                                                     r.stderr[-2000:])
