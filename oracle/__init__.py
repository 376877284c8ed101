"""CPU oracle for the persistent pipelined GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and it shares
nothing with this code: the arithmetic lives in ``oracle.c`` (plain C, fp64),
compiled with gcc into ``liboracle.so``; this module only marshals numpy
arrays into it and holds the acceptance rule.

Functions
---------
build()                  compile oracle.c with gcc (OpenMP, no FP contraction)
gemm(...)                full fp64 reference and |a*b| sums, all M x N entries
gemm_entries(...)        the same definition at chosen (i, j) entries only
tile_rowstats(...)       consumer-stage recompute from a bf16 D
bf16_value / e4m3_value  exact decoders for one code
check(...)               per-element acceptance test

Acceptance rule (stated with each GEMM config): for bf16 operands
``|D - ref| <= 2^-8 |ref| + 1e-4 |alpha| sum_k |a b|``; for e4m3 operands
``|D - ref| <= 2^-7 |ref| + 2e-3 |alpha| sum_k |a b|``, with a and b the
encoded operand values (per-tensor scales are folded into alpha).  D must be
finite.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at deliberately broken builds of oracle.c to
# check that the pins catch them.
_LIB_OVERRIDE = os.environ.get("MIGEMM_ORACLE_LIB")

BF16 = 1
E4M3 = 2

# Tolerances: (relative coefficient, coefficient of |alpha| * sum |a*b|).
TOLERANCE = {BF16: (2.0 ** -8, 1e-4), E4M3: (2.0 ** -7, 2e-3)}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c -> liboracle.so with gcc.  Returns the library path."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = dbl
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = dbl
    mat = [i32, vp, i64, i64]
    lib.orc_gemm.argtypes = [i64, i64, i64] + mat * 3 + [dbl, dbl, vp, vp, i32]
    lib.orc_gemm.restype = i32
    lib.orc_gemm_entries.argtypes = ([i64, i64, i64] + mat * 3 + [dbl, dbl, vp, vp, i64, vp, vp, i32])
    lib.orc_gemm_entries.restype = i32
    lib.orc_tile_rowstats.argtypes = [i64, i64, vp, i64, i64, i64, vp, vp]
    lib.orc_tile_rowstats.restype = i32
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def bf16_value(code: int) -> float:
    return float(_load().orc_bf16_value(int(code) & 0xFFFF))


def e4m3_value(code: int) -> float:
    return float(_load().orc_e4m3_value(int(code) & 0xFF))


class Operand:
    """A matrix operand as the oracle sees it: raw element codes plus strides.

    ``codes`` is a numpy array of uint16 (bf16) or uint8 (e4m3) holding the
    storage; element (r, c) is ``codes.flat[r*rs + c*cs]``.
    """

    def __init__(self, dtype: int, codes: np.ndarray, rs: int, cs: int):
        want = np.uint16 if dtype == BF16 else np.uint8
        if dtype not in (BF16, E4M3):
            raise ValueError("dtype must be BF16 or E4M3")
        codes = np.ascontiguousarray(codes).reshape(-1)
        if codes.dtype != want:
            codes = codes.view(want)
        self.dtype, self.codes, self.rs, self.cs = dtype, codes, int(rs), int(cs)

    def ptr(self):
        return self.codes.ctypes.data


def _c_args(C):
    if C is None:
        return [BF16, None, 0, 0]
    return [C.dtype, C.ptr(), C.rs, C.cs]


def gemm(M, N, K, A: Operand, B: Operand, C: Operand | None, alpha: float, beta: float,
         nthreads: int = 0):
    """All entries: returns (ref, absum) as float64 [M, N] arrays."""
    lib = _load()
    ref = np.zeros((M, N), dtype=np.float64)
    absum = np.zeros((M, N), dtype=np.float64)
    rc = lib.orc_gemm(M, N, K, A.dtype, A.ptr(), A.rs, A.cs, B.dtype, B.ptr(), B.rs, B.cs,
                      *_c_args(C), float(alpha), float(beta),
                      ref.ctypes.data, absum.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("orc_gemm rejected its arguments")
    return ref, absum


def gemm_entries(M, N, K, A: Operand, B: Operand, C: Operand | None, alpha: float, beta: float,
                 rows, cols, nthreads: int = 0):
    """Chosen entries: returns (ref, absum) as float64 arrays of len(rows)."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in shape")
    n = rows.size
    ref = np.zeros(n, dtype=np.float64)
    absum = np.zeros(n, dtype=np.float64)
    rc = lib.orc_gemm_entries(M, N, K, A.dtype, A.ptr(), A.rs, A.cs, B.dtype, B.ptr(), B.rs, B.cs,
                              *_c_args(C), float(alpha), float(beta), rows.ctypes.data,
                              cols.ctypes.data, n, ref.ctypes.data, absum.ctypes.data,
                              int(nthreads))
    if rc != 0:
        raise ValueError("orc_gemm_entries rejected its arguments")
    return ref, absum


def tile_rowstats(D_codes: np.ndarray, M: int, N: int, d_rs: int, d_cs: int, tile_n: int = 256):
    """Row sums and row maxima per tile_n-wide slice of a bf16 D, as
    orc_tile_rowstats defines them: the sequential fp32 sum in ascending
    column order from +0.0, and the IEEE maximumNumber (NaN ignored, -0 < +0,
    -inf when the slice holds no number).
    Returns (row_sum, row_max), float32 [M, ceil(N/tile_n)]."""
    lib = _load()
    D_codes = np.ascontiguousarray(D_codes).reshape(-1).view(np.uint16)
    ld = (N + tile_n - 1) // tile_n
    rs = np.zeros((M, ld), dtype=np.float32)
    rm = np.zeros((M, ld), dtype=np.float32)
    rc = lib.orc_tile_rowstats(M, N, D_codes.ctypes.data, d_rs, d_cs, tile_n, rs.ctypes.data,
                               rm.ctypes.data)
    if rc != 0:
        raise ValueError("orc_tile_rowstats rejected its arguments")
    return rs, rm


def bf16_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 codes (uint16) to float64: the code is the top
    half of a binary32."""
    c = np.asarray(codes).view(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):   # signalling-NaN codes widen to NaN
        return c.view(np.float32).astype(np.float64)


def check(D_values, ref, absum, in_dtype: int, alpha: float):
    """Acceptance test for each element.  ``D_values`` are the GPU results
    widened to float64 (same shape as ref).  Returns a dict with the failure
    count, the count of non-finite D, and the worst |D-ref|/bound and its flat
    index."""
    rel, coef = TOLERANCE[in_dtype]
    D = np.asarray(D_values, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    absum = np.asarray(absum, dtype=np.float64)
    bound = rel * np.abs(ref) + coef * abs(float(alpha)) * absum
    err = np.abs(D - ref)
    finite = np.isfinite(D)
    bad = ~finite | (err > bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    ratio = np.where(finite, ratio, np.inf)
    worst = int(np.argmax(ratio)) if ratio.size else -1
    return {
        "n": int(D.size),
        "n_fail": int(bad.sum()),
        "n_nonfinite": int((~finite).sum()),
        "worst_ratio": float(ratio.flat[worst]) if ratio.size else 0.0,
        "worst_index": worst,
    }
