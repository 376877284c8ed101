"""Shared test plumbing: run the HIP GEMM through the C ABI on seeded inputs
and check the result with the CPU oracle.

The oracle is imported where a result is checked, not at module import:
bench.py draws its inputs with Problem too, and its timed path must not load
the oracle (only its CPU-baseline leg does)."""
from __future__ import annotations

import numpy as np
import torch

from warp_specialized_pipelined_amd import migemm, synth

BF16, E4M3 = synth.BF16, synth.E4M3


def codes(t: torch.Tensor) -> np.ndarray:
    """Raw element codes of a CPU or GPU tensor as a flat numpy array."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().reshape(-1)
    raise TypeError(t.dtype)


def _oracle():
    import oracle
    return oracle


def oracle_operand(t: torch.Tensor, rs: int, cs: int):
    oracle = _oracle()
    dt = oracle.BF16 if t.dtype == torch.bfloat16 else oracle.E4M3
    return oracle.Operand(dt, codes(t), rs, cs)


def padded_strides(layout, rows, cols, elem_bytes):
    """(rs, cs, storage shape) with the leading dimension rounded up to 16 bytes."""
    align = 16 // elem_bytes
    if layout == "row":
        ld = max(align, -(-cols // align) * align)
        return ld, 1, (rows, ld)
    ld = max(align, -(-rows // align) * align)
    return 1, ld, (cols, ld)


class Problem:
    """One GEMM problem: CPU storage tensors plus strides, ready for both the
    GPU path and the oracle.  Storage may be wider than the matrix (padded
    leading dimension); the padding holds random values the GEMM must ignore."""

    def __init__(self, M, N, K, A, B, C, a_rs, a_cs, b_rs, b_cs, alpha, beta, dtype=BF16,
                 d_layout="row"):
        self.M, self.N, self.K = M, N, K
        self.A, self.B, self.C = A, B, C
        self.a_rs, self.a_cs, self.b_rs, self.b_cs = a_rs, a_cs, b_rs, b_cs
        self.alpha, self.beta, self.dtype = alpha, beta, dtype
        self.d_layout = d_layout
        self.d_rs, self.d_cs, self.d_shape = padded_strides(d_layout, M, N, 2)
        self.c_rs, self.c_cs = self.d_rs, self.d_cs

    @classmethod
    def from_workload(cls, w: synth.Workload):
        x = synth.make_inputs(w)
        return cls(w.M, w.N, w.K, x["A"], x["B"], x["C"], x["a_rs"], x["a_cs"], x["b_rs"],
                   x["b_cs"], x["alpha"], x["beta"], w.dtype)

    @classmethod
    def random(cls, gen, M, N, K, la="row", lb="row", dtype=BF16, dist="uniform", alpha=1.0,
               beta=0.0, d_layout="row"):
        es = 2 if dtype == BF16 else 1
        a_rs, a_cs, a_shape = padded_strides(la, M, K, es)
        b_rs, b_cs, b_shape = padded_strides(lb, K, N, es)
        A = synth.random_matrix(gen, a_shape, dtype, dist, K)
        B = synth.random_matrix(gen, b_shape, dtype, dist, K)
        C = None
        if beta != 0.0:
            c_shape = padded_strides(d_layout, M, N, 2)[2]
            C = synth.random_matrix(gen, c_shape, BF16, "normal", K)
        return cls(M, N, K, A, B, C, a_rs, a_cs, b_rs, b_cs, alpha, beta, dtype, d_layout)

    def poison_padding(self):
        """Fill the storage past each operand row's last element (the padding
        of the leading dimension) with NaN codes: a kernel that let any of it
        reach an MFMA would give a non-finite D."""
        nan = 0x7FC0 if self.dtype == BF16 else 0x7F
        for t, rs, cs, rows, cols in ((self.A, self.a_rs, self.a_cs, self.M, self.K),
                                      (self.B, self.b_rs, self.b_cs, self.K, self.N)):
            v = t.view(torch.int16) if self.dtype == BF16 else t.view(torch.uint8)
            if cs == 1:
                v[:, cols:] = nan
            else:
                v[:, rows:] = nan
        return self

    def desc(self, flags=0, max_workgroups=0, device=0, **extra):
        t = migemm.MIGEMM_BF16 if self.dtype == BF16 else migemm.MIGEMM_FP8_E4M3
        return migemm.make_desc(self.M, self.N, self.K, t, t, self.a_rs, self.a_cs, self.b_rs,
                                self.b_cs, self.c_rs, self.c_cs, self.d_rs, self.d_cs, device=device,
                                flags=flags, max_workgroups=max_workgroups, **extra)

    # ---------------------------------------------------------------- GPU
    def to_device(self, device="cuda"):
        self.dA = self.A.to(device)
        self.dB = self.B.to(device)
        self.dC = self.C.to(device) if self.C is not None else None
        return self

    def new_d(self, fill=float("nan")):
        return torch.full(self.d_shape, fill, dtype=torch.bfloat16, device=self.dA.device)

    def run(self, plan, D=None, C_override="keep"):
        if D is None:
            D = self.new_d()
        C = self.dC if C_override == "keep" else C_override
        migemm.gemm_run(plan.handle, self.dA, self.dB, C, D, self.alpha, self.beta)
        return D

    # ------------------------------------------------------------- oracle
    def oracle_ops(self):
        Aop = oracle_operand(self.A, self.a_rs, self.a_cs)
        Bop = oracle_operand(self.B, self.b_rs, self.b_cs)
        Cop = oracle_operand(self.C, self.c_rs, self.c_cs) if self.C is not None else None
        return Aop, Bop, Cop

    def oracle_full(self, nthreads=0):
        Aop, Bop, Cop = self.oracle_ops()
        return _oracle().gemm(self.M, self.N, self.K, Aop, Bop, Cop, self.alpha, self.beta,
                              nthreads)

    def oracle_entries(self, rows, cols, nthreads=0):
        Aop, Bop, Cop = self.oracle_ops()
        return _oracle().gemm_entries(self.M, self.N, self.K, Aop, Bop, Cop, self.alpha, self.beta,
                                      rows, cols, nthreads)

    def d_values(self, D: torch.Tensor) -> np.ndarray:
        """GPU D (bf16) widened exactly to float64, as a logical M x N array."""
        v = _oracle().bf16_codes_to_f64(codes(D)).reshape(self.d_shape)
        if self.d_layout == "row":
            return v[:, :self.N]
        return v[:, :self.M].T

    def in_dtype(self):
        oracle = _oracle()
        return oracle.BF16 if self.dtype == BF16 else oracle.E4M3


def check_full(p: Problem, D: torch.Tensor, ref_absum=None):
    """Every output element against the oracle (ref_absum: a result of
    p.oracle_full() computed before, to reuse)."""
    ref, absum = ref_absum if ref_absum is not None else p.oracle_full()
    return _oracle().check(p.d_values(D), ref, absum, p.in_dtype(), p.alpha)


_WORKLOAD_REF = {}


def workload_reference(w: synth.Workload, p: Problem):
    """The oracle's full result for a named workload, computed once per test
    process (the 8192^3 one serves several tests)."""
    if w.name not in _WORKLOAD_REF:
        _WORKLOAD_REF[w.name] = p.oracle_full()
    return _WORKLOAD_REF[w.name]
