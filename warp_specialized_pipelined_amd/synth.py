"""Seeded synthetic inputs for the GEMM workloads.

This module draws random operands and nothing else: it holds none of the GEMM
arithmetic, and it is the only code that both the HIP path's callers and the
CPU oracle's callers share.  All draws use a CPU ``torch.Generator`` so that
the same seed gives the same bytes on every machine with this torch build.

Recipe (stated once, used everywhere):
  * each operand is drawn in its *storage* order (row-major A is drawn as
    [M, K], column-major A as [K, M], row-major B as [K, N], column-major B as
    [N, K]), A first, then B, then C;
  * "uniform" is 2*U[0,1) - 1, "normal" is N(0, 1), "normal_sqrtk" is
    N(0, 1) / sqrt(K); values are drawn in fp32 and rounded to bf16 with
    torch's round-to-nearest-even;
  * "e4m3" draws N(0, 1) in fp32, takes the per-tensor fp32 scale
    s = max|x| / 448, and encodes q = e4m3_rne(clamp(x / s, -448, 448)) with
    torch's float8_e4m3fn conversion.  The GEMM then runs on the codes q with
    alpha = fl32(s_A * s_B).
"""
from __future__ import annotations

import dataclasses
import math

import torch

BF16 = 1
E4M3 = 2
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: int = BF16           # operand type of A and B; C and D are bf16
    a_layout: str = "row"       # "row": [M, K] storage; "col": [K, M]
    b_layout: str = "row"       # "row": [K, N] storage; "col": [N, K]
    dist: str = "uniform"       # uniform | normal | normal_sqrtk | e4m3
    alpha: float = 1.0
    beta: float = 0.0
    has_c: bool = False
    consumer: bool = False      # hand finished 256x256 tiles to the consumer stage
    seed: int = 0

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


# The five workloads the library is measured and checked on.
WORKLOADS = [
    Workload("bf16_256_rowrow", 256, 256, 256, BF16, "row", "row", "uniform", 1.0, 0.0, False,
             False, 1000),
    Workload("bf16_4096_rowcol_beta", 4096, 4096, 4096, BF16, "row", "col", "normal", 1.0, 0.5,
             True, False, 1001),
    Workload("bf16_ragged_4000x3000x5000", 4000, 3000, 5000, BF16, "row", "row", "uniform", 1.0,
             0.0, False, False, 1002),
    Workload("bf16_8192_tile_consumer", 8192, 8192, 8192, BF16, "row", "row", "normal_sqrtk",
             1.0, 0.0, False, True, 1003),
    Workload("fp8_e4m3_8192x8192x16384", 8192, 8192, 16384, E4M3, "row", "row", "e4m3", 1.0, 0.0,
             False, False, 1004),
]


def strides(layout: str, rows: int, cols: int):
    """(row stride, column stride) in elements of a rows x cols matrix."""
    if layout == "row":
        return cols, 1
    if layout == "col":
        return 1, rows
    raise ValueError(layout)


def storage_shape(layout: str, rows: int, cols: int):
    return (rows, cols) if layout == "row" else (cols, rows)


def _draw_bf16(gen, shape, dist, K):
    if dist == "uniform":
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
    elif dist == "normal_sqrtk":
        x = torch.randn(shape, generator=gen, dtype=torch.float32) / math.sqrt(K)
    else:
        raise ValueError(dist)
    return x.to(torch.bfloat16)


def _draw_e4m3(gen, shape):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if x.numel() == 0:   # an empty operand (K = 0): nothing to scale
        return x.to(torch.float8_e4m3fn), 1.0
    scale = (x.abs().max() / E4M3_MAX).to(torch.float32)
    q = (x / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, float(scale)


def make_inputs(w: Workload):
    """Draw the operands of workload ``w`` on the CPU.

    Returns a dict with the storage tensors ``A``, ``B`` (bf16, or
    float8_e4m3fn for e4m3), ``C`` (bf16 or None), their strides in elements,
    and the ``alpha``/``beta`` to pass (alpha includes the fp8 scales)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    a_shape = storage_shape(w.a_layout, w.M, w.K)
    b_shape = storage_shape(w.b_layout, w.K, w.N)
    alpha = float(w.alpha)
    if w.dist == "e4m3":
        A, sa = _draw_e4m3(gen, a_shape)
        B, sb = _draw_e4m3(gen, b_shape)
        alpha = float(torch.tensor(sa, dtype=torch.float32) * torch.tensor(sb, dtype=torch.float32)
                      * torch.tensor(w.alpha, dtype=torch.float32))
        scales = (sa, sb)
    else:
        A = _draw_bf16(gen, a_shape, w.dist, w.K)
        B = _draw_bf16(gen, b_shape, w.dist, w.K)
        scales = None
    C = None
    if w.has_c:
        C = _draw_bf16(gen, (w.M, w.N), w.dist if w.dist != "e4m3" else "normal", w.K)
    a_rs, a_cs = strides(w.a_layout, w.M, w.K)
    b_rs, b_cs = strides(w.b_layout, w.K, w.N)
    return {
        "A": A, "B": B, "C": C,
        "a_rs": a_rs, "a_cs": a_cs, "b_rs": b_rs, "b_cs": b_cs,
        "c_rs": w.N, "c_cs": 1, "d_rs": w.N, "d_cs": 1,
        "alpha": alpha, "beta": float(w.beta), "scales": scales,
    }


def random_matrix(gen, shape, dtype=BF16, dist="uniform", K=1):
    """A single seeded operand (for shape sweeps)."""
    if dtype == E4M3:
        return _draw_e4m3(gen, shape)[0]
    return _draw_bf16(gen, shape, dist, K)


def small_int_matrix(gen, shape, lo=-1, hi=1, dtype=BF16):
    """Integers drawn uniformly from [lo, hi], exactly representable."""
    x = torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32).to(torch.float32)
    return x.to(torch.bfloat16 if dtype == BF16 else torch.float8_e4m3fn)
