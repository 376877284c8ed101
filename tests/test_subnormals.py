"""Subnormal numbers (GPU): kept, not flushed.

The kernels run with fp32 subnormals preserved (the code object's float
mode), and the MFMAs keep subnormal inputs and products.  Each case puts
exactly one nonzero product (or two) in an output, so the exact result is a
closed form; D must equal it rounded to bf16 (nearest even), bit for bit:
subnormal bf16 inputs times normal ones, normal inputs whose product is
subnormal, the smallest subnormal, two subnormal products that sum to the
smallest normal, and a product below half the smallest bf16 subnormal
(which rounds to zero).  e4m3's subnormal codes (exponent field 0) are
covered the same way.

The acceptance bound used elsewhere is relative; in bf16's subnormal range
(below 2^-126) the spacing of bf16 values is absolute (2^-133), so a
correctly rounded result there can miss that bound.  No workload reaches
that range; these cases compare with the correctly rounded value instead."""
from fractions import Fraction

import pytest
import torch

from warp_specialized_pipelined_amd import migemm

pytestmark = pytest.mark.gpu


def bf16_code_value(code: int) -> Fraction:
    """Exact value of a finite bf16 code (sign, 8-bit exponent bias 127, 7-bit mantissa)."""
    s = -1 if code & 0x8000 else 1
    e = (code >> 7) & 0xFF
    m = code & 0x7F
    if e == 0:
        return s * Fraction(m, 128) * Fraction(1, 2 ** 126)
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def e4m3_code_value(code: int) -> Fraction:
    """Exact value of a finite OCP e4m3 code (exponent bias 7, 3-bit mantissa)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


_BF16_POSITIVE = None


def bf16_rne_code(x: Fraction) -> int:
    """The bf16 code nearest to x, ties to the even code, found among the
    exact values of all finite codes (which increase with the code), so no
    floating point is involved.  A negative x that rounds to zero gives -0."""
    import bisect
    global _BF16_POSITIVE
    if _BF16_POSITIVE is None:
        _BF16_POSITIVE = [bf16_code_value(c) for c in range(0x7F80)]
    a = abs(x)
    i = bisect.bisect_left(_BF16_POSITIVE, a)
    if i == len(_BF16_POSITIVE):
        raise ValueError("beyond the largest finite bf16")
    if _BF16_POSITIVE[i] == a or i == 0:
        c = i
    else:
        lo, hi = _BF16_POSITIVE[i - 1], _BF16_POSITIVE[i]
        c = i - 1 if a - lo < hi - a else i if a - lo > hi - a else (i - 1 if (i - 1) % 2 == 0 else i)
    return c | (0x8000 if x < 0 else 0)


def run(dtype, A_codes, B_codes, la, lb, flags=0):
    """D = A B with the given element codes, A and B in the given layouts."""
    M, K = A_codes.shape
    N = B_codes.shape[1]
    if dtype == "bf16":
        A = torch.where(A_codes >= 0x8000, A_codes - 0x10000, A_codes).to(torch.int16).view(torch.bfloat16)
        B = torch.where(B_codes >= 0x8000, B_codes - 0x10000, B_codes).to(torch.int16).view(torch.bfloat16)
        t = migemm.MIGEMM_BF16
    else:
        A = A_codes.to(torch.uint8).view(torch.float8_e4m3fn)
        B = B_codes.to(torch.uint8).view(torch.float8_e4m3fn)
        t = migemm.MIGEMM_FP8_E4M3
    if la == "col":
        A = A.t().contiguous()                  # storage K x M
        a_rs, a_cs = 1, M
    else:
        a_rs, a_cs = K, 1
    if lb == "col":
        B = B.t().contiguous()                  # storage N x K
        b_rs, b_cs = 1, K
    else:
        b_rs, b_cs = N, 1
    desc = migemm.make_desc(M, N, K, t, t, a_rs, a_cs, b_rs, b_cs, N, 1, N, 1, flags=flags)
    plan = migemm.Plan(desc)
    dA, dB = A.cuda(), B.cuda()
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    migemm.gemm_run(plan, dA, dB, None, D, 1.0, 0.0)
    torch.cuda.synchronize()
    return D.view(torch.int16).cpu().to(torch.int32) & 0xFFFF


# (row, list of (k, a code, b code)) -- output (row, row) holds the sum of these products
BF16_CASES = [
    (0, [(0, 0x0008, 0x4480)]),                 # 2^-130 (subnormal) x 2^10 = 2^-120
    (1, [(1, 0x1F00, 0x1F00)]),                 # 2^-65 x 2^-65 = 2^-130 (subnormal product)
    (2, [(2, 0x0001, 0x7F00)]),                 # 2^-133 (smallest subnormal) x 2^127
    (3, [(3, 0x0080, 0x3F00)]),                 # 2^-126 x 0.5 = 2^-127
    (4, [(4, 0x0040, 0x3F80), (5, 0x0040, 0x3F80)]),   # 2^-127 + 2^-127 = 2^-126
    (5, [(6, 0x1E00, 0x1E80)]),                 # 2^-67 x 2^-66 = 2^-133: the smallest subnormal
    (6, [(7, 0x1E00, 0x1E00)]),                 # 2^-67 x 2^-67 = 2^-134: half of it, ties to even: 0
    (7, [(8, 0x1E00, 0x1EC0)]),                 # 2^-67 x 1.5 x 2^-66 = 1.5 x 2^-133 -> 2 x 2^-133
    (8, [(9, 0x8003, 0x4000)]),                 # -3 x 2^-133 x 2 = -6 x 2^-133
    (9, [(10, 0x1F40, 0x9F40)]),                # 1.5 x 2^-65 x -1.5 x 2^-65 = -2.25 x 2^-130
]

E4M3_CASES = [
    (0, [(0, 0x01, 0x7E)]),                     # 2^-9 x 448
    (1, [(1, 0x07, 0x01)]),                     # 7 x 2^-9 x 2^-9
    (2, [(2, 0x04, 0x38)]),                     # 2^-7 x 1
    (3, [(3, 0x86, 0x7E)]),                     # -6 x 2^-9 x 448
    (4, [(4, 0x01, 0x01)]),                     # 2^-18
]


@pytest.mark.parametrize("tile", [migemm.MIGEMM_F_TILE_M256, migemm.MIGEMM_F_TILE_M192],
                         ids=["m256", "m192"])
@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "col"), ("row", "col")])
def test_bf16_subnormals_are_kept(la, lb, tile):
    M = N = 256
    K = 64
    A = torch.zeros(M, K, dtype=torch.int32)
    B = torch.zeros(K, N, dtype=torch.int32)
    want = {}
    for row, prods in BF16_CASES:
        exact = Fraction(0)
        for k, a, b in prods:
            A[row, k] = a
            B[k, row] = b
            exact += bf16_code_value(a) * bf16_code_value(b)
        want[row] = bf16_rne_code(exact)
    D = run("bf16", A, B, la, lb, tile)
    for row, code in want.items():
        assert int(D[row, row]) == code, (row, hex(int(D[row, row])), hex(code))
    off = D.clone()
    for row in want:
        off[row, row] = 0
    assert int(((off & 0x7FFF) != 0).sum()) == 0, "outputs without products must be zero"


@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col")])
def test_e4m3_subnormal_codes_are_kept(la, lb):
    M = N = 256
    K = 128
    A = torch.zeros(M, K, dtype=torch.int32)
    B = torch.zeros(K, N, dtype=torch.int32)
    want = {}
    for row, prods in E4M3_CASES:
        exact = Fraction(0)
        for k, a, b in prods:
            A[row, k] = a
            B[k, row] = b
            exact += e4m3_code_value(a) * e4m3_code_value(b)
        want[row] = bf16_rne_code(exact)
    D = run("e4m3", A, B, la, lb)
    for row, code in want.items():
        assert int(D[row, row]) == code, (row, hex(int(D[row, row])), hex(code))
