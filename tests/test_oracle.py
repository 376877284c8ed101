"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: the format
definitions of bf16 and OCP e4m3, exact rational arithmetic, identity and
permutation matrices, the transpose identity, scaling by powers of two,
integer arithmetic for e4m3 products, and hand-built cases for the acceptance
rule and for the consumer recompute's summation order.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import synth

BF16, E4M3 = oracle.BF16, oracle.E4M3


def codes(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().view(torch.uint8).numpy()


def operand(t: torch.Tensor, rs: int, cs: int) -> oracle.Operand:
    return oracle.Operand(BF16 if t.dtype == torch.bfloat16 else E4M3, codes(t), rs, cs)


def as_storage(logical: torch.Tensor, layout: str) -> torch.Tensor:
    """Store a logical rows x cols matrix in the given layout."""
    return logical.contiguous() if layout == "row" else logical.t().contiguous()


def run_oracle(A_log, B_log, C=None, alpha=1.0, beta=0.0, la="row", lb="row"):
    M, K = A_log.shape
    N = B_log.shape[1]
    A = operand(as_storage(A_log, la), *synth.strides(la, M, K))
    B = operand(as_storage(B_log, lb), *synth.strides(lb, K, N))
    Cop = operand(C.contiguous(), N, 1) if C is not None else None
    return oracle.gemm(M, N, K, A, B, Cop, alpha, beta)


LAYOUTS = list(itertools.product(["row", "col"], ["row", "col"]))


# ---------------------------------------------------------------- decoders (P-a)

def test_bf16_decoder_all_codes_match_torch():
    allc = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(allc.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(c)) for c in allc])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zeros
    assert math.copysign(1.0, oracle.bf16_value(0x8000)) == -1.0


def test_bf16_decoder_closed_forms():
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x3FC0) == 1.5
    assert oracle.bf16_value(0x0001) == 2.0 ** -133       # smallest subnormal
    assert oracle.bf16_value(0x0080) == 2.0 ** -126       # smallest normal
    assert oracle.bf16_value(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.bf16_value(0x7F80) == math.inf
    assert math.isnan(oracle.bf16_value(0x7FC0))


def test_bf16_widening_of_gpu_results_all_codes():
    """bf16_codes_to_f64 (which widens every GPU D before the acceptance
    check) against the exact decoder over all 65,536 codes: equal values with
    equal signs (so -0 stays -0), NaN exactly for the NaN codes."""
    allc = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_codes_to_f64(allc)
    want = np.array([oracle.bf16_value(int(c)) for c in allc], dtype=np.float64)
    nan_codes = ((allc & 0x7F80) == 0x7F80) & ((allc & 0x7F) != 0)
    assert np.array_equal(np.isnan(got), nan_codes)
    assert np.array_equal(np.isnan(want), nan_codes)
    ok = ~nan_codes
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    # spot values from the format: 0x3F80 = 1, 0xC000 = -2, 0x0001 = 2^-133,
    # 0x7F7F = (2 - 2^-7) 2^127, 0xFF80 = -inf
    spot = oracle.bf16_codes_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0xFF80], np.uint16))
    assert spot.tolist() == [1.0, -2.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -np.inf]


def test_e4m3_decoder_all_codes_match_torch():
    allc = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(allc.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in allc])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_e4m3_decoder_closed_forms():
    assert oracle.e4m3_value(0x7E) == 448.0               # largest finite
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6           # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9           # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x3C) == 1.5
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0
    # no infinities in the format: every code other than the two NaNs is finite
    vals = [oracle.e4m3_value(c) for c in range(256) if c not in (0x7F, 0xFF)]
    assert all(math.isfinite(v) for v in vals)


# ------------------------------------------------------- exact dot products (P-c)

def exact_gemm(A_log, B_log, C, alpha, beta):
    """Exact rational result of alpha*A*B + beta*C."""
    a = [[Fraction(float(x)) for x in row] for row in A_log.to(torch.float64).tolist()]
    b = [[Fraction(float(x)) for x in row] for row in B_log.to(torch.float64).tolist()]
    M, K, N = len(a), len(b), len(b[0]) if b else 0
    c = C.to(torch.float64).tolist() if C is not None else None
    out, tabs = [], []
    for i in range(M):
        row, trow = [], []
        for j in range(N):
            s = sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0))
            t = sum((abs(a[i][k] * b[k][j]) for k in range(K)), Fraction(0))
            r = Fraction(alpha) * s
            if beta != 0:
                r += Fraction(beta) * Fraction(c[i][j])
            row.append(r)
            trow.append(t)
        out.append(row)
        tabs.append(trow)
    return out, tabs


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dot_products_against_exact_rationals(la, lb, seed):
    g = torch.Generator().manual_seed(seed)
    M, N, K = [int(x) for x in torch.randint(1, 9, (3,), generator=g)]
    A = synth.random_matrix(g, (M, K))
    B = synth.random_matrix(g, (K, N))
    C = synth.random_matrix(g, (M, N))
    alpha, beta = -1.25, 0.5
    ref, absum = run_oracle(A, B, C, alpha, beta, la, lb)
    ex, ext = exact_gemm(A, B, C, alpha, beta)
    for i in range(M):
        for j in range(N):
            # K fp64 additions: error at most K * 2^-53 * (|alpha| T + |beta c|)
            bound = Fraction(K + 2, 2 ** 53) * (abs(Fraction(alpha)) * ext[i][j]
                                                 + abs(Fraction(beta)) * abs(Fraction(float(C[i, j]))))
            assert abs(Fraction(ref[i, j]) - ex[i][j]) <= bound
            assert abs(Fraction(absum[i, j]) - ext[i][j]) <= Fraction(K, 2 ** 53) * ext[i][j]


def test_one_by_one_all_sign_patterns():
    for sa, sb, sc in itertools.product([1.0, -1.0], repeat=3):
        A = torch.tensor([[1.5 * sa]], dtype=torch.bfloat16)
        B = torch.tensor([[-0.75 * sb]], dtype=torch.bfloat16)
        C = torch.tensor([[3.0 * sc]], dtype=torch.bfloat16)
        ref, absum = run_oracle(A, B, C, 2.0, -0.5)
        assert ref[0, 0] == 2.0 * (1.5 * sa) * (-0.75 * sb) - 0.5 * 3.0 * sc
        assert absum[0, 0] == 1.125


def test_all_ones_gives_k():
    for K in (1, 7, 64, 300):
        A = torch.ones((5, K), dtype=torch.bfloat16)
        B = torch.ones((K, 3), dtype=torch.bfloat16)
        ref, absum = run_oracle(A, B)
        assert np.all(ref == K) and np.all(absum == K)


# ---------------------------------------------------- indexing and strides (P-d)

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_identity_and_permutation(la, lb):
    g = torch.Generator().manual_seed(7)
    n, N = 13, 9
    B = synth.random_matrix(g, (n, N))
    Ident = torch.eye(n, dtype=torch.bfloat16)
    ref, _ = run_oracle(Ident, B, la=la, lb=lb)
    assert np.array_equal(ref, B.to(torch.float64).numpy())
    perm = torch.randperm(n, generator=g)
    P = Ident[perm]
    ref, _ = run_oracle(P, B, la=la, lb=lb)
    assert np.array_equal(ref, B[perm].to(torch.float64).numpy())
    A = synth.random_matrix(g, (N, n))
    ref, _ = run_oracle(A, Ident, la=la, lb=lb)
    assert np.array_equal(ref, A.to(torch.float64).numpy())
    # A * P^T permutes columns
    ref, _ = run_oracle(A, P.t().contiguous(), la=la, lb=lb)
    assert np.array_equal(ref, A[:, perm].to(torch.float64).numpy())


def test_e4m3_identity():
    g = torch.Generator().manual_seed(3)
    B, _ = synth._draw_e4m3(g, (16, 11))
    Ident = torch.eye(16).to(torch.float8_e4m3fn)
    ref, _ = run_oracle(Ident, B)
    assert np.array_equal(ref, B.to(torch.float64).numpy())


# ---------------------------------------------------------- transpose (P-e)

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_transpose_identity_bitwise(la, lb):
    g = torch.Generator().manual_seed(11)
    M, N, K = 17, 23, 41
    A_log = synth.random_matrix(g, (M, K), dist="normal")
    B_log = synth.random_matrix(g, (K, N), dist="normal")
    As, Bs = as_storage(A_log, la), as_storage(B_log, lb)
    a_rs, a_cs = synth.strides(la, M, K)
    b_rs, b_cs = synth.strides(lb, K, N)
    ref, absum = oracle.gemm(M, N, K, operand(As, a_rs, a_cs), operand(Bs, b_rs, b_cs), None, 1.0, 0.0)
    # (A B)^T = B^T A^T with pure stride swaps of the same storage
    ref2, absum2 = oracle.gemm(N, M, K, operand(Bs, b_cs, b_rs), operand(As, a_cs, a_rs), None, 1.0, 0.0)
    assert np.array_equal(ref.T, ref2)
    assert np.array_equal(absum.T, absum2)


# ---------------------------------------------------------- linearity (P-f)

def test_linearity_in_alpha_and_beta():
    g = torch.Generator().manual_seed(5)
    M, N, K = 9, 14, 33
    A = synth.random_matrix(g, (M, K), dist="normal")
    B = synth.random_matrix(g, (K, N), dist="normal")
    C = synth.random_matrix(g, (M, N), dist="normal")
    r1, t1 = run_oracle(A, B)
    for p in (-3, 5):
        rp, tp = run_oracle(A, B, alpha=2.0 ** p)
        assert np.array_equal(rp, r1 * 2.0 ** p)
        assert np.array_equal(tp, t1)
    c64 = C.to(torch.float64).numpy()
    r0, _ = run_oracle(A, B, C, alpha=0.0, beta=-0.75)
    assert np.array_equal(r0, -0.75 * c64)
    rab, _ = run_oracle(A, B, C, alpha=1.5, beta=0.5)
    ra0, _ = run_oracle(A, B, None, alpha=1.5, beta=0.0)
    diff = rab - ra0
    assert np.all(np.abs(diff - 0.5 * c64) <= np.spacing(np.abs(rab)) + np.spacing(np.abs(ra0)))


def test_beta_zero_never_reads_c():
    g = torch.Generator().manual_seed(8)
    A = synth.random_matrix(g, (4, 6))
    B = synth.random_matrix(g, (6, 5))
    nanC = torch.full((4, 5), float("nan"), dtype=torch.bfloat16)
    r_nan, _ = run_oracle(A, B, nanC, 1.0, 0.0)
    r_none, _ = run_oracle(A, B, None, 1.0, 0.0)
    assert np.array_equal(r_nan, r_none)


# ------------------------------------------------------ e4m3 exactness (P-g)

def test_e4m3_sums_are_exact_integers():
    g = torch.Generator().manual_seed(21)
    M, N, K = 6, 7, 512
    qa = torch.randint(0, 256, (M, K), generator=g, dtype=torch.int32).to(torch.uint8)
    qb = torch.randint(0, 256, (K, N), generator=g, dtype=torch.int32).to(torch.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E       # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x7E
    A = qa.view(torch.float8_e4m3fn)
    B = qb.view(torch.float8_e4m3fn)
    ref, absum = run_oracle(A, B)
    # every e4m3 value times 2^9 is an integer of magnitude <= 229376
    ia = (A.to(torch.float64) * 512).to(torch.int64)
    ib = (B.to(torch.float64) * 512).to(torch.int64)
    assert torch.equal(ia.to(torch.float64), A.to(torch.float64) * 512)
    exact = (ia @ ib).numpy()                     # int64, no rounding
    exact_abs = (ia.abs() @ ib.abs()).numpy()
    assert np.array_equal(ref * 2 ** 18, exact.astype(np.float64))
    assert np.array_equal(absum * 2 ** 18, exact_abs.astype(np.float64))


# --------------------------------------------- full vs chosen entries (P-h)

@pytest.mark.parametrize("la,lb", LAYOUTS)
def test_full_and_entries_agree_bitwise(la, lb):
    g = torch.Generator().manual_seed(31)
    M, N, K = 37, 29, 130
    A_log = synth.random_matrix(g, (M, K), dist="normal")
    B_log = synth.random_matrix(g, (K, N), dist="normal")
    C = synth.random_matrix(g, (M, N), dist="normal")
    Aop = operand(as_storage(A_log, la), *synth.strides(la, M, K))
    Bop = operand(as_storage(B_log, lb), *synth.strides(lb, K, N))
    Cop = operand(C, N, 1)
    ref, absum = oracle.gemm(M, N, K, Aop, Bop, Cop, 0.75, -2.0)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    r2, t2 = oracle.gemm_entries(M, N, K, Aop, Bop, Cop, 0.75, -2.0, ii.ravel(), jj.ravel())
    assert np.array_equal(ref.ravel(), r2) and np.array_equal(absum.ravel(), t2)
    # thread count does not change any element
    r3, _ = oracle.gemm(M, N, K, Aop, Bop, Cop, 0.75, -2.0, nthreads=1)
    assert np.array_equal(ref, r3)


def test_zero_k_and_empty():
    A = torch.zeros((3, 0), dtype=torch.bfloat16)
    B = torch.zeros((0, 4), dtype=torch.bfloat16)
    C = torch.arange(12, dtype=torch.float32).reshape(3, 4).to(torch.bfloat16)
    ref, absum = run_oracle(A, B, C, 1.0, 2.0)
    assert np.array_equal(ref, 2.0 * C.to(torch.float64).numpy()) and np.all(absum == 0)
    A = torch.zeros((0, 5), dtype=torch.bfloat16)
    B = torch.zeros((5, 4), dtype=torch.bfloat16)
    ref, _ = run_oracle(A, B)
    assert ref.shape == (0, 4)


# ------------------------------------------------------- acceptance rule (P-i)

def test_checker_bound_edges_bf16():
    ref = np.array([1.0, 1.0, 1.0, 1.0, -4.0, 0.0, 0.0, 1.0])
    absum = np.array([0.0, 0.0, 100.0, 100.0, 0.0, 0.0, 10.0, 0.0])
    D = np.array([
        1.0 + 2.0 ** -8,           # exactly on the relative bound: pass
        1.0 + 2.0 ** -7,           # twice the bound: fail
        1.0 + 2.0 ** -8 + 0.0099,  # inside 2^-8 + 1e-4*100
        1.0 + 2.0 ** -8 + 0.0101,  # outside
        -4.0 - 2.0 ** -6,          # |ref| scales the bound: exactly on it
        0.0,                       # ref 0, absum 0: only 0 passes
        0.0009,                    # ref 0, bound 1e-3: pass
        np.nan,
    ])
    r = oracle.check(D, ref, absum, BF16, 1.0)
    bad = [i for i in range(len(D)) if not (np.isfinite(D[i]) and abs(D[i] - ref[i]) <= 2.0 ** -8 * abs(ref[i]) + 1e-4 * absum[i])]
    assert bad == [1, 3, 7]
    assert r["n_fail"] == 3 and r["n_nonfinite"] == 1 and r["worst_index"] == 7
    # |alpha| scales the sum term
    r = oracle.check(np.array([1.0 + 2.0 ** -8 + 0.009]), np.array([1.0]), np.array([100.0]), BF16, -0.5)
    assert r["n_fail"] == 1
    r = oracle.check(np.array([1.0 + 2.0 ** -8 + 0.0049]), np.array([1.0]), np.array([100.0]), BF16, -0.5)
    assert r["n_fail"] == 0


def test_checker_flags_exactly_the_planted_ulps():
    g = torch.Generator().manual_seed(4)
    ref = (torch.rand((64, 64), generator=g) + 0.5).to(torch.bfloat16)   # values in [0.5, 1.5]
    r64 = ref.to(torch.float64).numpy()
    bits = ref.view(torch.int16).numpy().copy()
    planted3 = [(3, 7), (40, 2), (63, 63)]
    planted1 = [(10, 10), (20, 30)]
    for (i, j) in planted3:
        bits[i, j] += 3
    for (i, j) in planted1:
        bits[i, j] += 1
    D = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    r = oracle.check(D, r64, np.zeros_like(r64), BF16, 1.0)
    # 3 ulps of a value in [0.5, 2) is at least 3*2^-8*|ref|/2 > 2^-8|ref|: flagged.
    # 1 ulp is flagged only when it exceeds 2^-8 |ref| (mantissa below 1.0).
    expected = set(planted3)
    for (i, j) in planted1:
        if D[i, j] - r64[i, j] > 2.0 ** -8 * r64[i, j]:
            expected.add((i, j))
    failed = set(zip(*np.nonzero(np.abs(D - r64) > 2.0 ** -8 * np.abs(r64))))
    assert failed == expected
    assert r["n_fail"] == len(expected)


def test_checker_e4m3_constants():
    r = oracle.check(np.array([1.0 + 2.0 ** -7]), np.array([1.0]), np.array([0.0]), E4M3, 1.0)
    assert r["n_fail"] == 0
    r = oracle.check(np.array([1.0 + 2.0 ** -7 + 0.0199]), np.array([1.0]), np.array([10.0]), E4M3, 1.0)
    assert r["n_fail"] == 0
    r = oracle.check(np.array([1.0 + 2.0 ** -7 + 0.0201]), np.array([1.0]), np.array([10.0]), E4M3, 1.0)
    assert r["n_fail"] == 1


# ------------------------------------------------- consumer recompute (P-j)

def bf16_codes(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rsum(vals, N=None, tile_n=256):
    """The oracle's row sums of one row of values (bf16-exact), all slices."""
    N = len(vals) if N is None else N
    s, _ = oracle.tile_rowstats(bf16_codes([vals]), 1, N, N, 1, tile_n)
    return s[0]


def test_rowstats_sum_is_sequential_in_column_order():
    """Closed forms of the sequential fp32 sum from +0.0 in ascending column
    order, on rows where a pairwise or tree order, the reverse order, an fp64
    accumulator or another start value would each give a different result."""
    tiny = 2.0 ** -24
    # all ones: 256 in any order
    assert rsum([1.0] * 256)[0] == np.float32(256.0)
    # 1 first, then 255 x 2^-24: each addition is half an ulp of 1 and rounds
    # back to 1 (ties to even), so the sum stays 1.  Pairwise or tree orders
    # add the small values among themselves first (to 127.5 ulps of 1), and
    # fp64 keeps them: both give 1 + 2^-16.
    assert rsum([1.0] + [tiny] * 255)[0] == np.float32(1.0)
    # the same values with the 1 last: the small ones add exactly to
    # 255 x 2^-24 first, and 1 + 127.5 ulps rounds to 1 + 128 ulps = 1 + 2^-16.
    # (A descending order would give 1.)
    assert rsum([tiny] * 255 + [1.0])[0] == np.float32(1.0 + 2.0 ** -16)
    # 2^24 first, then 255 ones: every + 1 is half an ulp of 2^24 and rounds
    # back (ties to even): 2^24.
    assert rsum([2.0 ** 24] + [1.0] * 255)[0] == np.float32(2.0 ** 24)
    # 255 ones first (exactly 255), then 2^24: 2^24 + 255 lies halfway between
    # 2^24 + 254 and 2^24 + 256 and rounds to the even one, 2^24 + 256.
    assert rsum([1.0] * 255 + [2.0 ** 24])[0] == np.float32(2.0 ** 24 + 256)
    # the position of the large value decides how many ones survive: with
    # 2^24 at column 100 the first 100 ones add exactly (100), 2^24 + 100 is
    # exact (even), and the 155 ones after it each round away.
    row = [1.0] * 100 + [2.0 ** 24] + [1.0] * 155
    assert rsum(row)[0] == np.float32(2.0 ** 24 + 100)


def test_rowstats_sum_starts_at_plus_zero_and_covers_valid_columns_only():
    # from +0.0: +0 + (-0) = +0, so a slice of negative zeros sums to +0
    # (starting from the first value would keep -0)
    s = rsum([-0.0] * 256)
    assert s.view(np.uint32)[0] == 0x00000000
    # a slice cut short by N covers only its columns: 300 columns give a
    # second slice of 44 values
    row = [0.5] * 256 + [0.25] * 44
    s = rsum(row)
    assert s[0] == np.float32(128.0) and s[1] == np.float32(11.0)
    # slices never mix: a huge value in slice 0 does not absorb slice 1
    row = [2.0 ** 24] + [0.0] * 255 + [1.0] * 3
    s = rsum(row)
    assert s[0] == np.float32(2.0 ** 24) and s[1] == np.float32(3.0)
    # NaN and infinities propagate through the sum as IEEE addition says
    assert np.isnan(rsum([1.0, float("nan")] + [0.0] * 254)[0])
    assert rsum([float("inf")] + [1.0] * 255)[0] == np.float32(np.inf)
    assert np.isnan(rsum([float("inf"), float("-inf")] + [0.0] * 254)[0])
    # other slice widths follow the same definition
    s, _ = oracle.tile_rowstats(bf16_codes([[1.0] + [2.0 ** -24] * 7]), 1, 8, 8, 1, 8)
    assert s[0, 0] == np.float32(1.0)


def test_rowstats_sum_brute_force_on_random_rows():
    """Against a step-by-step numpy fp32 recurrence (one float32 addition per
    column, in column order), on rows whose magnitudes span many binades so
    that any other order or precision rounds differently somewhere."""
    rng = np.random.default_rng(7)
    M, N = 40, 700
    vals = rng.standard_normal((M, N)) * np.exp2(rng.integers(-20, 20, (M, N)))
    D = bf16_codes(vals.tolist())
    s, _ = oracle.tile_rowstats(D, M, N, N, 1, 256)
    x = torch.from_numpy(D.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    x = x.reshape(M, N)
    differs_from_pairwise = 0
    for r in range(M):
        for t in range(3):
            seg = x[r, 256 * t: min(N, 256 * t + 256)]
            acc = np.float32(0.0)
            for v in seg:
                acc = np.float32(acc + v)
            assert s[r, t].view(np.uint32) == acc.view(np.uint32), (r, t)
            differs_from_pairwise += int(np.float32(np.sum(seg)) != acc)
    # the rows are chosen so that numpy's pairwise sum differs often: the pin
    # would catch a pairwise oracle
    assert differs_from_pairwise > 20


def test_rowstats_max_rules():
    def rmax(vals):
        _, m = oracle.tile_rowstats(bf16_codes([vals]), 1, len(vals), len(vals), 1, 256)
        return m[0, 0]
    base = [-3.0] * 256
    v = list(base); v[200] = 0.0; v[10] = -0.0
    assert np.float32(rmax(v)).view(np.uint32) == 0x00000000        # +0 beats -0 wherever it is
    v = list(base); v[10] = 0.0; v[200] = -0.0
    assert np.float32(rmax(v)).view(np.uint32) == 0x00000000
    v = list(base); v[5] = float("nan"); v[100] = -1.0
    assert rmax(v) == np.float32(-1.0)                               # NaN ignored
    assert rmax([float("nan")] * 256) == np.float32(-np.inf)         # nothing left: -inf
    v = list(base); v[255] = 2.0 ** 100
    assert rmax(v) == np.float32(2.0 ** 100)


def test_rowstats_slices_and_max():
    M, N = 3, 600                               # slices of 256, 256, 88 columns
    vals = -np.abs(np.random.default_rng(0).standard_normal((M, N))) - 1.0
    vals[1, 300] = -0.0
    vals[2, 520] = 0.0
    D = bf16_codes(vals.tolist())
    s, m = oracle.tile_rowstats(D, M, N, N, 1, 256)
    assert s.shape == (3, 3) and m.shape == (3, 3)
    dv = torch.from_numpy(D.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    for r in range(M):
        for t, (lo, hi) in enumerate([(0, 256), (256, 512), (512, 600)]):
            seg = dv[r, lo:hi]
            # all values are in [-5, -1] or zero and have 8 significant bits,
            # so every partial sum of up to 256 of them is exact in fp32 and
            # any order gives the exact sum
            assert s[r, t] == np.float32(np.sum(seg.astype(np.float64)))
            assert m[r, t] == seg.max()
    assert m[1, 1] == 0.0 and m[2, 2] == 0.0
    # column-major D gives the same statistics
    Dt = np.ascontiguousarray(D.reshape(M, N).T)
    s2, m2 = oracle.tile_rowstats(Dt, M, N, 1, M, 256)
    assert np.array_equal(s, s2) and np.array_equal(m, m2)
