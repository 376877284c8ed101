"""Non-finite inputs (GPU): NaN and infinities inside A and B.

The GEMM is the plain definition in IEEE arithmetic, so a NaN anywhere in a
dot product makes that output NaN, an infinity times a nonzero finite value
an infinity of the product's sign, an infinity times zero NaN, and
infinities of both signs in one sum NaN.  None of these depend on the order
of the additions (no finite value here comes near overflow), so the oracle,
which follows the same rules in fp64, fixes the class of every output:
NaN, +inf, -inf or finite.  Every output is compared with it: the class
exactly (any NaN payload), and finite ones within the usual tolerance.

bf16 has NaNs and infinities; OCP e4m3 ("fn") has NaN codes (S.1111.111)
and no infinity."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, codes

pytestmark = pytest.mark.gpu

BF16_NAN, BF16_PINF, BF16_NINF = 0x7FC0, 0x7F80, 0xFF80
E4M3_NAN, E4M3_NNAN = 0x7F, 0xFF


def plant(t: torch.Tensor, rs: int, cs: int, r: int, c: int, code: int):
    """Set logical element (r, c) of an operand stored with strides (rs, cs)."""
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).reshape(-1)[r * rs + c * cs] = code - 0x10000 if code >= 0x8000 else code
    else:
        t.view(torch.uint8).reshape(-1)[r * rs + c * cs] = code


def classify(x: np.ndarray) -> np.ndarray:
    """0 finite, 1 NaN, 2 +inf, 3 -inf."""
    out = np.zeros(x.shape, dtype=np.int8)
    out[np.isnan(x)] = 1
    out[np.isposinf(x)] = 2
    out[np.isneginf(x)] = 3
    return out


def check_classes(p: Problem, D: torch.Tensor):
    ref, absum = p.oracle_full()
    got = p.d_values(D)
    want_cls, got_cls = classify(ref), classify(got)
    bad = np.argwhere(want_cls != got_cls)
    assert bad.size == 0, (f"{len(bad)} outputs of the wrong class, first at {tuple(bad[0])}: "
                           f"oracle {ref[tuple(bad[0])]}, GPU {got[tuple(bad[0])]}")
    fin = want_cls == 0
    r = oracle.check(got[fin], ref[fin], absum[fin], p.in_dtype(), p.alpha)
    assert r["n_fail"] == 0, r
    return int((want_cls == 1).sum()), int((want_cls >= 2).sum()), int(fin.sum())


@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_bf16_nan_and_infinities_propagate(la, lb):
    M, N, K = 300, 280, 200
    g = torch.Generator().manual_seed(900)
    p = Problem.random(g, M, N, K, la, lb, dist="normal", alpha=0.5, beta=0.25)
    plant(p.A, p.a_rs, p.a_cs, 5, 17, BF16_NAN)       # row 5: NaN
    plant(p.A, p.a_rs, p.a_cs, 9, 3, BF16_PINF)       # row 9: +-inf by the sign of B[3, j]
    plant(p.B, p.b_rs, p.b_cs, 40, 7, BF16_NINF)      # column 7: -+inf by the sign of A[i, 40]
    plant(p.B, p.b_rs, p.b_cs, 199, 270, BF16_NAN)    # column 270 (last K row, last tile): NaN
    plant(p.A, p.a_rs, p.a_cs, 260, 120, BF16_PINF)   # row 260 (second tile row): +inf ...
    plant(p.B, p.b_rs, p.b_cs, 120, 11, 0)            # ... times a zero in column 11: NaN there
    plant(p.A, p.a_rs, p.a_cs, 261, 50, BF16_PINF)    # row 261: +inf and -inf in one sum when
    plant(p.A, p.a_rs, p.a_cs, 261, 51, BF16_NINF)    # B[50, j] and B[51, j] share a sign
    p.to_device()
    plan = migemm.Plan(p.desc())
    D = p.new_d()
    migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta)
    torch.cuda.synchronize()
    n_nan, n_inf, n_fin = check_classes(p, D)
    print(f"[nonfinite] bf16 {la}/{lb}: {n_nan} NaN, {n_inf} inf, {n_fin} finite outputs", flush=True)
    assert n_nan > 2 * N and n_inf > N

    # The other tile height (192 or 256 rows): the same bits, NaNs included.
    other = migemm.MIGEMM_F_TILE_M256 if plan.info.tile_m == 192 else migemm.MIGEMM_F_TILE_M192
    Do = p.new_d()
    migemm.gemm_run(migemm.Plan(p.desc(flags=other)), p.dA, p.dB, p.dC, Do, p.alpha, p.beta)
    torch.cuda.synchronize()
    assert torch.equal(Do.view(torch.int16), D.view(torch.int16))

    # Stream-K: the specials meet in partial sums and in the fixup's adds.
    pk = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K | migemm.MIGEMM_F_STREAM_K_FORCE))
    ws = torch.empty(pk.workspace_size, dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(pk.handle, ws)
    Dk = p.new_d()
    migemm.gemm_run(pk.handle, p.dA, p.dB, p.dC, Dk, p.alpha, p.beta, ws)
    torch.cuda.synchronize()
    check_classes(p, Dk)

    # The tile consumer (row-major D only): D bit for bit as gemm_run's, the
    # copy bit for bit, and the row statistics over NaN and infinite values
    # exactly as the oracle recomputes them from D.
    if p.d_layout == "row":
        pc = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER))
        tn = -(-N // 256)
        D2 = p.new_d()
        Dc = torch.full_like(D2, float("nan"))
        rs = torch.full((M, tn), 1.0, dtype=torch.float32, device="cuda")
        rm = torch.full_like(rs, 1.0)
        migemm.gemm_run_with_tile_consumer(pc.handle, p.dA, p.dB, p.dC, D2, p.alpha, p.beta, rs,
                                           rm, Dc)
        torch.cuda.synchronize()
        assert torch.equal(D2.view(torch.int16), D.view(torch.int16))
        assert torch.equal(Dc.view(torch.int16)[:, :N], D.view(torch.int16)[:, :N])
        dc = codes(D).reshape(p.d_shape)
        want_s, want_m = oracle.tile_rowstats(dc, M, N, p.d_rs, p.d_cs, 256)
        got_s, got_m = rs.cpu().numpy(), rm.cpu().numpy()
        assert np.array_equal(classify(got_s), classify(want_s))
        fs = np.isfinite(want_s)
        assert np.array_equal(got_s[fs].view(np.uint32), want_s[fs].view(np.uint32))
        assert np.array_equal(np.where(got_m == 0, 0, got_m), np.where(want_m == 0, 0, want_m))


@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col")])
def test_e4m3_nan_codes_propagate(la, lb):
    M, N, K = 300, 280, 384
    g = torch.Generator().manual_seed(901)
    p = Problem.random(g, M, N, K, la, lb, dtype=synth.E4M3, alpha=0.03125)
    plant(p.A, p.a_rs, p.a_cs, 5, 17, E4M3_NAN)
    plant(p.A, p.a_rs, p.a_cs, 290, 383, E4M3_NNAN)   # last K element of a partial tile row
    plant(p.B, p.b_rs, p.b_cs, 130, 260, E4M3_NAN)
    p.to_device()
    plan = migemm.Plan(p.desc())
    D = p.new_d()
    migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, p.alpha, 0.0)
    torch.cuda.synchronize()
    n_nan, n_inf, n_fin = check_classes(p, D)
    print(f"[nonfinite] e4m3 {la}/{lb}: {n_nan} NaN, {n_inf} inf, {n_fin} finite outputs", flush=True)
    assert n_nan == 2 * N + M - 2 and n_inf == 0
