"""The tile hand-off ring and its consumer stage (GPU).

gemm_run_with_tile_consumer must give the same D as gemm_run, bit for bit;
its consumer outputs have exactly one correct value given that D: a bit copy
of D, and per 256-column tile slice of every row the fp32 sum taken one
column at a time in ascending order from +0.0 and the largest non-NaN value
(-0 < +0), which the
oracle recomputes from the GPU's own D and which must match exactly.
Outputs are poisoned first with a NaN whose payload no result can carry
(results derived from bf16 values have zero low 16 bits), so an unconsumed
tile shows.  Both schedules of the consumer stage run every case: right
after each tile's commit on the tile staged in LDS (the default), and
inside the next tile's K loop on the tile fetched back from D
(MIGEMM_F_CONSUMER_OVERLAP); their outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full, codes, workload_reference

pytestmark = pytest.mark.gpu

POISON = 0x7FBADBAD


def poisoned(rows, cols):
    return torch.full((rows, cols), POISON, dtype=torch.int32, device="cuda").view(torch.float32)


MODES = {"staged": migemm.MIGEMM_F_TILE_CONSUMER,
         "overlap": migemm.MIGEMM_F_TILE_CONSUMER | migemm.MIGEMM_F_CONSUMER_OVERLAP}


def run_consumer(p: Problem, max_workgroups=0, mode="staged"):
    plan = migemm.Plan(p.desc(flags=MODES[mode], max_workgroups=max_workgroups))
    ld = (p.N + 255) // 256
    D = p.new_d()
    Dc = p.new_d()
    rs = poisoned(p.M, ld)
    rm = poisoned(p.M, ld)
    migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, rs, rm, Dc)
    torch.cuda.synchronize()
    return plan, D, Dc, rs, rm


def check_consumer_outputs(p: Problem, D, Dc, rs, rm):
    """Exact checks of the consumer stage against a recompute from D."""
    dcodes = codes(D).reshape(p.d_shape)
    ccodes = codes(Dc).reshape(p.d_shape)
    assert np.array_equal(dcodes[:, :p.N], ccodes[:, :p.N]), "D_copy differs from D"
    want_s, want_m = oracle.tile_rowstats(dcodes, p.M, p.N, p.d_rs, p.d_cs, 256)
    got_s, got_m = rs.cpu().numpy(), rm.cpu().numpy()
    assert not (got_s.view(np.uint32) == POISON).any(), "a tile's sums were never written"
    assert not (got_m.view(np.uint32) == POISON).any(), "a tile's maxima were never written"
    # Sums: identical bits, except that a NaN may carry any payload.  Maxima
    # are never NaN: identical bits (so -0 and +0 are told apart).
    both_nan = np.isnan(got_s) & np.isnan(want_s)
    same_s = (got_s.view(np.uint32) == want_s.view(np.uint32)) | both_nan
    assert same_s.all(), "row sums differ at %s" % (np.argwhere(~same_s)[:5].tolist(),)
    same_m = got_m.view(np.uint32) == want_m.view(np.uint32)
    assert same_m.all(), "row maxima differ at %s" % (np.argwhere(~same_m)[:5].tolist(),)


@pytest.mark.parametrize("mode", MODES)
def test_tile_consumer_workload_8192(mode):
    w = synth.WORKLOADS[3]
    print(f"[consumer] workload {w.name} {mode}", flush=True)
    p = Problem.from_workload(w).to_device()
    plan, D, Dc, rs, rm = run_consumer(p, mode=mode)
    r = check_full(p, D, workload_reference(w, p))
    print(f"[consumer] {w.name} {mode}: {r['n']} elements, {r['n_fail']} outside the bound, "
          f"worst ratio {r['worst_ratio']:.4f}", flush=True)
    assert r["n"] == w.M * w.N
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    check_consumer_outputs(p, D, Dc, rs, rm)
    D2 = p.run(migemm.Plan(p.desc()))
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16)), "consumer variant changed D"


@pytest.mark.parametrize("M,N,K,mw", [
    (256, 256, 64, 0),        # one tile: consumed after the loop
    (1000, 600, 136, 0),      # ragged tile edges, N tail of 88 columns
    (300, 300, 264, 0),       # N = 300: a partial 16-byte chunk at the row end
    (1024, 1024, 520, 1),     # one workgroup: 16 tiles through a 2-slot ring
    (1024, 1280, 1000, 3),    # uneven tiles per workgroup
    (768, 768, 8, 2),         # K shorter than the overlapped copy's 33 steps
    (520, 600, 0, 2),         # K = 0: D = beta * C, still handed off tile by tile
])
@pytest.mark.parametrize("mode", MODES)
def test_tile_consumer_shapes(M, N, K, mw, mode):
    g = torch.Generator().manual_seed(M + N + K + mw)
    p = Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=0.5, beta=0.25).to_device()
    print(f"[consumer] {M}x{N}x{K} grid cap {mw} {mode}", flush=True)
    plan, D, Dc, rs, rm = run_consumer(p, mw, mode)
    r = check_full(p, D)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    check_consumer_outputs(p, D, Dc, rs, rm)


def special_rows(rng, n):
    """bf16 codes for rows of n columns whose statistics exercise the edge
    rules: NaNs of both signs (ignored by the maximum), infinities, signed
    zeros (-0 < +0), subnormals, rows with no number at all (maximum -inf)."""
    nan_codes = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF, 0xFFFF], dtype=np.uint16)
    def normal(k):
        return (torch.randn(k, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
                .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    rows = []
    # values with a few NaNs and infinities
    r = normal(n); m = rng.random(n)
    r[m < 0.05] = rng.choice(nan_codes, (m < 0.05).sum())
    r[(m >= 0.05) & (m < 0.07)] = 0x7F80
    r[(m >= 0.07) & (m < 0.09)] = 0xFF80
    rows.append(r)
    rows.append(rng.choice(nan_codes, n).astype(np.uint16))                      # no number
    r = normal(n) | 0x8000; r[rng.random(n) < 0.1] = 0x8000; rows.append(r)    # max is -0
    rows.append(rng.choice(np.array([0x0000, 0x8000], dtype=np.uint16), n))      # +0 beats -0
    rows.append(np.full(n, 0x8000, dtype=np.uint16))                            # only -0
    rows.append(np.full(n, 0xFF80, dtype=np.uint16))                            # only -inf
    r = rng.choice(nan_codes, n).astype(np.uint16); r[rng.integers(n)] = 0x7F80; rows.append(r)
    r = rng.choice(np.array([0xFFC0, 0xFF81, 0xFFFF], dtype=np.uint16), n)
    r[rng.integers(n)] = 0xFF80; rows.append(r)                                 # -NaNs and -inf
    r = rng.choice(np.array([0x7FC0, 0x7FFF], dtype=np.uint16), n)
    r[rng.integers(n)] = 0x7F7F; rows.append(r)                                 # +NaNs, max finite
    rows.append(rng.integers(0, 0x80, n).astype(np.uint16) | rng.choice(np.array([0, 0x8000], dtype=np.uint16), n))
    rows.append(normal(n))
    return rows


@pytest.mark.parametrize("mode", MODES)
def test_tile_consumer_special_values(mode):
    # alpha = -1 and beta = 1 with zero rows in A give D = (-0) + C exactly on
    # those rows, so C plants NaN, +-inf, -0 and subnormal codes in D.  N has
    # a 56-column tail, so both the whole-slice and the partial-slice forms
    # of the fold see them.
    M, N, K = 512, 824, 64
    g = torch.Generator().manual_seed(2024)
    p = Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=-1.0, beta=1.0)
    rng = np.random.default_rng(5)
    A = p.A.view(torch.int16).numpy()
    C = p.C.view(torch.int16).numpy().view(np.uint16)
    kinds = special_rows(rng, N)
    for r in range(0, M, 2):
        A[r, :] = 0
        C[r, :N] = kinds[(r // 2) % len(kinds)]
    print(f"[consumer] special values {M}x{N}x{K} {mode}", flush=True)
    p.to_device()
    plan, D, Dc, rs, rm = run_consumer(p, mode=mode)
    check_consumer_outputs(p, D, Dc, rs, rm)
    dc = codes(D).reshape(p.d_shape)[:, :N]
    want = C[0::2, :N]
    # (a NaN may come out quieted or with another payload, a subnormal flushed)
    got = dc[0::2]
    same = ((got == want) | (((got & 0x7FFF) > 0x7F80) & ((want & 0x7FFF) > 0x7F80))
            | (((want & 0x7F80) == 0) & ((got & 0x7FFF) == 0)))
    assert same.all(), "zero rows of A must give D = C"
    D2 = p.run(migemm.Plan(p.desc()))
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16)), "consumer variant changed D"


@pytest.mark.parametrize("mode", MODES)
def test_tile_consumer_other_layouts_and_fp8(mode):
    g = torch.Generator().manual_seed(77)
    for la, lb, dt in [("col", "col", synth.BF16), ("row", "col", synth.E4M3), ("col", "row", synth.E4M3)]:
        p = Problem.random(g, 520, 700, 256, la, lb, dtype=dt, alpha=0.03125).to_device()
        print(f"[consumer] layouts {la} {lb} {dt} {mode}", flush=True)
        plan, D, Dc, rs, rm = run_consumer(p, mode=mode)
        r = check_full(p, D)
        assert r["n_fail"] == 0, (la, lb, dt, r)
        check_consumer_outputs(p, D, Dc, rs, rm)


def test_tile_consumer_is_deterministic_across_grids_and_schedules():
    # Same outputs bit for bit whatever the grid and whichever schedule runs
    # the consumer stage.
    g = torch.Generator().manual_seed(9)
    p = Problem.random(g, 1280, 1024, 264, "row", "row", dist="normal").to_device()
    outs = [run_consumer(p, mw, mode) for mw in (0, 5, 0) for mode in MODES]
    for o in outs[1:]:
        for a, b in zip(o[1:], outs[0][1:]):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_tile_consumer_requires_flag_and_buffers():
    g = torch.Generator().manual_seed(1)
    p = Problem.random(g, 256, 256, 64).to_device()
    plain = migemm.Plan(p.desc())
    D = p.new_d()
    st = migemm.gemm_run_with_tile_consumer(plain.handle, p.dA, p.dB, None, D, 1.0, 0.0, D, D, D,
                                            check=False)
    assert st == migemm.MIGEMM_ERR_INVALID_ARG
    cons = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER))
    st = migemm.gemm_run_with_tile_consumer(cons.handle, p.dA, p.dB, None, D, 1.0, 0.0, None, D, D,
                                            check=False)
    assert st == migemm.MIGEMM_ERR_INVALID_ARG
