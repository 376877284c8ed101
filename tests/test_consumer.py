"""The tile hand-off ring and its consumer stage (GPU).

gemm_run_with_tile_consumer must give the same D as gemm_run, bit for bit;
its consumer outputs have exactly one correct value given that D: a bit copy
of D, and per 256-column tile slice of every row a sequential fp32 sum and a
maxNum, which the oracle recomputes from the GPU's own D and which must match
exactly.  Outputs are poisoned with NaN first, so an unconsumed tile shows."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full, check_sampled, codes

pytestmark = pytest.mark.gpu


def run_consumer(p: Problem, max_workgroups=0):
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER, max_workgroups=max_workgroups))
    ld = (p.N + 255) // 256
    D = p.new_d()
    Dc = p.new_d()
    rs = torch.full((p.M, ld), float("nan"), dtype=torch.float32, device="cuda")
    rm = torch.full((p.M, ld), float("nan"), dtype=torch.float32, device="cuda")
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
    assert not np.isnan(got_s).any() and not np.isnan(got_m).any(), "a tile was never consumed"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "row sums differ"
    assert np.array_equal(got_m, want_m), "row maxima differ"


def test_tile_consumer_workload_8192():
    w = synth.WORKLOADS[3]
    print(f"[consumer] workload {w.name}", flush=True)
    p = Problem.from_workload(w).to_device()
    plan, D, Dc, rs, rm = run_consumer(p)
    r = check_sampled(p, D, n_random=4096, seed=w.seed)
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
    (768, 768, 8, 2),         # K shorter than the consumer's 33 steps
])
def test_tile_consumer_shapes(M, N, K, mw):
    g = torch.Generator().manual_seed(M + N + K + mw)
    p = Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=0.5, beta=0.25).to_device()
    plan, D, Dc, rs, rm = run_consumer(p, mw)
    r = check_full(p, D)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    check_consumer_outputs(p, D, Dc, rs, rm)


def test_tile_consumer_other_layouts_and_fp8():
    g = torch.Generator().manual_seed(77)
    for la, lb, dt in [("col", "col", synth.BF16), ("row", "col", synth.E4M3), ("col", "row", synth.E4M3)]:
        p = Problem.random(g, 520, 700, 256, la, lb, dtype=dt, alpha=0.03125).to_device()
        plan, D, Dc, rs, rm = run_consumer(p)
        r = check_full(p, D)
        assert r["n_fail"] == 0, (la, lb, dt, r)
        check_consumer_outputs(p, D, Dc, rs, rm)


def test_tile_consumer_is_deterministic_across_grids():
    g = torch.Generator().manual_seed(9)
    p = Problem.random(g, 1280, 1024, 264, "row", "row", dist="normal").to_device()
    outs = [run_consumer(p, mw) for mw in (0, 5, 0)]
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
