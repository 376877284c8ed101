"""Stream-K (GPU): the tiles of the last round cut into K-stage ranges over
the whole grid, their fp32 partials added by the fixup in the workspace.

Every case is checked element by element against the oracle within the
GEMM tolerance (a K split changes only the fp32 summation order).  A plan
must give the same D bit for bit on every run: the partials are added in K
order whatever the arrival order, and the arrival counters must be back at
zero after each run (a counter left over would make the wrong wave finish a
tile on the next run)."""
import pytest
import torch

from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full

pytestmark = pytest.mark.gpu


def sk_plan(p: Problem, max_workgroups=0, flags=migemm.MIGEMM_F_STREAM_K_FORCE):
    plan = migemm.Plan(p.desc(flags=flags, max_workgroups=max_workgroups))
    size = plan.workspace_size
    ws = torch.empty(size, dtype=torch.uint8, device="cuda") if size else None
    if ws is not None:
        migemm.gemm_workspace_init(plan.handle, ws)
    return plan, ws


def sk_runs(p: Problem, plan, ws, runs=2):
    outs = []
    for _ in range(runs):
        D = p.new_d()
        migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, ws)
        outs.append(D)
    torch.cuda.synchronize()
    return outs


def assert_same_bits(outs):
    for D in outs[1:]:
        assert torch.equal(D.view(torch.int16), outs[0].view(torch.int16)), "runs differ"


def test_stream_k_ragged_4000x3000x5000():
    # 16 x 12 = 192 tiles on 256 compute units: all of them cut into units.
    w = synth.WORKLOADS[2]
    print(f"[stream-k] workload {w.name}", flush=True)
    p = Problem.from_workload(w).to_device()
    plan, ws = sk_plan(p)
    info = plan.info
    assert info.stream_k_tiles == info.num_tiles == 192
    assert info.stream_k_units_per_tile == -(-w.K // info.tile_k)
    assert info.grid == min(info.cu_count, 192 * info.stream_k_units_per_tile)
    outs = sk_runs(p, plan, ws, runs=3)
    r = check_full(p, outs[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    assert_same_bits(outs)


def test_stream_k_one_gpu_share_8192x1024x8192():
    # One GPU's share when N is split 8 ways: 128 tiles, 256 compute units.
    g = torch.Generator().manual_seed(81)
    p = Problem.random(g, 8192, 1024, 8192, "row", "row", dist="normal").to_device()
    print("[stream-k] 8192x1024x8192", flush=True)
    plan, ws = sk_plan(p)
    assert plan.info.stream_k_tiles == 128
    outs = sk_runs(p, plan, ws, runs=2)
    r = check_full(p, outs[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    assert_same_bits(outs)


@pytest.mark.parametrize("M,N,K,mw,beta", [
    (1024, 1024, 1000, 5, 0.0),     # 16 tiles on 5: 10 whole, then 6 cut over 5
    (1024, 1024, 520, 3, 0.5),      # 16 tiles on 3: 12 whole, 4 cut over 3; beta
    (600, 700, 136, 7, 0.0),        # ragged edges, 3 x 3 tiles, 3 stages each
    (256, 256, 8, 4, 0.0),          # K inside one stage: 1 unit, grid shrinks to 1
    (512, 512, 4096, 0, 0.25),      # 4 tiles x 64 stages over all compute units
    (768, 512, 1024, 1, 0.0),       # one workgroup: every tile whole
    (512, 256, 256, 3, 0.0),        # 2 tiles x 4 stages on 3: ranges 2, 3, 3
])
def test_stream_k_shapes(M, N, K, mw, beta):
    g = torch.Generator().manual_seed(M + N + K + mw)
    p = Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=0.75, beta=beta).to_device()
    print(f"[stream-k] {M}x{N}x{K} grid cap {mw} beta {beta}", flush=True)
    plan, ws = sk_plan(p, mw)
    outs = sk_runs(p, plan, ws)
    r = check_full(p, outs[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, (plan.info.grid, r)
    assert_same_bits(outs)


def test_stream_k_partials_cross_xcds_bitwise_over_runs():
    # 64 tiles of 64 stages on every compute unit: 4 contributors per tile,
    # spread over XCDs with private L2s.  A partial read before its writer's
    # stores were visible would change the sum, so 20 runs must agree bit
    # for bit (and the first must pass the oracle).
    g = torch.Generator().manual_seed(64)
    p = Problem.random(g, 2048, 2048, 4096, "row", "row", dist="normal").to_device()
    plan, ws = sk_plan(p)
    assert plan.info.stream_k_tiles == 64 and plan.info.grid == plan.info.cu_count
    outs = sk_runs(p, plan, ws, runs=20)
    r = check_full(p, outs[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    assert_same_bits(outs)


def test_stream_k_layouts_and_fp8():
    g = torch.Generator().manual_seed(23)
    cases = [("col", "col", synth.BF16, "row"), ("row", "col", synth.E4M3, "row"),
             ("col", "row", synth.E4M3, "row"), ("row", "row", synth.BF16, "col")]
    for la, lb, dt, dl in cases:
        p = Problem.random(g, 1000, 900, 776 if dt == synth.BF16 else 768, la, lb, dtype=dt,
                           alpha=0.03125 if dt == synth.E4M3 else 1.0, d_layout=dl).to_device()
        print(f"[stream-k] layouts {la} {lb} {dt} D {dl}", flush=True)
        plan, ws = sk_plan(p, 48)
        outs = sk_runs(p, plan, ws)
        r = check_full(p, outs[0])
        assert r["n_fail"] == 0, (la, lb, dt, dl, r)
        assert_same_bits(outs)


def test_stream_k_matches_whole_tiles_within_tolerance():
    # The whole-tile plan and the stream-K plan sum K in different groupings;
    # both must pass the oracle, and most entries agree exactly.
    g = torch.Generator().manual_seed(5)
    p = Problem.random(g, 1280, 768, 2048, "row", "row", dist="normal").to_device()
    plan, ws = sk_plan(p)
    D_sk = sk_runs(p, plan, ws, runs=1)[0]
    D_dp = p.run(migemm.Plan(p.desc()))
    torch.cuda.synchronize()
    for D in (D_sk, D_dp):
        r = check_full(p, D)
        assert r["n_fail"] == 0, r
    same = (D_sk.view(torch.int16) == D_dp.view(torch.int16)).float().mean().item()
    assert same > 0.5, same


def test_stream_k_k_zero_needs_no_workspace():
    g = torch.Generator().manual_seed(3)
    p = Problem.random(g, 300, 200, 0, "row", "row", alpha=1.0, beta=0.5).to_device()
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE))
    assert plan.workspace_size == 0 and plan.info.stream_k_tiles == 0
    D = p.new_d()
    migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, None)
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert r["n_fail"] == 0, r


def test_stream_k_cost_model_choices():
    # MIGEMM_F_STREAM_K splits only where the model predicts a gain.
    def chosen(M, N, K, mw=0):
        d = migemm.make_desc(M, N, K, 1, 1, K, 1, N, 1, N, 1, N, 1, flags=migemm.MIGEMM_F_STREAM_K,
                             max_workgroups=mw)
        return migemm.Plan(d).info
    share = chosen(8192, 1024, 8192)       # 128 tiles of 128 stages on 256 CUs: split
    assert share.stream_k_tiles == 128 and share.grid == share.cu_count
    assert chosen(4000, 3000, 5000).stream_k_tiles == 0   # 79 stages: 60 + fixup > 79
    assert chosen(8192, 8192, 8192).stream_k_tiles == 0   # 4 rounds of whole tiles
    assert chosen(2048, 2048, 8192).stream_k_tiles == 64  # 64 tiles of 128 stages
    assert chosen(256, 256, 256).stream_k_tiles == 0      # one tile of 4 stages


def test_stream_k_workspace_errors():
    g = torch.Generator().manual_seed(4)
    p = Problem.random(g, 512, 512, 512).to_device()
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE))
    size = plan.workspace_size
    assert size > 0 and size % 256 == 0
    D = p.new_d()
    st = migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, 1.0, 0.0, None, check=False)
    assert st == migemm.MIGEMM_ERR_INVALID_ARG
    ws = torch.empty(size + 256, dtype=torch.uint8, device="cuda")
    st = migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, 1.0, 0.0, ws[16:], check=False)
    assert st == migemm.MIGEMM_ERR_MISALIGNED
    assert migemm.gemm_workspace_init(plan.handle, None, check=False) == migemm.MIGEMM_ERR_INVALID_ARG
    assert migemm.gemm_workspace_init(plan.handle, ws[16:], check=False) == migemm.MIGEMM_ERR_MISALIGNED
    # A plan without stream-K tiles takes no workspace, and init is a no-op.
    plain = migemm.Plan(p.desc())
    assert plain.workspace_size == 0
    assert migemm.gemm_workspace_init(plain.handle, None) == migemm.MIGEMM_OK
