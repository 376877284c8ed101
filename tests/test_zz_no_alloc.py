"""gemm_run_no_alloc: the entry point that allocates nothing (GPU).

It must give what gemm_run gives with a caller-owned workspace, bit for bit,
for stream-K plans that use its fixed device scratch: on two calls in a row,
the second with a smaller problem (so a smaller counter area and partials
over the first call's leftovers), and every D must also pass the oracle.
Plans without a workspace run as gemm_run does; plans whose workspace
exceeds the scratch are rejected before anything is launched."""
import pytest
import torch

from warp_specialized_pipelined_amd import migemm
from tests.helpers import Problem, check_full

pytestmark = pytest.mark.gpu


def ok(r):
    return r["n_fail"] == 0 and r["n_nonfinite"] == 0


def run_both(p, plan):
    """D from gemm_run with a fresh caller workspace, and D from
    gemm_run_no_alloc, on the same plan and inputs."""
    ws = torch.empty(max(plan.workspace_size, 256), dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(plan.handle, ws)
    D_ref = p.new_d()
    migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D_ref, p.alpha, p.beta, ws)
    D = p.new_d()
    migemm.gemm_run_no_alloc(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta)
    torch.cuda.synchronize()
    return D_ref, D


def test_no_alloc_matches_gemm_run_on_two_calls_in_a_row():
    # (M, N, K, grid cap): 64 tiles of 64 stages over 48 workgroups, then 12
    # tiles of 16 stages over 20: both split tiles, the second plan's
    # workspace (counters and partials) smaller than the first's.
    sizes = []
    for i, (M, N, K, mw) in enumerate([(2048, 2048, 4096, 48), (1000, 700, 1000, 20)]):
        g = torch.Generator().manual_seed(700 + i)
        p = Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=0.75,
                           beta=0.5).to_device()
        plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=mw))
        print(f"[no-alloc] call {i}: {M}x{N}x{K} grid {plan.info.grid} "
              f"workspace {plan.workspace_size}", flush=True)
        assert plan.info.stream_k_tiles > 0
        assert 0 < plan.workspace_size <= migemm.MIGEMM_NO_ALLOC_SCRATCH_BYTES
        sizes.append(plan.workspace_size)
        D_ref, D = run_both(p, plan)
        assert torch.equal(D.view(torch.int16), D_ref.view(torch.int16)), "differs from gemm_run"
        r = check_full(p, D)
        assert ok(r), r
    assert sizes[1] < sizes[0]


def test_no_alloc_repeated_calls_reset_their_counters():
    g = torch.Generator().manual_seed(710)
    p = Problem.random(g, 768, 1024, 2000, "row", "col", dist="normal").to_device()
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=37))
    outs = []
    for _ in range(3):
        D = p.new_d()
        migemm.gemm_run_no_alloc(plan.handle, p.dA, p.dB, None, D, p.alpha, 0.0)
        outs.append(D)
    torch.cuda.synchronize()
    for D in outs[1:]:
        assert torch.equal(D.view(torch.int16), outs[0].view(torch.int16))
    assert ok(check_full(p, outs[0]))


def test_no_alloc_without_workspace_is_gemm_run():
    g = torch.Generator().manual_seed(711)
    p = Problem.random(g, 600, 520, 264, "row", "row", dist="normal").to_device()
    plan = migemm.Plan(p.desc())
    assert plan.workspace_size == 0
    D_ref, D = run_both(p, plan)
    assert torch.equal(D.view(torch.int16), D_ref.view(torch.int16))


def test_no_alloc_rejects_a_plan_beyond_its_scratch():
    g = torch.Generator().manual_seed(712)
    p = Problem.random(g, 2048, 2048, 1024, "row", "row", dist="normal").to_device()
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE))   # one workgroup per CU
    assert plan.workspace_size > migemm.MIGEMM_NO_ALLOC_SCRATCH_BYTES
    D = p.new_d(1.0)
    st = migemm.gemm_run_no_alloc(plan.handle, p.dA, p.dB, None, D, 1.0, 0.0, check=False)
    torch.cuda.synchronize()
    assert st == migemm.MIGEMM_ERR_SCRATCH
    assert "MIGEMM_NO_ALLOC_SCRATCH_BYTES" in migemm.gemm_status_string(st)
    assert torch.all(D == 1.0), "nothing may run when the plan is rejected"
