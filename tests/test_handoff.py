"""The hand-off ring's protocol, seen through its debug trace (GPU).

With MIGEMM_F_HANDOFF_DEBUG every wave records the device clock at each step
of acquire / commit / wait / release and of the consumer's copy, and the
ring's occupancy after each commit.  In the overlapped schedule the copy of a
workgroup's tile n must run inside its K loop of tile n+1 and the slot of
tile n must be released only after tile n+1 is committed, so the 2-slot ring
holds two committed tiles; in the staged schedule the copy runs between the
commit and the next K loop and the ring holds one.  The results must not
change: D, copy and statistics bit for bit as without debugging.  A bounded
wait that the host makes impossible must give up, be reported as
MIGEMM_ERR_TIMEOUT, and leave every kernel to finish normally."""
import numpy as np
import pytest
import torch

from warp_specialized_pipelined_amd import handoff_trace, migemm
from tests.helpers import Problem, check_full
from tests.test_consumer import check_consumer_outputs, poisoned

pytestmark = pytest.mark.gpu

MODES = {"staged": migemm.MIGEMM_F_TILE_CONSUMER,
         "overlapped": migemm.MIGEMM_F_TILE_CONSUMER | migemm.MIGEMM_F_CONSUMER_OVERLAP}


def run_traced(p, mode, max_workgroups, **dbg):
    plan = migemm.Plan(p.desc(flags=MODES[mode] | migemm.MIGEMM_F_HANDOFF_DEBUG,
                              max_workgroups=max_workgroups, **dbg))
    ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(plan.handle, ws)
    ld = (p.N + 255) // 256
    D, Dc = p.new_d(), p.new_d()
    rs, rm = poisoned(p.M, ld), poisoned(p.M, ld)
    migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, rs, rm,
                                       Dc, ws)
    st, info = migemm.gemm_debug_read(plan.handle, ws)
    return plan, ws, st, info, (D, Dc, rs, rm)


def problem(seed, M=1024, N=1024, K=4096):
    g = torch.Generator().manual_seed(seed)
    return Problem.random(g, M, N, K, "row", "row", dist="normal", alpha=0.5).to_device()


@pytest.mark.parametrize("mode", MODES)
def test_trace_shows_the_schedule(mode):
    # 16 tiles on 4 workgroups: 4 tiles each, K loops of 64 stages (the
    # overlapped copy needs 34 iterations).
    p = problem(900)
    print(f"[handoff] trace {mode}", flush=True)
    plan, ws, st, info, out = run_traced(p, mode, 4)
    assert st == migemm.MIGEMM_OK and info.waits_given_up == 0
    r = check_full(p, out[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    check_consumer_outputs(p, *out)
    # debugging changes no result
    plain = migemm.Plan(p.desc(flags=MODES[mode], max_workgroups=4))
    D2 = p.new_d()
    migemm.gemm_run(plain.handle, p.dA, p.dB, None, D2, p.alpha, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out[0].view(torch.int16), D2.view(torch.int16))

    rec = handoff_trace.records(ws, info)
    assert rec.shape == (4, 4, 4, 16)
    present = rec[..., 0] != 0
    assert present.all(), "every wave of every workgroup has 4 tiles"
    ids = rec[..., handoff_trace.TILE_ID]
    assert sorted(set(ids[:, 0].reshape(-1).tolist())) == list(range(16))
    assert (ids == ids[:, :1]).all(), "the waves of a workgroup agree on its tiles"
    summ = handoff_trace.summarize(rec, mode)
    print(summ, flush=True)
    ev = {e: rec[..., i].astype(np.int64) for i, e in enumerate(handoff_trace.EVENTS)}
    # every record is ordered: K loop, acquire, commit, consumer's wait
    for a, b in (("loop_begin", "loop_end"), ("loop_end", "acquired"), ("acquired", "committed"),
                 ("committed", "wait_done"), ("copy_first", "copy_last"),
                 ("copy_last", "released")):
        assert (ev[a] <= ev[b]).all(), (a, b)
    if mode == "overlapped":
        assert summ["copy_of_tile_n_inside_k_loop_of_tile_n_plus_1"] == 1.0
        assert summ["release_of_tile_n_after_commit_of_tile_n_plus_1"] == 1.0
        # at the last wave's commit of tile n+1 no wave has released tile n
        assert info.max_occupancy == 2 and summ["max_committed_unreleased_tiles"] == 2
        # the last tile of each workgroup is copied after its own commit
        assert (ev["copy_first"][..., -1] >= ev["committed"][..., -1]).all()
    else:
        assert summ["copy_of_tile_n_before_k_loop_of_tile_n_plus_1"] == 1.0
        assert (ev["released"][..., :-1] <= ev["loop_begin"][..., 1:]).all()
        assert info.max_occupancy == 1


@pytest.mark.parametrize("mode", MODES)
def test_forced_wait_gives_up_and_reports_timeout(mode):
    """Every acquire waits for one release more than can ever come; with a
    budget of 2000 ticks (20 us) each gives up, the kernel ends normally,
    gemm_debug_read says MIGEMM_ERR_TIMEOUT, and -- since program order on
    each wave already covers what acquire guards -- the results still
    match."""
    p = problem(901, 768, 768, 512)
    plan, ws, st, info, out = run_traced(p, mode, 3, debug_wait_ticks=2000, debug_force_wait=1)
    torch.cuda.synchronize()
    assert st == migemm.MIGEMM_ERR_TIMEOUT
    # 9 tiles on 3 workgroups, 4 waves each: at least one expired acquire per
    # wave and tile
    assert info.waits_given_up >= 9 * 4
    r = check_full(p, out[0])
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    check_consumer_outputs(p, *out)
    # the workspace init clears the count
    migemm.gemm_workspace_init(plan.handle, ws)
    st2, info2 = migemm.gemm_debug_read(plan.handle, ws)
    assert st2 == migemm.MIGEMM_OK and info2.waits_given_up == 0


def test_debug_plan_needs_its_workspace():
    p = problem(902, 256, 256, 64)
    plan = migemm.Plan(p.desc(flags=MODES["staged"] | migemm.MIGEMM_F_HANDOFF_DEBUG))
    assert plan.workspace_size > 0
    D = p.new_d()
    st = migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, 1.0, 0.0, None, check=False)
    assert st == migemm.MIGEMM_ERR_INVALID_ARG
