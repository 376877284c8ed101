"""HIP graph capture (GPU).

The library enqueues kernels only (no memset, no allocation, no
synchronization), so its calls can be captured in a HIP graph and replayed.
Each test captures a call once, replays it several times with the program's
own eager work and synchronizations in between, and checks every replay bit
for bit against the same call made eagerly."""
import pytest
import torch

from warp_specialized_pipelined_amd import migemm
from tests.helpers import Problem

pytestmark = pytest.mark.gpu

REPLAYS = 4


def capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(s)  # warm-up outside the graph on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, want, scribble):
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scribble()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.int32) if o.dtype == torch.float32 else o.view(torch.int16),
                               w.view(torch.int32) if w.dtype == torch.float32 else w.view(torch.int16)), i


def test_graph_plain_and_stream_k():
    gen = torch.Generator().manual_seed(11)
    p = Problem.random(gen, 1000, 700, 520, "row", "row", dist="normal", beta=0.5).to_device()
    plan = migemm.Plan(p.desc())                                     # 192-row tiles
    plan_l = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_M256))   # C read in the K loop
    assert plan.info.tile_m == 192 and plan_l.info.c_in_k_loop == 1
    sk = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=6))
    ws = torch.empty(sk.workspace_size, dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(sk.handle, ws)
    D1, D2, D3 = p.new_d(), p.new_d(), p.new_d()
    junk = torch.empty(1 << 20, device="cuda")

    def calls(stream):
        migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D1, p.alpha, p.beta, None, stream)
        migemm.gemm_run(sk.handle, p.dA, p.dB, p.dC, D2, p.alpha, p.beta, ws, stream)
        migemm.gemm_run(plan_l.handle, p.dA, p.dB, p.dC, D3, p.alpha, p.beta, None, stream)

    calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [D1.clone(), D2.clone(), D3.clone()]
    assert torch.equal(want[0].view(torch.int16), want[2].view(torch.int16))
    g = capture(calls)
    replay_and_check(g, [D1, D2, D3], want, lambda: junk.uniform_())


@pytest.mark.parametrize("overlap", [False, True], ids=["staged", "overlap"])
def test_graph_tile_consumer(overlap):
    gen = torch.Generator().manual_seed(12)
    p = Problem.random(gen, 768, 1000, 264, "row", "row", dist="normal").to_device()
    flags = migemm.MIGEMM_F_TILE_CONSUMER | (migemm.MIGEMM_F_CONSUMER_OVERLAP if overlap else 0)
    plan = migemm.Plan(p.desc(flags=flags, max_workgroups=3))
    ld = (p.N + 255) // 256
    D, Dc = p.new_d(), p.new_d()
    rs = torch.empty((p.M, ld), dtype=torch.float32, device="cuda")
    rm = torch.empty_like(rs)

    def call(stream):
        migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, None, D, p.alpha, 0.0, rs, rm,
                                           Dc, None, stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [D.clone(), Dc.clone(), rs.clone(), rm.clone()]
    g = capture(call)
    replay_and_check(g, [D, Dc, rs, rm], want, lambda: torch.cuda.synchronize())


def test_graph_no_alloc_stream_k():
    # gemm_run_no_alloc is for callers that cannot allocate, such as code under
    # graph capture: a stream-K plan takes its workspace from the library's
    # fixed scratch, and the captured call clears the scratch's counters with
    # a fill kernel of its own.  Between replays another plan's eager
    # no-allocation run reuses that scratch; every replay must still give the
    # eager result.
    gen = torch.Generator().manual_seed(13)
    p = Problem.random(gen, 1000, 700, 520, "row", "row", dist="normal", beta=0.5).to_device()
    q = Problem.random(gen, 600, 520, 300, "row", "col", dist="normal").to_device()
    sk = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=6))
    sk_other = migemm.Plan(q.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=5))
    assert sk.info.stream_k_tiles > 0 and sk_other.info.stream_k_tiles > 0
    D, Dq = p.new_d(), q.new_d()

    def call(stream):
        migemm.gemm_run_no_alloc(sk, p.dA, p.dB, p.dC, D, p.alpha, p.beta, stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [D.clone()]
    g = capture(call)

    def other_run():
        migemm.gemm_run_no_alloc(sk_other, q.dA, q.dB, None, Dq, q.alpha, 0.0)
        torch.cuda.synchronize()

    replay_and_check(g, [D], want, other_run)
