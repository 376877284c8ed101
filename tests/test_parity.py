"""Parity of the HIP GEMM with the CPU oracle, element by element, through
the C ABI (GPU).

Every output element is checked, the five full-size workloads included (the
largest, 8192 x 8192 x 16384 e4m3, is 2.2e12 flops of fp64 oracle work).  The
bar is the per-element acceptance rule held by the oracle package."""
import itertools

import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full, codes, workload_reference

pytestmark = pytest.mark.gpu

LAYOUTS = list(itertools.product(["row", "col"], ["row", "col"]))
# bf16 plans without the consumer take 256- or 192-row tiles (the plan
# chooses; these flags force one).
TILES = {"m256": migemm.MIGEMM_F_TILE_M256, "m192": migemm.MIGEMM_F_TILE_M192}


def plan_for(p: Problem, **kw):
    return migemm.Plan(p.desc(**kw))


def ok(r):
    return r["n_fail"] == 0 and r["n_nonfinite"] == 0


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------- full workloads

@pytest.mark.parametrize("w", synth.WORKLOADS, ids=lambda w: w.name)
def test_workload(w):
    """The workload through gemm_run, every element against the oracle (the
    8192^3 one's tile-consumer variant has tests of its own)."""
    print(f"[parity] workload {w.name}", flush=True)
    p = Problem.from_workload(w).to_device()
    plan = plan_for(p)
    D = p.run(plan)
    torch.cuda.synchronize()
    r = check_full(p, D, workload_reference(w, p))
    print(f"[parity] {w.name}: {r['n']} elements, {r['n_fail']} outside the bound, "
          f"worst |D-ref|/bound {r['worst_ratio']:.4f} at flat index {r['worst_index']}", flush=True)
    assert r["n"] == w.M * w.N
    assert ok(r), r


# --------------------------------------------------------------- shape sweep

SHAPES_K_ALIGNED = [(1, 1, 8), (17, 33, 8), (64, 64, 64), (255, 257, 136), (256, 256, 256),
                    (257, 255, 264), (300, 520, 520), (513, 129, 1000)]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES_K_ALIGNED)
def test_shapes_bf16(la, lb, M, N, K, tile):
    g = torch.Generator().manual_seed(M * 7919 + N * 31 + K)
    p = Problem.random(g, M, N, K, la, lb, dist="normal").to_device()
    plan = plan_for(p, flags=TILES[tile])
    assert plan.info.tile_m == int(tile[1:])
    D = p.run(plan)
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert ok(r), (la, lb, M, N, K, r)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (15, 17, 17), (100, 300, 255), (257, 129, 63),
                                   (450, 200, 130)])
def test_shapes_any_k_mn_contiguous(M, N, K, tile):
    """A column-major and B row-major: K needs no alignment."""
    g = torch.Generator().manual_seed(K)
    p = Problem.random(g, M, N, K, "col", "row", dist="normal").to_device()
    D = p.run(plan_for(p, flags=TILES[tile]))
    torch.cuda.synchronize()
    assert ok(check_full(p, D))


K_TAIL_LAYOUTS = [("row", "col"), ("row", "row"), ("col", "col")]   # a K-contiguous operand


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("la,lb", K_TAIL_LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(64, 64, 1), (100, 130, 7), (257, 129, 9), (300, 260, 5001),
                                   (520, 264, 71)])
def test_any_k_with_k_contiguous_operands(la, lb, M, N, K, tile):
    """K not a multiple of 8: the last 16-byte chunk of a K-contiguous row
    holds padding past K (NaN here), which the K loop must clear."""
    g = torch.Generator().manual_seed(K * 131 + M)
    p = Problem.random(g, M, N, K, la, lb, dist="normal").poison_padding().to_device()
    print(f"[parity] any K {M}x{N}x{K} A {la} B {lb} tile {tile}", flush=True)
    D = p.run(plan_for(p, flags=TILES[tile]))
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert ok(r), (la, lb, M, N, K, r)


@pytest.mark.parametrize("la,lb", K_TAIL_LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(64, 64, 1), (130, 200, 15), (257, 129, 17), (300, 260, 1001)])
def test_any_k_with_k_contiguous_operands_fp8(la, lb, M, N, K):
    g = torch.Generator().manual_seed(K * 17 + N)
    p = Problem.random(g, M, N, K, la, lb, dtype=synth.E4M3, alpha=0.0625).poison_padding()
    p.to_device()
    print(f"[parity] any K e4m3 {M}x{N}x{K} A {la} B {lb}", flush=True)
    D = p.run(plan_for(p))
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert ok(r), (la, lb, M, N, K, r)


def test_any_k_stream_k():
    """The K tail in the last stream-K range of each tile."""
    g = torch.Generator().manual_seed(5001)
    p = Problem.random(g, 512, 512, 5001, "row", "col", dist="normal", alpha=0.5,
                       beta=0.25).poison_padding().to_device()
    plan = plan_for(p, flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=7)
    assert plan.info.stream_k_tiles > 0
    ws = torch.empty(max(plan.workspace_size, 256), dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(plan.handle, ws)
    D = p.new_d()
    migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, ws)
    torch.cuda.synchronize()
    assert ok(check_full(p, D))


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (257, 300, 192), (128, 384, 1040)])
def test_shapes_fp8(la, lb, M, N, K):
    g = torch.Generator().manual_seed(M + N + K)
    p = Problem.random(g, M, N, K, la, lb, dtype=synth.E4M3, alpha=0.0625).to_device()
    D = p.run(plan_for(p))
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert ok(r), (la, lb, M, N, K, r)


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.5), (-0.5, 1.0), (0.125, -2.0), (0.0, 1.0)])
def test_alpha_beta(alpha, beta):
    g = torch.Generator().manual_seed(99)
    p = Problem.random(g, 300, 280, 264, "row", "col", dist="normal", alpha=alpha, beta=beta)
    p.to_device()
    D = p.run(plan_for(p))
    torch.cuda.synchronize()
    assert ok(check_full(p, D))


@pytest.mark.parametrize("M,N,K,la,lb", [
    (300, 280, 264, "row", "col"),     # ragged tiles, K stages 5 (last ragged)
    (1000, 1200, 520, "row", "row"),   # several tiles per workgroup
    (512, 512, 64, "col", "row"),      # one K stage: C is read in the epilogue
    (512, 384, 72, "row", "col"),      # two K stages, the second ragged
    (640, 520, 2048, "col", "col"),
])
def test_c_read_schedules_agree(M, N, K, la, lb):
    """beta != 0: C loaded in the K loop's last two iterations (the default
    of 256-row tiles) or in the epilogue (MIGEMM_F_C_IN_EPILOGUE, and 192-row
    tiles) -- the same D bit for bit, and within the bound."""
    g = torch.Generator().manual_seed(M + K)
    p = Problem.random(g, M, N, K, la, lb, dist="normal", alpha=0.75, beta=-0.5).to_device()
    m256 = migemm.MIGEMM_F_TILE_M256
    plan = plan_for(p, flags=m256)
    plan_e = plan_for(p, flags=m256 | migemm.MIGEMM_F_C_IN_EPILOGUE)
    plan_s = plan_for(p, flags=migemm.MIGEMM_F_TILE_M192)
    assert plan.info.c_in_k_loop == int(plan.info.num_tiles <= plan.info.grid and K > 64)
    assert plan_e.info.c_in_k_loop == 0 and plan_s.info.c_in_k_loop == 0
    D1 = p.run(plan)
    D2 = p.run(plan_e)
    D3 = p.run(plan_s)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    assert torch.equal(D1.view(torch.int16), D3.view(torch.int16))
    assert ok(check_full(p, D1))


def test_column_major_d_and_c():
    g = torch.Generator().manual_seed(5)
    p = Problem.random(g, 300, 200, 136, "row", "row", dist="normal", alpha=1.0, beta=0.75,
                       d_layout="col").to_device()
    plan = plan_for(p)
    assert plan.info.swapped == 1
    D = p.run(plan)
    torch.cuda.synchronize()
    assert ok(check_full(p, D))


# ------------------------------------------------------ semantics and edges

def test_beta_zero_ignores_c_even_nan():
    g = torch.Generator().manual_seed(6)
    p = Problem.random(g, 256, 256, 128, dist="normal").to_device()
    plan = plan_for(p)
    D1 = p.run(plan, C_override=None)
    nanC = torch.full((256, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    D2 = p.run(plan, C_override=nanC)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    assert ok(check_full(p, D1))


def test_k_zero_gives_beta_c():
    g = torch.Generator().manual_seed(1)
    p = Problem.random(g, 260, 130, 0, "row", "row", alpha=1.0, beta=2.0).to_device()
    D = p.run(plan_for(p))
    torch.cuda.synchronize()
    assert ok(check_full(p, D))
    want = (2.0 * p.C[:, :130].to(torch.float32)).to(torch.bfloat16)   # doubling is exact
    assert torch.equal(D.cpu()[:, :130].view(torch.int16), want.view(torch.int16))


def test_empty_output_is_a_no_op():
    for M, N in [(0, 64), (64, 0)]:
        desc = migemm.make_desc(M, N, 64, 1, 1, 64, 1, max(N, 8), 1, max(N, 8), 1, max(N, 8), 1)
        plan = migemm.Plan(desc)
        assert migemm.gemm_run(plan.handle, 0, 0, 0, 0, 1.0, 0.0) == migemm.MIGEMM_OK


def test_exact_small_integer_results():
    """All-ones gives K exactly; A = I gives B bit for bit; entries in
    {-1, 0, 1} with K <= 256 give exact integers."""
    K = 4096
    A = torch.ones((256, K), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((K, 256), dtype=torch.bfloat16, device="cuda")
    D = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    plan = migemm.Plan(migemm.make_desc(256, 256, K, 1, 1, K, 1, 256, 1, 256, 1, 256, 1))
    migemm.gemm_run(plan.handle, A, B, None, D, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.all(D.float() == K)

    g = torch.Generator().manual_seed(3)
    Bm = torch.randn((512, 384), generator=g).to(torch.bfloat16)
    I = torch.eye(512, dtype=torch.bfloat16)
    D = torch.empty((512, 384), dtype=torch.bfloat16, device="cuda")
    plan = migemm.Plan(migemm.make_desc(512, 384, 512, 1, 1, 512, 1, 384, 1, 384, 1, 384, 1))
    migemm.gemm_run(plan.handle, I.cuda(), Bm.cuda(), None, D, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(D.cpu().view(torch.int16), Bm.view(torch.int16))

    Ai = synth.small_int_matrix(g, (300, 256))
    Bi = synth.small_int_matrix(g, (256, 200))
    exact = Ai.to(torch.float64) @ Bi.to(torch.float64)
    D = torch.empty((300, 200), dtype=torch.bfloat16, device="cuda")
    plan = migemm.Plan(migemm.make_desc(300, 200, 256, 1, 1, 256, 1, 200, 1, 200, 1, 200, 1))
    migemm.gemm_run(plan.handle, Ai.cuda(), Bi.cuda(), None, D, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(D.cpu().to(torch.float64), exact)


def test_deterministic_across_runs_and_grid_sizes():
    g = torch.Generator().manual_seed(12)
    p = Problem.random(g, 1000, 1200, 520, "row", "row", dist="normal").to_device()
    outs = []
    for mw in (0, 0, 7, 64):
        outs.append(p.run(plan_for(p, max_workgroups=mw)))
    torch.cuda.synchronize()
    for D in outs[1:]:
        assert torch.equal(D.view(torch.int16), outs[0].view(torch.int16))
    assert ok(check_full(p, outs[0]))


def test_plan_info_matches_the_persistent_design():
    g = torch.Generator().manual_seed(1)
    p = Problem.random(g, 4000, 3000, 64)
    info = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_M256)).info
    assert (info.tiles_m, info.tiles_n, info.num_tiles) == (16, 12, 192)
    assert info.grid == min(192, info.cu_count)
    assert info.block_threads == 256 and info.tile_m == 256 and info.tile_n == 256
    # 192 tiles leave a quarter of 256 compute units idle; 192-row tiles fill them
    short = migemm.Plan(p.desc()).info
    if info.cu_count >= 252:
        assert (short.tile_m, short.tiles_m, short.num_tiles, short.grid) == (192, 21, 252, 252)
    assert info.lds_bytes <= 160 * 1024
    props = torch.cuda.get_device_properties(0)
    assert info.cu_count == props.multi_processor_count
    assert "gfx950" in props.gcnArchName


def test_destroyed_plan_is_rejected_before_launch():
    # A plan handle outlives its Plan object when it is taken from a
    # temporary (gemm_run(Plan(d).handle, ...)): the C plan is destroyed
    # before the call starts.  The library must refuse it, not launch with
    # arguments read from freed memory; D stays as it was.
    p = Problem.random(torch.Generator().manual_seed(61), 256, 256, 64).to_device()
    D = p.new_d()
    with pytest.raises(migemm.MigemmError) as e:
        migemm.gemm_run(migemm.Plan(p.desc()).handle, p.dA, p.dB, None, D, 1.0, 0.0)
    assert e.value.status == migemm.MIGEMM_ERR_INVALID_ARG
    plan = migemm.Plan(p.desc())
    h = plan.handle
    assert migemm.gemm_plan_destroy(h) == migemm.MIGEMM_OK
    assert migemm.gemm_plan_destroy(h) == migemm.MIGEMM_ERR_INVALID_ARG   # not twice
    assert migemm.gemm_run(h, p.dA, p.dB, None, D, 1.0, 0.0, check=False) == migemm.MIGEMM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.isnan(D.float()).all()
    plan.handle = None
    # A Plan object passed itself stays alive for the call.
    migemm.gemm_run(migemm.Plan(p.desc()), p.dA, p.dB, None, D, 1.0, 0.0)
    torch.cuda.synchronize()
    r = check_full(p, D)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r


def test_misaligned_pointer_is_rejected_before_launch():
    g = torch.Generator().manual_seed(2)
    p = Problem.random(g, 64, 64, 64).to_device()
    plan = plan_for(p)
    D = p.new_d()
    base = torch.empty(64 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    st = migemm.gemm_run(plan.handle, base[1:].data_ptr(), p.dB, None, D, 1.0, 0.0, check=False)
    assert st == migemm.MIGEMM_ERR_MISALIGNED
    st = migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, 1.0, 0.5, check=False)
    assert st == migemm.MIGEMM_ERR_INVALID_ARG   # beta != 0 needs C
