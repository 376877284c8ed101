"""192-row tiles (GPU).

bf16 plans without the tile consumer take 192 x 256 output tiles instead of
256 x 256 where that leaves each persistent workgroup less work (ceil(T/G)
tiles, a 192-row tile being 3/4 of a 256-row one).  Checked here: the plan's
choice against that rule; the forcing flags; and that both heights give the
same D bit for bit (every output's sum runs over K in the same order, with
the same MFMA steps) and pass the oracle -- across layouts, ragged shapes, K
tails, beta, batches, a column-major D and multi-round schedules."""
import itertools

import pytest
import torch

from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full
from tests.test_batched import Batched, run

pytestmark = pytest.mark.gpu

M256, M192 = migemm.MIGEMM_F_TILE_M256, migemm.MIGEMM_F_TILE_M192
LAYOUTS = list(itertools.product(["row", "col"], ["row", "col"]))


def cdiv(a, b):
    return -(-a // b)


def plan_info(M, N, K, flags=0, mw=0, fp8=False):
    """Row-major A, B, C and D, leading strides padded to 16 bytes."""
    t = migemm.MIGEMM_FP8_E4M3 if fp8 else migemm.MIGEMM_BF16
    lk, ln = max(16, cdiv(K, 16) * 16), max(16, cdiv(N, 16) * 16)
    d = migemm.make_desc(M, N, K, t, t, lk, 1, ln, 1, ln, 1, ln, 1, flags=flags, max_workgroups=mw)
    return migemm.Plan(d).info


def expected_height(M, N, K, G):
    """The rule: 192 rows where ceil(T192 / G) * 0.8 < ceil(T256 / G) (whole tiles;
    a 192-row tile is 3/4 of the flops at a 6% lower rate)."""
    if K == 0 or M == 0 or N == 0:
        return 256
    tn = cdiv(N, 256)
    return 192 if cdiv(cdiv(M, 192) * tn, G) * 800 < cdiv(cdiv(M, 256) * tn, G) * 1000 else 256


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_plan_chooses_the_height_with_less_work_per_workgroup():
    cu = plan_info(256, 256, 64).cu_count
    shapes = [(4000, 3000, 5000), (4096, 4096, 4096), (8192, 8192, 8192), (256, 256, 256),
              (8192, 1024, 8192), (1000, 1000, 1000), (300, 300, 64), (6000, 2560, 128),
              (192, 256, 64), (193, 256, 64), (4096, 4096, 0)]
    for M, N, K in shapes:
        for mw in (0, 7, 100):
            G = min(cu, mw) if mw else cu
            i = plan_info(M, N, K, mw=mw)
            assert i.tile_m == expected_height(M, N, K, G), (M, N, K, mw, i.tile_m)
            assert i.tiles_m == cdiv(M, i.tile_m) and i.num_tiles == i.tiles_m * i.tiles_n
    if cu >= 252:
        i = plan_info(4000, 3000, 5000)   # 192 tiles of 256 rows: a quarter of the CUs idle
        assert (i.tile_m, i.tiles_m, i.tiles_n, i.num_tiles, i.grid) == (192, 21, 12, 252, 252)
    assert plan_info(8192, 8192, 8192).tile_m == 256   # 4 rounds of 256 vs 6 x 3/4
    assert plan_info(4096, 4096, 4096).tile_m == 256   # exactly one round


def test_flags_force_or_exclude_192_rows():
    assert plan_info(8192, 8192, 8192, flags=M192).tile_m == 192
    assert plan_info(8192, 8192, 8192, flags=M192).tiles_m == 43
    assert plan_info(4000, 3000, 5000, flags=M256).tile_m == 256
    # the tile consumer, stream-K forced and e4m3 stay on 256-row tiles
    assert plan_info(4000, 3000, 5000, flags=migemm.MIGEMM_F_TILE_CONSUMER).tile_m == 256
    assert plan_info(4000, 3000, 5000, flags=migemm.MIGEMM_F_STREAM_K_FORCE).tile_m == 256
    assert plan_info(4000, 3000, 5000, fp8=True).tile_m == 256
    # with MIGEMM_F_STREAM_K the plan compares all three: the ragged shape
    # takes 192-row tiles (stream-K would not pay), the one-GPU share
    # splits (its model cost is below 192-row whole tiles)
    i = plan_info(4000, 3000, 5000, flags=migemm.MIGEMM_F_STREAM_K)
    if i.cu_count >= 252:
        assert i.tile_m == 192 and i.stream_k_tiles == 0
    share = plan_info(8192, 1024, 8192, flags=migemm.MIGEMM_F_STREAM_K)
    if share.cu_count == 256:
        assert share.tile_m == 256 and share.stream_k_tiles == 128
    # a 192-row plan reads C in the epilogue
    assert plan_info(300, 300, 640, flags=M192).c_in_k_loop == 0


@pytest.mark.parametrize("la,lb", LAYOUTS)
@pytest.mark.parametrize("M,N,K,beta,mw", [
    (192, 256, 128, 0.0, 0),      # exactly one tile
    (193, 257, 64, 0.5, 0),       # one row and column past it
    (577, 1030, 264, 0.0, 0),     # ragged in both, K stages 5 (last partial)
    (1000, 900, 520, -1.0, 3),    # several tiles per workgroup
    (2000, 300, 1000, 0.0, 7),
    (95, 96, 200, 0.5, 1),        # inside the first wave's rows only
])
def test_heights_agree_bitwise(la, lb, M, N, K, beta, mw):
    g = torch.Generator().manual_seed(M * 31 + N * 7 + K)
    p = Problem.random(g, M, N, K, la, lb, dist="normal", alpha=1.25, beta=beta).to_device()
    print(f"[m192] {M}x{N}x{K} A {la} B {lb} beta {beta} grid cap {mw}", flush=True)
    plan_s = migemm.Plan(p.desc(flags=M192, max_workgroups=mw))
    plan_l = migemm.Plan(p.desc(flags=M256, max_workgroups=mw))
    assert plan_s.info.tile_m == 192 and plan_l.info.tile_m == 256
    D_s = p.run(plan_s)
    D_l = p.run(plan_l)
    torch.cuda.synchronize()
    assert same(D_s, D_l)
    r = check_full(p, D_s)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r


@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "row"), ("row", "col")])
@pytest.mark.parametrize("M,N,K", [(300, 260, 5001), (257, 129, 9), (100, 130, 7)])
def test_k_tails_with_padding_poisoned(la, lb, M, N, K):
    """K not a multiple of 8 with a K-contiguous operand (the padding past K
    is NaN, which the K loop must clear in its 6-load A stages as well)."""
    g = torch.Generator().manual_seed(K * 17 + M)
    p = Problem.random(g, M, N, K, la, lb, dist="normal").poison_padding().to_device()
    D_s = p.run(migemm.Plan(p.desc(flags=M192)))
    D_l = p.run(migemm.Plan(p.desc(flags=M256)))
    torch.cuda.synchronize()
    assert same(D_s, D_l)
    r = check_full(p, D_s)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r


@pytest.mark.parametrize("L,M,N,K,la,lb,beta,d_layout", [
    (3, 600, 500, 264, "row", "row", 0.5, "row"),
    (2, 450, 700, 136, "col", "col", 0.0, "col"),   # column-major D: D^T = B^T A^T
    (4, 200, 330, 64, "row", "col", -1.0, "row"),
])
def test_batches_and_column_major_d(L, M, N, K, la, lb, beta, d_layout):
    g = torch.Generator().manual_seed(L * 1000 + M)
    b = Batched(g, L, M, N, K, la, lb, dtype=synth.BF16, beta=beta, d_layout=d_layout)
    D_s = run(b, migemm.Plan(b.desc(flags=M192)))
    D_l = run(b, migemm.Plan(b.desc(flags=M256)))
    assert same(D_s, D_l)
    b.check(D_s)


def test_ragged_workload_full_size_agrees_with_256_rows():
    """The 4000 x 3000 x 5000 workload (checked in full against the oracle by
    the parity tests, on the plan's own choice): 192- and 256-row tiles give
    the same bits."""
    w = synth.WORKLOADS[2]
    p = Problem.from_workload(w).to_device()
    D_s = p.run(migemm.Plan(p.desc(flags=M192)))
    D_l = p.run(migemm.Plan(p.desc(flags=M256)))
    torch.cuda.synchronize()
    assert same(D_s, D_l)
