"""Matrices past the 32-bit byte range (GPU).

The kernels address every operand through buffer resources whose 64-bit
base moves with the tile (and, for an MN-contiguous operand, with the K
stage), so that the 32-bit offsets inside stay small.  Each case here puts
one role beyond 4 GiB -- D and C, a K-contiguous A, an MN-contiguous A, the
batch strides -- and checks entries sampled over the whole result against
the oracle, one by one: random ones, the rows on both sides of every
2^31-byte boundary of D, the first and last rows and columns, and the
edges of the last tiles.  The tile consumer's copy and row statistics are
checked the same way (the copy bit for bit on the GPU, the statistics on
the sampled rows).  Inputs are drawn by the seeded generators of synth."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm
from tests.helpers import Problem, codes

pytestmark = pytest.mark.gpu

GiB = 1 << 30


def sample_entries(M, N, row_bytes, seed, n_random=4096):
    """(rows, cols) to check: random entries, rows around each 2^31-byte
    boundary of a row-major result whose rows are row_bytes apart, the first
    and last rows and columns, and the last tile row and column's edges."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(0, M, n_random)]
    cols = [rng.integers(0, N, n_random)]

    def add_rows(rs, per_row=64):
        for r in rs:
            if 0 <= r < M:
                rows.append(np.full(per_row, r))
                cols.append(np.concatenate([[0, N - 1], rng.integers(0, N, per_row - 2)]))

    def add_cols(cs, per_col=64):
        for c in cs:
            if 0 <= c < N:
                cols.append(np.full(per_col, c))
                rows.append(np.concatenate([[0, M - 1], rng.integers(0, M, per_col - 2)]))

    total = M * row_bytes
    for b in range(1, total // (1 << 31) + 1):
        r = (b << 31) // row_bytes
        add_rows([r - 1, r, r + 1])
    last_tm, last_tn = (M - 1) // 256 * 256, (N - 1) // 256 * 256
    add_rows([0, M - 1, last_tm - 1, last_tm])
    add_cols([0, N - 1, last_tn - 1, last_tn])
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def check_sampled(p: Problem, D: torch.Tensor, rows, cols):
    """Sampled entries of the GPU result (row-major D) against the oracle."""
    ref, absum = p.oracle_entries(rows, cols)
    idx = torch.from_numpy(rows * p.d_rs + cols).to(D.device)
    got = D.reshape(-1)[idx].cpu()
    r = oracle.check(oracle.bf16_codes_to_f64(codes(got)), ref, absum, p.in_dtype(), p.alpha)
    assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, r
    return r


def big_problem(seed, M, N, K, la, lb, beta=0.0):
    g = torch.Generator().manual_seed(seed)
    print(f"[max] drawing {M}x{N}x{K} A {la} B {lb} beta {beta}", flush=True)
    return Problem.random(g, M, N, K, la, lb, dist="uniform", beta=beta)


def test_d_and_c_beyond_4gib_with_both_consumer_schedules():
    # D and C: 65792 x 32776 bf16, 4.3 GB each (K = 64: one stage per tile).
    M, N, K = 65792, 32776, 64
    p = big_problem(301, M, N, K, "row", "row", beta=0.5).to_device()
    assert M * p.d_rs * 2 > 4 * GiB and M * p.c_rs * 2 > 4 * GiB
    rows, cols = sample_entries(M, N, p.d_rs * 2, 301)
    D = p.new_d()
    plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_M256))
    print("[max] D, C > 4 GiB: gemm_run", flush=True)
    migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta)
    torch.cuda.synchronize()
    r = check_sampled(p, D, rows, cols)
    print(f"[max] {r['n']} entries, worst {r['worst_ratio']:.3f}", flush=True)

    # 192-row tiles: D bit for bit as with 256-row ones
    print("[max] D, C > 4 GiB: gemm_run, 192-row tiles", flush=True)
    D3 = p.new_d()
    migemm.gemm_run(migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_M192)), p.dA, p.dB, p.dC, D3,
                    p.alpha, p.beta)
    torch.cuda.synchronize()
    assert torch.equal(D3.view(torch.int16), D.view(torch.int16))
    del D3

    # The tile consumer on the same problem, both schedules: D bit for bit as
    # gemm_run's, the copy bit for bit as D, the statistics of the sampled
    # rows as the oracle recomputes them from those rows of D.
    tn = -(-N // 256)
    srows = np.unique(rows[:4096])[:512]
    d_rows = D[torch.from_numpy(srows).cuda(), :N].cpu()
    want_sum, want_max = oracle.tile_rowstats(codes(d_rows), len(srows), N, N, 1)
    for flags in (migemm.MIGEMM_F_TILE_CONSUMER,
                  migemm.MIGEMM_F_TILE_CONSUMER | migemm.MIGEMM_F_CONSUMER_OVERLAP):
        print(f"[max] D, C > 4 GiB: tile consumer flags {flags:#x}", flush=True)
        pc = migemm.Plan(p.desc(flags=flags))
        D2 = p.new_d()
        Dc = torch.full_like(D2, float("nan"))
        rs = torch.full((M, tn), float("nan"), dtype=torch.float32, device="cuda")
        rm = torch.full_like(rs, float("nan"))
        migemm.gemm_run_with_tile_consumer(pc.handle, p.dA, p.dB, p.dC, D2, p.alpha, p.beta, rs,
                                           rm, Dc)
        torch.cuda.synchronize()
        assert torch.equal(D2.view(torch.int16), D.view(torch.int16))
        assert torch.equal(Dc.view(torch.int16)[:, :N], D.view(torch.int16)[:, :N])
        sel = torch.from_numpy(srows).cuda()
        got_sum = rs[sel].cpu().numpy()
        got_max = rm[sel].cpu().numpy()
        assert np.array_equal(got_sum.view(np.uint32), want_sum.view(np.uint32))
        assert np.array_equal(np.where(got_max == 0, 0, got_max), np.where(want_max == 0, 0, want_max))
        del D2, Dc, rs, rm


@pytest.mark.parametrize("tile", [migemm.MIGEMM_F_TILE_M256, migemm.MIGEMM_F_TILE_M192],
                         ids=["m256", "m192"])
def test_k_contiguous_a_beyond_4gib(tile):
    # Row-major A of 262300 x 8200 bf16 (4.3 GB): the last tile rows start
    # past 2^32 bytes; ragged M, N and a K tail of 8; both tile heights.
    M, N, K = 262300, 200, 8200
    p = big_problem(302, M, N, K, "row", "row").to_device()
    assert M * p.a_rs * 2 > 4 * GiB
    rows, cols = sample_entries(M, N, p.d_rs * 2, 302)
    # rows whose A lies past 2^31 and 2^32 bytes
    rows = np.concatenate([rows, np.arange(M - 600, M), np.full(256, (1 << 31) // (K * 2) + 1)])
    cols = np.concatenate([cols, np.arange(600) % N, np.arange(256) % N])
    D = p.new_d()
    print(f"[max] K-contiguous A > 4 GiB, tile flag {tile:#x}", flush=True)
    plan = migemm.Plan(p.desc(flags=tile))
    migemm.gemm_run(plan, p.dA, p.dB, None, D, p.alpha, 0.0)
    torch.cuda.synchronize()
    check_sampled(p, D, rows, cols)


@pytest.fixture(scope="module")
def mn_problem():
    # Column-major A of 16384 x 131200 bf16 (4.3 GB): the K stages of A step
    # 2 MiB apart, so the stage bases pass 2^32 bytes.
    M, N, K = 16384, 64, 131200
    p = big_problem(303, M, N, K, "col", "row").to_device()
    assert K * p.a_cs * 2 > 4 * GiB
    yield p
    del p.dA, p.dB


@pytest.mark.parametrize("mode", ["m256", "m192", "stream_k"])
def test_mn_contiguous_a_beyond_4gib(mn_problem, mode):
    # Whole tiles (64 of 256 rows, or 86 of 192), and stream-K cutting each
    # 256-row tile into K ranges of four workgroups whose partials meet in
    # the fixup.
    p = mn_problem
    stream_k = mode == "stream_k"
    rows, cols = sample_entries(p.M, p.N, p.d_rs * 2, 303, n_random=768)
    flags = {"m256": migemm.MIGEMM_F_TILE_M256, "m192": migemm.MIGEMM_F_TILE_M192,
             "stream_k": migemm.MIGEMM_F_STREAM_K | migemm.MIGEMM_F_STREAM_K_FORCE}[mode]
    plan = migemm.Plan(p.desc(flags=flags))
    if stream_k:
        assert plan.info.stream_k_tiles == 64
    ws = None
    if plan.workspace_size:
        ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
        migemm.gemm_workspace_init(plan.handle, ws)
    D = p.new_d()
    print(f"[max] MN-contiguous A > 4 GiB, {mode}", flush=True)
    migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, p.alpha, 0.0, ws)
    torch.cuda.synchronize()
    check_sampled(p, D, rows, cols)


def test_batch_strides_beyond_4gib():
    # Two batches whose A, C and D matrices lie 4 GiB + 4 KiB apart (B shared);
    # the storage between them is never written or read.
    L, M, N, K = 2, 520, 300, 264
    gap = (4 * GiB + 4096) // 2   # elements
    g = torch.Generator().manual_seed(304)
    ps = [Problem.random(g, M, N, K, "row", "col", dist="normal", beta=0.25) for _ in range(L)]
    for q in ps[1:]:
        q.B = ps[0].B
    print("[max] batch strides > 4 GiB", flush=True)
    dA = torch.empty(gap + ps[0].A.numel(), dtype=torch.bfloat16, device="cuda")
    dC = torch.empty(gap + ps[0].C.numel(), dtype=torch.bfloat16, device="cuda")
    d_elems = int(np.prod(ps[0].d_shape))
    dD = torch.full((gap + d_elems,), float("nan"), dtype=torch.bfloat16, device="cuda")
    for l, q in enumerate(ps):
        dA[l * gap:l * gap + q.A.numel()] = q.A.reshape(-1).cuda()
        dC[l * gap:l * gap + q.C.numel()] = q.C.reshape(-1).cuda()
    dB = ps[0].B.cuda()
    p0 = ps[0]
    desc = migemm.make_desc(M, N, K, migemm.MIGEMM_BF16, migemm.MIGEMM_BF16, p0.a_rs, p0.a_cs,
                            p0.b_rs, p0.b_cs, p0.c_rs, p0.c_cs, p0.d_rs, p0.d_cs, L=L, a_bs=gap,
                            b_bs=0, c_bs=gap, d_bs=gap)
    refs = [q.oracle_full() for q in ps]
    for tile in (migemm.MIGEMM_F_TILE_M256, migemm.MIGEMM_F_TILE_M192):
        desc.flags = tile
        plan = migemm.Plan(desc)
        dD.fill_(float("nan"))
        migemm.gemm_run(plan.handle, dA, dB, dC, dD, p0.alpha, p0.beta)
        torch.cuda.synchronize()
        for l, q in enumerate(ps):
            Dl = dD[l * gap:l * gap + d_elems].reshape(q.d_shape)
            ref, absum = refs[l]
            r = oracle.check(q.d_values(Dl), ref, absum, q.in_dtype(), q.alpha)
            assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, (tile, l, r)
