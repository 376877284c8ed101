"""Batched GEMM (GPU): L products in one launch, matrix l of each operand at
a batch stride from the first (the pages' rank-4 problem shape, L appended
to MNK).  Every batch is checked element by element against the oracle,
which computes one product at a time."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import Problem, check_full, codes

pytestmark = pytest.mark.gpu


class Batched:
    """L problems of one shape and layout, stored back to back (or sharing
    one B), with the strides of the batched description."""

    def __init__(self, gen, L, M, N, K, la="row", lb="row", dtype=synth.BF16, beta=0.0,
                 d_layout="row", share_b=False):
        alpha = 0.03125 if dtype == synth.E4M3 else 0.75
        self.ps = [Problem.random(gen, M, N, K, la, lb, dtype=dtype, dist="normal", alpha=alpha,
                                  beta=beta, d_layout=d_layout) for _ in range(L)]
        p0 = self.ps[0]
        if share_b:
            for p in self.ps[1:]:
                p.B = p0.B
        self.L, self.p0, self.share_b = L, p0, share_b
        self.A = torch.stack([p.A for p in self.ps]).cuda()
        self.B = p0.B.cuda() if share_b else torch.stack([p.B for p in self.ps]).cuda()
        self.C = torch.stack([p.C for p in self.ps]).cuda() if beta != 0.0 else None
        self.a_bs = p0.A.numel()
        self.b_bs = 0 if share_b else p0.B.numel()
        self.c_bs = self.d_bs = int(np.prod(p0.d_shape))

    def desc(self, flags=0, max_workgroups=0):
        p = self.p0
        t = migemm.MIGEMM_BF16 if p.dtype == synth.BF16 else migemm.MIGEMM_FP8_E4M3
        return migemm.make_desc(p.M, p.N, p.K, t, t, p.a_rs, p.a_cs, p.b_rs, p.b_cs, p.c_rs, p.c_cs,
                                p.d_rs, p.d_cs, flags=flags, max_workgroups=max_workgroups,
                                L=self.L, a_bs=self.a_bs, b_bs=self.b_bs, c_bs=self.c_bs,
                                d_bs=self.d_bs)

    def new_d(self):
        return torch.full((self.L, *self.p0.d_shape), float("nan"), dtype=torch.bfloat16,
                          device="cuda")

    def check(self, D):
        for l, p in enumerate(self.ps):
            r = check_full(p, D[l])
            assert r["n_fail"] == 0 and r["n_nonfinite"] == 0, (l, r)


def run(b: Batched, plan, ws=None):
    D = b.new_d()
    migemm.gemm_run(plan.handle, b.A, b.B, b.C, D, b.p0.alpha, b.p0.beta, ws)
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("L,M,N,K,la,lb,beta", [
    (3, 600, 500, 264, "row", "row", 0.5),     # ragged tiles, K tail, batched C
    (2, 256, 256, 64, "col", "col", 0.0),      # one tile per batch
    (5, 300, 770, 136, "row", "col", 0.0),     # tiles of a raster group span batches
])
def test_batched_bf16(L, M, N, K, la, lb, beta):
    g = torch.Generator().manual_seed(L * 1000 + M)
    b = Batched(g, L, M, N, K, la, lb, beta=beta)
    print(f"[batched] L={L} {M}x{N}x{K} {la}/{lb} beta={beta}", flush=True)
    plan = migemm.Plan(b.desc())
    assert plan.info.batches == L and plan.info.num_tiles == L * plan.info.tiles_m * plan.info.tiles_n
    b.check(run(b, plan))


def test_batched_shared_b_fp8():
    g = torch.Generator().manual_seed(41)
    b = Batched(g, 4, 520, 384, 256, "row", "col", dtype=synth.E4M3, share_b=True)
    print("[batched] e4m3 shared B", flush=True)
    b.check(run(b, migemm.Plan(b.desc())))


def test_batched_column_major_d():
    g = torch.Generator().manual_seed(42)
    b = Batched(g, 3, 400, 300, 200, "row", "row", beta=0.25, d_layout="col")
    print("[batched] column-major D", flush=True)
    plan = migemm.Plan(b.desc())
    assert plan.info.swapped == 1
    b.check(run(b, plan))


def test_batched_stream_k_ranges_cross_batches():
    # 3 batches x 4 tiles on 5 workgroups: unit ranges run across batch edges.
    g = torch.Generator().manual_seed(43)
    b = Batched(g, 3, 512, 512, 1000, "row", "row", beta=0.5)
    plan = migemm.Plan(b.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=5))
    assert plan.info.stream_k_tiles == 12 - 5
    ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
    migemm.gemm_workspace_init(plan.handle, ws)
    print("[batched] stream-K", flush=True)
    D1 = run(b, plan, ws)
    b.check(D1)
    D2 = run(b, plan, ws)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


@pytest.mark.parametrize("overlap", [False, True], ids=["staged", "overlap"])
def test_batched_tile_consumer(overlap):
    g = torch.Generator().manual_seed(44)
    L, M, N = 3, 520, 600
    b = Batched(g, L, M, N, 136, "row", "row")
    flags = migemm.MIGEMM_F_TILE_CONSUMER | (migemm.MIGEMM_F_CONSUMER_OVERLAP if overlap else 0)
    plan = migemm.Plan(b.desc(flags=flags, max_workgroups=4))
    ld = (N + 255) // 256
    poison = torch.full((L * M, ld), 0x7FBADBAD, dtype=torch.int32, device="cuda").view(torch.float32)
    rs, rm = poison.clone(), poison.clone()
    D, Dc = b.new_d(), b.new_d()
    print(f"[batched] tile consumer overlap={overlap}", flush=True)
    migemm.gemm_run_with_tile_consumer(plan.handle, b.A, b.B, None, D, b.p0.alpha, 0.0, rs, rm, Dc)
    torch.cuda.synchronize()
    b.check(D)
    p0 = b.p0
    for l in range(L):
        dcodes = codes(D[l]).reshape(p0.d_shape)
        assert np.array_equal(dcodes[:, :N], codes(Dc[l]).reshape(p0.d_shape)[:, :N]), l
        want_s, want_m = oracle.tile_rowstats(dcodes, M, N, p0.d_rs, p0.d_cs, 256)
        got_s = rs[l * M:(l + 1) * M].cpu().numpy()
        got_m = rm[l * M:(l + 1) * M].cpu().numpy()
        assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), l
        assert np.array_equal(got_m.view(np.uint32), want_m.view(np.uint32)), l
