"""Seeded sweep (GPU): random valid combinations of shape, operand layouts,
element type, alpha/beta, D orientation, batch count, grid cap and mode
(whole tiles, forced stream-K, tile consumer in either schedule), each checked in full against
the oracle; the consumer's copy and statistics exactly; bf16 whole tiles
also under the other tile height (192 or 256 rows), bit for bit.  The draws are fixed
by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import oracle
from warp_specialized_pipelined_amd import migemm, synth
from tests.helpers import codes
from tests.test_batched import Batched, run

pytestmark = pytest.mark.gpu

N_CASES = 160


def draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = synth.E4M3 if rng.random() < 0.35 else synth.BF16
    la = rng.choice(["row", "col"])
    lb = rng.choice(["row", "col"])
    mode = rng.choice(["whole", "stream_k", "consumer"])
    d_layout = "col" if (mode != "consumer" and rng.random() < 0.25) else "row"
    M = int(rng.integers(1, 1100))
    N = int(rng.integers(1, 1100))
    K = int(rng.integers(0, 520))
    es = 2 if dtype == synth.BF16 else 1
    if la == "row" or lb == "col":         # a K-contiguous operand: 16-byte K rows
        K = K // (16 // es) * (16 // es)
    beta = float(rng.choice([0.0, 0.5, -1.0])) if dtype == synth.BF16 else 0.0
    L = int(rng.choice([1, 1, 2, 3]))
    mw = int(rng.choice([0, 0, 1, 3, 7, 13]))
    overlap = bool(rng.random() < 0.5)   # the consumer's schedule (drawn last: earlier draws kept)
    return dict(dtype=dtype, la=str(la), lb=str(lb), mode=str(mode), d_layout=d_layout, M=M, N=N,
                K=K, beta=beta, L=L, mw=mw, overlap=overlap)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    c = draw(i)
    print(f"[sweep] case {i}: {c}", flush=True)
    g = torch.Generator().manual_seed(2000 + i)
    b = Batched(g, c["L"], c["M"], c["N"], c["K"], c["la"], c["lb"], dtype=c["dtype"],
                beta=c["beta"], d_layout=c["d_layout"])
    p0 = b.p0
    if c["mode"] == "whole":
        plan = migemm.Plan(b.desc(max_workgroups=c["mw"]))
        D = run(b, plan)
        b.check(D)
        if c["dtype"] == synth.BF16:
            # the other tile height gives the same bits (each output's sum runs
            # over K in the same order)
            other = migemm.MIGEMM_F_TILE_M256 if plan.info.tile_m == 192 else migemm.MIGEMM_F_TILE_M192
            D2 = run(b, migemm.Plan(b.desc(flags=other, max_workgroups=c["mw"])))
            assert torch.equal(D.view(torch.int16), D2.view(torch.int16)), "tile heights differ"
    elif c["mode"] == "stream_k":
        plan = migemm.Plan(b.desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=c["mw"]))
        ws = None
        if plan.workspace_size:
            ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
            migemm.gemm_workspace_init(plan.handle, ws)
        D1 = run(b, plan, ws)
        b.check(D1)
        D2 = run(b, plan, ws)
        assert torch.equal(D1.view(torch.int16), D2.view(torch.int16)), "stream-K runs differ"
    else:
        flags = migemm.MIGEMM_F_TILE_CONSUMER | (migemm.MIGEMM_F_CONSUMER_OVERLAP if c["overlap"] else 0)
        plan = migemm.Plan(b.desc(flags=flags, max_workgroups=c["mw"]))
        L, M, N = c["L"], c["M"], c["N"]
        ld = (N + 255) // 256
        poison = torch.full((L * M, ld), 0x7FBADBAD, dtype=torch.int32, device="cuda")
        rs, rm = poison.clone().view(torch.float32), poison.clone().view(torch.float32)
        D, Dc = b.new_d(), b.new_d()
        migemm.gemm_run_with_tile_consumer(plan.handle, b.A, b.B, b.C, D, p0.alpha, p0.beta, rs, rm,
                                           Dc)
        torch.cuda.synchronize()
        b.check(D)
        for l in range(L):
            dcodes = codes(D[l]).reshape(p0.d_shape)
            assert np.array_equal(dcodes[:, :N], codes(Dc[l]).reshape(p0.d_shape)[:, :N]), l
            want_s, want_m = oracle.tile_rowstats(dcodes, M, N, p0.d_rs, p0.d_cs, 256)
            got_s = rs[l * M:(l + 1) * M].cpu().numpy()
            got_m = rm[l * M:(l + 1) * M].cpu().numpy()
            same_s = (got_s.view(np.uint32) == want_s.view(np.uint32)) | (np.isnan(got_s) & np.isnan(want_s))
            assert same_s.all(), l
            assert np.array_equal(got_m.view(np.uint32), want_m.view(np.uint32)), l
