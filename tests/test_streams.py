"""Concurrent runs (GPU).

A plan is immutable after creation, so one plan may run on several streams
at once, each run with its own outputs (and, for stream-K, its own
workspace); several host threads may call the library at once.  Every
concurrent result must equal, bit for bit, the same call made alone."""
import threading

import pytest
import torch

from warp_specialized_pipelined_amd import migemm
from tests.helpers import Problem

pytestmark = pytest.mark.gpu


def eager(fn):
    fn(torch.cuda.current_stream())
    torch.cuda.synchronize()


def same(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_one_plan_on_three_streams():
    gen = torch.Generator().manual_seed(21)
    ps = [Problem.random(gen, 1000, 900, 520, "row", "col", dist="normal", beta=0.5).to_device()
          for _ in range(3)]
    plan = migemm.Plan(ps[0].desc())          # one plan: the problems share shape and strides
    want = []
    for p in ps:
        D = p.new_d()
        eager(lambda s: migemm.gemm_run(plan, p.dA, p.dB, p.dC, D, p.alpha, p.beta, None, s))
        want.append(D)
    streams = [torch.cuda.Stream() for _ in ps]
    outs = [p.new_d() for p in ps]
    torch.cuda.synchronize()
    for rep in range(5):
        for p, D, s in zip(ps, outs, streams):
            migemm.gemm_run(plan, p.dA, p.dB, p.dC, D, p.alpha, p.beta, None, s)
        torch.cuda.synchronize()
        for D, w in zip(outs, want):
            assert same(D, w), rep


def test_stream_k_plan_on_two_streams_with_own_workspaces():
    gen = torch.Generator().manual_seed(22)
    ps = [Problem.random(gen, 700, 600, 1000, "row", "row", dist="normal").to_device()
          for _ in range(2)]
    # 9 tiles of 16 stages over 7 workgroups: ranges cross tile edges (fixups)
    plan = migemm.Plan(ps[0].desc(flags=migemm.MIGEMM_F_STREAM_K_FORCE, max_workgroups=7))
    assert plan.info.stream_k_tiles > 0
    wss = []
    for _ in ps:
        ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
        migemm.gemm_workspace_init(plan, ws)
        wss.append(ws)
    want = []
    for p, ws in zip(ps, wss):
        D = p.new_d()
        eager(lambda s: migemm.gemm_run(plan, p.dA, p.dB, None, D, p.alpha, 0.0, ws, s))
        want.append(D)
    streams = [torch.cuda.Stream() for _ in ps]
    outs = [p.new_d() for p in ps]
    torch.cuda.synchronize()
    for rep in range(5):
        for p, D, ws, s in zip(ps, outs, wss, streams):
            migemm.gemm_run(plan, p.dA, p.dB, None, D, p.alpha, 0.0, ws, s)
        torch.cuda.synchronize()
        for D, w in zip(outs, want):
            assert same(D, w), rep


def test_tile_consumer_plan_on_two_streams():
    gen = torch.Generator().manual_seed(23)
    ps = [Problem.random(gen, 768, 1000, 264, "row", "row", dist="normal").to_device()
          for _ in range(2)]
    plan = migemm.Plan(ps[0].desc(flags=migemm.MIGEMM_F_TILE_CONSUMER, max_workgroups=5))
    ld = (ps[0].N + 255) // 256

    def outputs(p):
        D, Dc = p.new_d(), p.new_d()
        rs = torch.full((p.M, ld), float("nan"), dtype=torch.float32, device="cuda")
        return [D, Dc, rs, torch.full_like(rs, float("nan"))]

    def run(p, o, s):
        migemm.gemm_run_with_tile_consumer(plan, p.dA, p.dB, None, o[0], p.alpha, 0.0, o[2], o[3],
                                           o[1], None, s)

    want = []
    for p in ps:
        o = outputs(p)
        eager(lambda s: run(p, o, s))
        want.append(o)
    streams = [torch.cuda.Stream() for _ in ps]
    outs = [outputs(p) for p in ps]
    torch.cuda.synchronize()
    for rep in range(3):
        for p, o, s in zip(ps, outs, streams):
            run(p, o, s)
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert all(same(a, b) for a, b in zip(o, w)), rep


def test_host_threads_calling_at_once():
    # Four threads, each with its own stream and outputs, each launching 20
    # runs of the same plan, while the main thread creates and destroys
    # other plans (the library's set of live plans is shared).
    gen = torch.Generator().manual_seed(24)
    p = Problem.random(gen, 512, 768, 256, "row", "row", dist="normal").to_device()
    plan = migemm.Plan(p.desc())
    want = p.new_d()
    eager(lambda s: migemm.gemm_run(plan, p.dA, p.dB, None, want, p.alpha, 0.0, None, s))
    outs = [p.new_d() for _ in range(4)]
    errors = []

    def worker(D):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    migemm.gemm_run(plan, p.dA, p.dB, None, D, p.alpha, 0.0, None, s)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(D,)) for D in outs]
    for t in threads:
        t.start()
    for _ in range(50):
        migemm.Plan(p.desc(max_workgroups=3))   # created and destroyed meanwhile
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for D in outs:
        assert same(D, want)
