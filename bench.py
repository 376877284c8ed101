#!/usr/bin/env python3
"""Throughput of the persistent pipelined GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one call of the whole hot path on the 8192^3 bf16 workload (entries
N(0,1)/sqrt(K), row-major A and B, bf16 D) with the tile hand-off consumer
(row sum/max + tile copy per finished 256 x 256 tile) when the library has it.
Inputs are seeded, synthetic and resident in HBM before timing starts.  The
script prints ONE JSON line on stdout; diagnostics go to stderr.

The roofline object prices the GEMM kernel against MI355X's dense bf16 MFMA
peak (2.5166 PFLOP/s = 256 CUs x 2.4 GHz x 4096 flop/clk/CU), using the
algorithmic 2*M*N*K flops per launch over the kernel's mean duration measured
with HIP events on the launch stream.  The CPU baseline times the oracle (the
plain fp64 CPU GEMM) on a bounded slice of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # 2516.6
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS           # 5033.2
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(HERE, "profiles", "traffic_gemm_consumer_bf16_8192.txt")


def kernel_source_hash() -> str:
    """sha1 over the device-side sources (the kernel translation unit and its
    headers), in a fixed order: identifies the kernel whose counters a
    traffic profile holds."""
    import hashlib
    csrc = os.path.join(HERE, "warp_specialized_pipelined_amd", "csrc")
    files = [os.path.join(csrc, "gemm_kernels.hip"), os.path.join(csrc, "launch.h")]
    kdir = os.path.join(csrc, "kernel")
    files += [os.path.join(kdir, f) for f in sorted(os.listdir(kdir)) if f.endswith(".hpp")]
    h = hashlib.sha1()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter profile, or None if there is none or the kernel has
    changed since it was taken."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha1") != kernel_source_hash():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first: a fresh process needs ~30 to reach steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the plain/fp8 side measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-baseline duration")
    ap.add_argument("--variant", choices=["full", "consumer", "plain", "fp8", "copy"], default="full",
                    help="profiling runs: time one kernel only and print a short line "
                         "(copy = a plain 128 MiB device copy, the byte-counter calibration)")
    return ap.parse_args()


def run_variant(args):
    """One kernel, timed alone (for rocprofv3 counter passes)."""
    import torch
    from warp_specialized_pipelined_amd import migemm, synth
    from tests.helpers import Problem
    stream = torch.cuda.current_stream()
    if args.variant == "copy":
        n = 64 * 1024 * 1024                       # 128 MiB of bf16 read + 128 MiB written
        src = torch.randn(n, device="cuda").to(torch.bfloat16)
        dst = torch.empty_like(src)
        ms = time_calls(lambda: dst.copy_(src), args.steps, args.warmup, stream)
        print(json.dumps({"variant": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                          "ms": round(ms, 4), "GB/s": round(4 * n / (ms * 1e-3) / 1e9, 1)}))
        return
    w = synth.WORKLOADS[4] if args.variant == "fp8" else synth.WORKLOADS[3]
    p = Problem.from_workload(w).to_device()
    D = p.new_d(0.0)
    if args.variant == "consumer":
        plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER))
        ld = (w.N + 255) // 256
        rs = torch.empty((w.M, ld), dtype=torch.float32, device="cuda")
        rm = torch.empty_like(rs)
        Dc = torch.empty_like(D)
        fn = lambda: migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, None, D, p.alpha,
                                                        0.0, rs, rm, Dc, None, stream)
    else:
        plan = migemm.Plan(p.desc())
        fn = lambda: migemm.gemm_run(plan.handle, p.dA, p.dB, None, D, p.alpha, 0.0, None, stream)
    ms = time_calls(fn, args.steps, args.warmup, stream)
    print(json.dumps({"variant": args.variant, "workload": w.name, "ms": round(ms, 4),
                      "TFLOP/s": round(w.flops / (ms * 1e-3) / 1e12, 1)}))


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms per call


def sysfs_gpu_dir():
    """The sysfs directory of GPU 0 (by its PCI address when torch reports
    one, else the only amdgpu card present), or None."""
    import glob
    import torch
    prop = torch.cuda.get_device_properties(0)
    bus = getattr(prop, "pci_bus_id", None)
    if bus is not None:
        d = f"/sys/bus/pci/devices/{getattr(prop, 'pci_domain_id', 0):04x}:{bus:02x}:" \
            f"{getattr(prop, 'pci_device_id', 0):02x}.0"
        if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
            return d
    cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return os.path.dirname(cards[0]) if len(cards) == 1 else None


def read_sclk_mhz(path):
    """Current shader clock from amdgpu's pp_dpm_sclk: the level marked '*'."""
    with open(path) as f:
        for line in f:
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().split("M")[0])
    return None


def observe_clock(step, stream, ms_per_step, seconds=1.5, period=0.01):
    """Run `step` back to back for about `seconds` while a thread samples the
    shader clock (and the board power, where hwmon reports it) every
    `period` s.  Returns the median clock, the throughput of that run and
    the sample counts; None where the driver exposes nothing."""
    import glob
    import statistics
    import threading
    import torch
    d = sysfs_gpu_dir()
    if d is None:
        return None
    sclk_path = os.path.join(d, "pp_dpm_sclk")
    pw = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_average")) +
                glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input")))
    clocks, watts, stop = [], [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                c = read_sclk_mhz(sclk_path)
                if c is not None:
                    clocks.append(c)
                if pw:
                    with open(pw[0]) as f:
                        watts.append(int(f.read()) / 1e6)
            except (OSError, ValueError, IndexError):
                pass
            time.sleep(period)

    n = max(10, int(seconds * 1e3 / ms_per_step))
    torch.cuda.synchronize()
    t = threading.Thread(target=sample, daemon=True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(n):
        step()
        if i == n // 10:
            t.start()               # sample once the run is under way
    end.record(stream)
    torch.cuda.synchronize()
    stop.set()
    t.join()
    if not clocks:
        return None
    return {"sclk_mhz": statistics.median(clocks), "sclk_samples": len(clocks),
            "watts": statistics.median(watts) if watts else None,
            "ms": start.elapsed_time(end) / n, "steps": n}


def cpu_baseline(p, target_s):
    """Time the oracle on the first R rows of the workload (all N columns,
    full K), R chosen so the run takes about target_s seconds."""
    import oracle
    from tests.helpers import oracle_operand
    Aop = oracle_operand(p.A, p.a_rs, p.a_cs)
    Bop = oracle_operand(p.B, p.b_rs, p.b_cs)
    threads = oracle.max_threads()

    def run(rows):
        t0 = time.perf_counter()
        oracle.gemm(rows, p.N, p.K, Aop, Bop, None, p.alpha, 0.0)
        return time.perf_counter() - t0

    probe_rows = min(p.M, max(16, 4 * threads))   # rows are split over the threads
    t = run(probe_rows)
    rows = int(min(p.M, max(probe_rows, probe_rows * target_s / max(t, 1e-3))))
    rows = max(threads, rows // threads * threads)
    t = run(rows)
    flops = 2.0 * rows * p.N * p.K
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} rows of the {p.M}x{p.N}x{p.K} product (all columns, full K), "
                  f"fp64 accumulation, {t:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from warp_specialized_pipelined_amd import migemm, synth
    from tests.helpers import Problem

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    if args.variant != "full":
        run_variant(args)
        return
    stream = torch.cuda.current_stream()
    dev = torch.cuda.get_device_properties(0)
    log(f"[bench] device {dev.name} {dev.gcnArchName} cus={dev.multi_processor_count}")

    w = synth.WORKLOADS[3]                      # 8192^3 bf16, tile consumer
    log(f"[bench] drawing inputs for {w.name}")
    p = Problem.from_workload(w).to_device()
    D = p.new_d(0.0)
    plan_plain = migemm.Plan(p.desc())
    consumer = False
    try:
        plan_cons = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER))
        stat_ld = (w.N + 255) // 256
        row_sum = torch.empty((w.M, stat_ld), dtype=torch.float32, device="cuda")
        row_max = torch.empty((w.M, stat_ld), dtype=torch.float32, device="cuda")
        D_copy = torch.empty_like(D)
        st = migemm.gemm_run_with_tile_consumer(plan_cons.handle, p.dA, p.dB, None, D, p.alpha, 0.0,
                                                row_sum, row_max, D_copy, check=False)
        torch.cuda.synchronize()
        consumer = st == migemm.MIGEMM_OK
        if not consumer:
            log(f"[bench] tile consumer unavailable: {migemm.gemm_status_string(st)}")
    except migemm.MigemmError as e:
        log(f"[bench] tile consumer plan failed: {e}")

    def step_plain():
        migemm.gemm_run(plan_plain.handle, p.dA, p.dB, None, D, p.alpha, 0.0, None, stream)

    def step_cons():
        migemm.gemm_run_with_tile_consumer(plan_cons.handle, p.dA, p.dB, None, D, p.alpha, 0.0,
                                           row_sum, row_max, D_copy, None, stream)

    step = step_cons if consumer else step_plain
    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up (consumer={consumer})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_calls(step, args.steps, args.warmup, stream)
    wall = time.perf_counter() - t0
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step  {tflops:.1f} TFLOP/s  ({wall:.1f} s wall)")

    extra = {"consumer_variant": consumer}

    def clock_extras(prefix, fn, ms_step, flops, flop_per_clk_cu):
        """The shader clock under this load (amdgpu's DPM readout), the board
        power, and the throughput as a fraction of the MFMA peak at that
        clock: context for the nominal fraction, which prices every cycle at
        2.4 GHz."""
        clk = observe_clock(fn, stream, ms_step)
        log(f"[bench] clock run {prefix}: {clk}")
        if clk is None:
            return
        t_clk = flops / (clk["ms"] * 1e-3) / 1e12
        extra[prefix + "sclk_mhz_median"] = clk["sclk_mhz"]
        extra[prefix + "tflops_during_clock_run"] = round(t_clk, 1)
        extra[prefix + "frac_of_peak_at_observed_sclk"] = round(
            t_clk / (256 * clk["sclk_mhz"] * 1e6 * flop_per_clk_cu / 1e12), 4)
        if clk["watts"] is not None:
            extra[prefix + "board_power_w_median"] = round(clk["watts"], 1)

    clock_extras("", step, ms, w.flops, 4096)
    if not args.no_extra:
        ms_plain = time_calls(step_plain, args.steps, max(2, args.warmup // 2), stream)
        extra["plain_gemm_ms"] = round(ms_plain, 4)
        extra["plain_gemm_tflops"] = round(w.flops / (ms_plain * 1e-3) / 1e12, 1)
        extra["plain_gemm_frac_of_peak"] = round(extra["plain_gemm_tflops"] / PEAK_BF16_TFLOPS, 4)
        if consumer:
            extra["consumer_over_plain_time"] = round(ms / ms_plain, 4)
            clock_extras("plain_gemm_", step_plain, ms_plain, w.flops, 4096)
            # The other schedule of the consumer stage: inside the next
            # tile's K loop, on the tile fetched back from D.
            plan_ov = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER |
                                         migemm.MIGEMM_F_CONSUMER_OVERLAP))
            ms_ov = time_calls(lambda: migemm.gemm_run_with_tile_consumer(
                plan_ov.handle, p.dA, p.dB, None, D, p.alpha, 0.0, row_sum, row_max, D_copy, None,
                stream), args.steps, max(2, args.warmup // 2), stream)
            extra["consumer_overlapped_tflops"] = round(w.flops / (ms_ov * 1e-3) / 1e12, 1)
            extra["consumer_overlapped_over_plain_time"] = round(ms_ov / ms_plain, 4)
        # The vendor library on the same inputs, for reference only: torch's
        # bf16 matmul (hipBLASLt) of the same row-major A and B, contiguous.
        if p.a_rs == w.K and p.b_rs == w.N and p.a_cs == 1 and p.b_cs == 1:
            A2 = p.dA.view(w.M, w.K)
            B2 = p.dB.view(w.K, w.N)
            out2 = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
            ms_lib = time_calls(lambda: torch.matmul(A2, B2, out=out2), max(10, args.steps // 2),
                                max(5, args.warmup // 2), stream)
            extra["library_gemm_tflops"] = round(w.flops / (ms_lib * 1e-3) / 1e12, 1)
            extra["library_gemm"] = "torch.matmul bf16 (hipBLASLt), same A and B, no consumer"
            clock_extras("library_gemm_", lambda: torch.matmul(A2, B2, out=out2), ms_lib, w.flops,
                         4096)
            del out2
        # fp8 e4m3 8192 x 8192 x 16384
        w8 = synth.WORKLOADS[4]
        log(f"[bench] drawing inputs for {w8.name}")
        p8 = Problem.from_workload(w8).to_device()
        D8 = p8.new_d(0.0)
        plan8 = migemm.Plan(p8.desc())

        def step8():
            migemm.gemm_run(plan8.handle, p8.dA, p8.dB, None, D8, p8.alpha, 0.0, None, stream)

        ms8 = time_calls(step8, max(5, args.steps // 2), max(2, args.warmup // 2), stream)
        extra["fp8_gemm_ms"] = round(ms8, 4)
        extra["fp8_gemm_tflops"] = round(w8.flops / (ms8 * 1e-3) / 1e12, 1)
        extra["fp8_gemm_frac_of_peak"] = round(extra["fp8_gemm_tflops"] / PEAK_FP8_TFLOPS, 4)
        clock_extras("fp8_gemm_", step8, ms8, w8.flops, 8192)
        del p8, D8
        # One GPU's share of an 8-way split of N, 8192 x 1024 x 8192 bf16: 128
        # tiles on 256 compute units, whole tiles against the stream-K plan.
        log("[bench] drawing inputs for 8192x1024x8192")
        g = torch.Generator().manual_seed(81)
        ps = Problem.random(g, 8192, 1024, 8192, "row", "row", dist="normal").to_device()
        Ds = ps.new_d(0.0)
        plan_w = migemm.Plan(ps.desc())
        plan_s = migemm.Plan(ps.desc(flags=migemm.MIGEMM_F_STREAM_K))
        ws = None
        if plan_s.workspace_size:
            ws = torch.empty(plan_s.workspace_size, dtype=torch.uint8, device="cuda")
            migemm.gemm_workspace_init(plan_s.handle, ws)
        flops_s = 2.0 * ps.M * ps.N * ps.K
        n_s, w_s = max(10, args.steps // 2), max(5, args.warmup // 2)
        ms_w = time_calls(lambda: migemm.gemm_run(plan_w.handle, ps.dA, ps.dB, None, Ds, 1.0, 0.0,
                                                  None, stream), n_s, w_s, stream)
        ms_s = time_calls(lambda: migemm.gemm_run(plan_s.handle, ps.dA, ps.dB, None, Ds, 1.0, 0.0,
                                                  ws, stream), n_s, w_s, stream)
        extra["share_8192x1024x8192_whole_tiles_tflops"] = round(flops_s / (ms_w * 1e-3) / 1e12, 1)
        extra["share_8192x1024x8192_stream_k_tflops"] = round(flops_s / (ms_s * 1e-3) / 1e12, 1)
        extra["share_8192x1024x8192_stream_k_tiles"] = int(plan_s.info.stream_k_tiles)
        del ps, Ds, ws
        # 2048 x 2048 x 8192: 64 tiles, each split over four workgroups by
        # the stream-K plan (the cost model's choice), whole tiles beside it.
        log("[bench] drawing inputs for 2048x2048x8192")
        g = torch.Generator().manual_seed(82)
        pm = Problem.random(g, 2048, 2048, 8192, "row", "row", dist="normal").to_device()
        Dm = pm.new_d(0.0)
        plan_mw = migemm.Plan(pm.desc())
        plan_ms = migemm.Plan(pm.desc(flags=migemm.MIGEMM_F_STREAM_K))
        wsm = None
        if plan_ms.workspace_size:
            wsm = torch.empty(plan_ms.workspace_size, dtype=torch.uint8, device="cuda")
            migemm.gemm_workspace_init(plan_ms.handle, wsm)
        flops_m = 2.0 * pm.M * pm.N * pm.K
        ms_mw = time_calls(lambda: migemm.gemm_run(plan_mw.handle, pm.dA, pm.dB, None, Dm, 1.0, 0.0,
                                                   None, stream), n_s, w_s, stream)
        ms_ms = time_calls(lambda: migemm.gemm_run(plan_ms.handle, pm.dA, pm.dB, None, Dm, 1.0, 0.0,
                                                   wsm, stream), n_s, w_s, stream)
        extra["gemm_2048x2048x8192_whole_tiles_tflops"] = round(flops_m / (ms_mw * 1e-3) / 1e12, 1)
        extra["gemm_2048x2048x8192_stream_k_tflops"] = round(flops_m / (ms_ms * 1e-3) / 1e12, 1)
        extra["gemm_2048x2048x8192_stream_k_tiles"] = int(plan_ms.info.stream_k_tiles)
        del pm, Dm, wsm

    out = {
        "metric": "GEMM TFLOP/s and % of MI355X MFMA peak (bf16 8192^3, fp8) on 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "M": w.M, "N": w.N, "K": w.K,
            "a_layout": w.a_layout, "b_layout": w.b_layout,
            "entries": "N(0,1)/sqrt(K) rounded to bf16",
            "tile_consumer": consumer,
            "parallelism": "single GPU, persistent grid",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(),
        },
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a slice of the workload")
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
