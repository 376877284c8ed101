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


def code_tokens(text: str) -> str:
    """C++ source without its comments, and with every run of white space
    made one space: what the compiler sees, so that an edit to a comment
    leaves the kernel, and its hash, unchanged.  (String and character
    literals are kept whole, so a "//" inside one is not a comment.)"""
    import re
    pat = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)
    out = pat.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(out.split())


def kernel_source_hash() -> str:
    """sha1 over the device-side sources (the kernel translation unit and its
    headers, comments and layout left out), in a fixed order: identifies the
    kernel whose counters a traffic profile holds."""
    import hashlib
    csrc = os.path.join(HERE, "warp_specialized_pipelined_amd", "csrc")
    files = [os.path.join(csrc, "gemm_kernels.hip"), os.path.join(csrc, "launch.h")]
    kdir = os.path.join(csrc, "kernel")
    files += [os.path.join(kdir, f) for f in sorted(os.listdir(kdir)) if f.endswith(".hpp")]
    h = hashlib.sha1()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
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
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="untimed back-to-back steps before the warm-up, for steady clocks")
    ap.add_argument("--variant", choices=["full", "consumer", "overlap", "plain", "fp8", "cfg1", "cfg2",
                                          "cfg3", "cfg3_m256", "copy", "trace"], default="full",
                    help="profiling runs: time one kernel only and print a short line "
                         "(copy = a plain 128 MiB device copy, the byte-counter calibration; "
                         "cfg3_m256 = the ragged workload on 256-row tiles instead of the "
                         "plan's 192)")
    return ap.parse_args()


VARIANTS = {"consumer": 3, "overlap": 3, "plain": 3, "fp8": 4, "cfg1": 0, "cfg2": 1, "cfg3": 2,
            "cfg3_m256": 2}


def run_variant(args):
    """One kernel, timed alone (for rocprofv3 counter passes): the 8192^3
    bf16 workload with the tile consumer (staged or overlapped schedule) or
    plain, the e4m3 workload, one of the three smaller workloads, or a
    128 MiB device copy (the byte-counter calibration)."""
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
    if args.variant == "trace":
        run_trace(args)
        return
    w = synth.WORKLOADS[VARIANTS[args.variant]]
    p = Problem.from_workload(w).to_device()
    D = p.new_d(0.0)
    if args.variant in ("consumer", "overlap"):
        flags = migemm.MIGEMM_F_TILE_CONSUMER
        if args.variant == "overlap":
            flags |= migemm.MIGEMM_F_CONSUMER_OVERLAP
        plan = migemm.Plan(p.desc(flags=flags))
        ld = (w.N + 255) // 256
        rs = torch.empty((w.M, ld), dtype=torch.float32, device="cuda")
        rm = torch.empty_like(rs)
        Dc = torch.empty_like(D)
        fn = lambda: migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, None, D, p.alpha,
                                                        0.0, rs, rm, Dc, None, stream)
    else:
        flags = migemm.MIGEMM_F_TILE_M256 if args.variant == "cfg3_m256" else 0
        plan = migemm.Plan(p.desc(flags=flags))
        fn = lambda: migemm.gemm_run(plan.handle, p.dA, p.dB, p.dC, D, p.alpha, p.beta, None,
                                     stream)
    ms = time_calls(fn, args.steps, args.warmup, stream)
    print(json.dumps({"variant": args.variant, "workload": w.name, "ms": round(ms, 4),
                      "TFLOP/s": round(w.flops / (ms * 1e-3) / 1e12, 1),
                      "tile_m": int(plan.info.tile_m)}))


def run_trace(args):
    """The 8192^3 tile-consumer workload with the hand-off debug trace, in
    both schedules: a few untimed runs, then one traced run each, summarized
    (where each tile's copy ran against the next tile's K loop, the ring's
    occupancy, the waits)."""
    import torch
    from warp_specialized_pipelined_amd import handoff_trace, migemm, synth
    from tests.helpers import Problem
    w = synth.WORKLOADS[3]
    p = Problem.from_workload(w).to_device()
    D = p.new_d(0.0)
    ld = (w.N + 255) // 256
    rs = torch.empty((w.M, ld), dtype=torch.float32, device="cuda")
    rm = torch.empty_like(rs)
    Dc = torch.empty_like(D)
    out = {"workload": w.name}
    for name, extra in (("staged", 0), ("overlapped", migemm.MIGEMM_F_CONSUMER_OVERLAP)):
        plan = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER | extra |
                                  migemm.MIGEMM_F_HANDOFF_DEBUG))
        ws = torch.empty(plan.workspace_size, dtype=torch.uint8, device="cuda")
        run = lambda: migemm.gemm_run_with_tile_consumer(plan.handle, p.dA, p.dB, None, D, p.alpha,
                                                         0.0, rs, rm, Dc, ws)
        migemm.gemm_workspace_init(plan.handle, ws)
        for _ in range(max(args.warmup, 1)):
            run()
        migemm.gemm_workspace_init(plan.handle, ws)
        run()
        st, info = migemm.gemm_debug_read(plan.handle, ws)
        summ = handoff_trace.summarize(handoff_trace.records(ws, info), name)
        summ["status"] = migemm.gemm_status_string(st)
        summ["waits_given_up"] = int(info.waits_given_up)
        out[name] = summ
    print(json.dumps(out))


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


def settle(fn, stream, seconds):
    """Run `fn` back to back for about `seconds` (untimed): the board's clock
    and power take ~30 launches of a large GEMM to reach their steady state,
    which a fresh process has not yet reached after a few warm-up steps."""
    import torch
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    return n


def per_launch_ms(fn, n, stream):
    """n back-to-back launches with a HIP event recorded on the launch stream
    between consecutive ones; returns the n per-launch times in ms."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def summary_us(ms_list):
    import statistics
    return {"median_us": round(1e3 * statistics.median(ms_list), 2),
            "min_us": round(1e3 * min(ms_list), 2),
            "mean_us": round(1e3 * sum(ms_list) / len(ms_list), 2),
            "launches": len(ms_list)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
    the sample counts; None where amdgpu's sysfs exposes no clock."""
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
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"first {rows} rows of the {p.M}x{p.N}x{p.K} product (all columns, full K), "
                  f"fp64 accumulation, {t:.1f} s",
    }


def algorithmic_bytes(w, consumer=False):
    """Bytes the method must move per launch: A and B read once, D written
    once, C read once when beta != 0; the tile consumer adds the copy
    (MN x 2) and the two statistics arrays (2 M ceil(N/256) x 4)."""
    es = 2 if w.dtype == 1 else 1
    b = (w.M * w.K + w.K * w.N) * es + w.M * w.N * 2
    if w.beta != 0.0:
        b += w.M * w.N * 2
    if consumer:
        b += w.M * w.N * 2 + 2 * w.M * ((w.N + 255) // 256) * 4
    return b


def config_figures(w, ms_list, consumer=False):
    """Median/min time of one workload with its roofline: MFMA-bound when its
    arithmetic intensity is above the ridge point (peak flop/s / 8 TB/s),
    HBM-bound below it."""
    import statistics
    peak = PEAK_BF16_TFLOPS if w.dtype == 1 else PEAK_FP8_TFLOPS
    med = statistics.median(ms_list)
    tflops = w.flops / (med * 1e-3) / 1e12
    nbytes = algorithmic_bytes(w, consumer)
    gbs = nbytes / (med * 1e-3) / 1e9
    ai = w.flops / nbytes
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if ai >= ridge else "hbm"
    out = summary_us(ms_list)
    out.update({
        "shape": f"{w.M}x{w.N}x{w.K}", "dtype": "bf16" if w.dtype == 1 else "e4m3",
        "layouts": f"A {w.a_layout}, B {w.b_layout}", "alpha": w.alpha, "beta": w.beta,
        "tflops_at_median": round(tflops, 1), "mfma_peak_tflops": round(peak, 1),
        "frac_of_mfma_peak": round(tflops / peak, 4),
        "algorithmic_bytes": nbytes, "hbm_gbs_at_median": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "arithmetic_intensity": round(ai, 1), "bound": bound,
        "frac_of_roofline": round(tflops / peak if bound == "mfma" else gbs / HBM_PEAK_GBS, 4),
    })
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import statistics
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
    plan_cons = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER))
    plan_ov = migemm.Plan(p.desc(flags=migemm.MIGEMM_F_TILE_CONSUMER |
                                 migemm.MIGEMM_F_CONSUMER_OVERLAP))
    stat_ld = (w.N + 255) // 256
    row_sum = torch.empty((w.M, stat_ld), dtype=torch.float32, device="cuda")
    row_max = torch.empty((w.M, stat_ld), dtype=torch.float32, device="cuda")
    D_copy = torch.empty_like(D)

    def step_plain():
        migemm.gemm_run(plan_plain.handle, p.dA, p.dB, None, D, p.alpha, 0.0, None, stream)

    def step_cons():
        migemm.gemm_run_with_tile_consumer(plan_cons.handle, p.dA, p.dB, None, D, p.alpha, 0.0,
                                           row_sum, row_max, D_copy, None, stream)

    def step_ov():
        migemm.gemm_run_with_tile_consumer(plan_ov.handle, p.dA, p.dB, None, D, p.alpha, 0.0,
                                           row_sum, row_max, D_copy, None, stream)

    step = step_cons
    # The board needs ~30 launches of this GEMM to reach the clock and power
    # it then holds; a settle run first, so the timed steps measure that
    # steady state rather than the ramp.
    n_settle = settle(step, stream, args.settle_seconds)
    log(f"[bench] settled with {n_settle} untimed steps; timing {args.steps} steps after "
        f"{args.warmup} warm-up")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_calls(step, args.steps, args.warmup, stream)
    wall = time.perf_counter() - t0
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step  {tflops:.1f} TFLOP/s  ({wall:.1f} s wall)")

    extra = {"consumer_schedule": "staged (the default of gemm_run_with_tile_consumer)",
             "settle_steps": n_settle,
             "pages_throughput_figures": "none: the pages publish no throughput figures, so there "
                                         "is no external number to compare with"}

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

    if not args.no_extra:
        # Plain GEMM against both schedules of the tile consumer, interleaved
        # (plain, staged, overlapped) x 5 rounds on the same inputs, so that
        # clock drift falls on all three alike.
        n_i = max(10, args.steps // 2)
        times = {"plain": [], "staged": [], "overlapped": []}
        fns = {"plain": step_plain, "staged": step_cons, "overlapped": step_ov}
        for _ in range(5):
            for name, fn in fns.items():
                fn()                              # one untimed launch at each switch
                times[name] += per_launch_ms(fn, n_i, stream)
        med = {k: statistics.median(v) for k, v in times.items()}
        extra["interleaved_8192"] = {
            "order": "(plain, staged consumer, overlapped consumer) x 5 rounds of "
                     f"{n_i} launches each, per-launch HIP events",
            "plain": config_figures(w, times["plain"]),
            "staged": config_figures(w, times["staged"], consumer=True),
            "overlapped": config_figures(w, times["overlapped"], consumer=True),
            "staged_over_plain_time": round(med["staged"] / med["plain"], 4),
            "overlapped_over_plain_time": round(med["overlapped"] / med["plain"], 4),
        }
        log(f"[bench] interleaved medians (ms): {med}")
        extra["plain_gemm_tflops"] = extra["interleaved_8192"]["plain"]["tflops_at_median"]
        extra["plain_gemm_frac_of_peak"] = extra["interleaved_8192"]["plain"]["frac_of_mfma_peak"]
        extra["consumer_over_plain_time"] = extra["interleaved_8192"]["staged_over_plain_time"]
        extra["consumer_overlapped_over_plain_time"] = \
            extra["interleaved_8192"]["overlapped_over_plain_time"]
        clock_extras("", step, ms, w.flops, 4096)
        clock_extras("plain_gemm_", step_plain, med["plain"], w.flops, 4096)
        # The vendor library on the same inputs, for reference only: torch's
        # bf16 matmul (hipBLASLt) of the same row-major A and B, contiguous.
        if p.a_rs == w.K and p.b_rs == w.N and p.a_cs == 1 and p.b_cs == 1:
            A2 = p.dA.view(w.M, w.K)
            B2 = p.dB.view(w.K, w.N)
            out2 = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
            lib = lambda: torch.matmul(A2, B2, out=out2)
            settle(lib, stream, 0.5)
            ms_lib = statistics.median(per_launch_ms(lib, max(10, args.steps // 2), stream))
            extra["library_gemm_tflops"] = round(w.flops / (ms_lib * 1e-3) / 1e12, 1)
            extra["library_gemm"] = "torch.matmul bf16 (hipBLASLt), same A and B, no consumer"
            clock_extras("library_gemm_", lib, ms_lib, w.flops, 4096)
            del out2
        del D_copy, row_sum, row_max

        # Every workload of the set, one after another: gemm_run on its own
        # plan (the 8192^3 one is the interleaved block above).
        configs = {}
        for wc in synth.WORKLOADS:
            if wc is w:
                continue
            log(f"[bench] workload {wc.name}")
            pc = Problem.from_workload(wc).to_device()
            Dc = pc.new_d(0.0)
            plan_c = migemm.Plan(pc.desc())
            fn = lambda: migemm.gemm_run(plan_c.handle, pc.dA, pc.dB, pc.dC, Dc, pc.alpha,
                                         pc.beta, None, stream)
            settle(fn, stream, 0.4)
            n_c = max(20, args.steps)
            if wc.M * wc.N * wc.K <= 256 ** 3:
                n_c = 200                         # a few microseconds each
            configs[wc.name] = config_figures(wc, per_launch_ms(fn, n_c, stream))
            configs[wc.name]["tile_m"] = int(plan_c.info.tile_m)   # the plan's tile height
            if wc.dtype == synth.E4M3:
                clock_extras("fp8_gemm_", fn, statistics.median(per_launch_ms(fn, 5, stream)),
                             wc.flops, 8192)
            del pc, Dc
        configs[w.name] = extra["interleaved_8192"]["staged"]
        # The source C of the beta = 0.5 workload: read during the K loop's
        # last two iterations (the plan's choice here) or in the epilogue,
        # against the same GEMM with beta = 0, interleaved x 5.
        w2 = synth.WORKLOADS[1]
        p2 = Problem.from_workload(w2).to_device()
        D2 = p2.new_d(0.0)
        plan_k = migemm.Plan(p2.desc())
        plan_e = migemm.Plan(p2.desc(flags=migemm.MIGEMM_F_C_IN_EPILOGUE))
        fc = {"c_in_k_loop": lambda: migemm.gemm_run(plan_k.handle, p2.dA, p2.dB, p2.dC, D2, 1.0,
                                                       p2.beta, None, stream),
              "c_in_epilogue": lambda: migemm.gemm_run(plan_e.handle, p2.dA, p2.dB, p2.dC, D2, 1.0,
                                                         p2.beta, None, stream),
              "beta_zero": lambda: migemm.gemm_run(plan_k.handle, p2.dA, p2.dB, None, D2, 1.0, 0.0,
                                                   None, stream)}
        settle(fc["c_in_k_loop"], stream, 0.3)
        tc = {k: [] for k in fc}
        for _ in range(5):
            for name, fn in fc.items():
                fn()
                tc[name] += per_launch_ms(fn, max(10, args.steps // 2), stream)
        mc = {k: statistics.median(v) for k, v in tc.items()}
        extra["c_read_" + w2.name] = {
            "plan_reads_c_in_k_loop": int(plan_k.info.c_in_k_loop),
            **{k + "_median_us": round(1e3 * v, 2) for k, v in mc.items()},
            "c_in_k_loop_over_beta_zero": round(mc["c_in_k_loop"] / mc["beta_zero"], 4),
            "c_in_epilogue_over_beta_zero": round(mc["c_in_epilogue"] / mc["beta_zero"], 4),
        }
        del p2, D2
        extra["workloads"] = configs
        w8 = synth.WORKLOADS[4]
        extra["fp8_gemm_tflops"] = configs[w8.name]["tflops_at_median"]
        extra["fp8_gemm_frac_of_peak"] = configs[w8.name]["frac_of_mfma_peak"]

        # One GPU's share of an 8-way split of N, 8192 x 1024 x 8192 bf16: 128
        # tiles on 256 compute units, whole 256-row tiles against 192-row
        # tiles (172 of them) and the plan that may choose stream-K; and
        # 2048 x 2048 x 8192 (64 tiles, each split four ways).
        for (M_, N_, K_, seed, key) in ((8192, 1024, 8192, 81, "share_8192x1024x8192"),
                                        (2048, 2048, 8192, 82, "gemm_2048x2048x8192")):
            log(f"[bench] drawing inputs for {M_}x{N_}x{K_}")
            g = torch.Generator().manual_seed(seed)
            ps = Problem.random(g, M_, N_, K_, "row", "row", dist="normal").to_device()
            Ds = ps.new_d(0.0)
            plan_w = migemm.Plan(ps.desc(flags=migemm.MIGEMM_F_TILE_M256))
            plan_t = migemm.Plan(ps.desc(flags=migemm.MIGEMM_F_TILE_M192))
            plan_s = migemm.Plan(ps.desc(flags=migemm.MIGEMM_F_STREAM_K))
            ws = None
            if plan_s.workspace_size:
                ws = torch.empty(plan_s.workspace_size, dtype=torch.uint8, device="cuda")
                migemm.gemm_workspace_init(plan_s.handle, ws)
            flops_s = 2.0 * M_ * N_ * K_
            fw = lambda: migemm.gemm_run(plan_w.handle, ps.dA, ps.dB, None, Ds, 1.0, 0.0, None,
                                         stream)
            fs = lambda: migemm.gemm_run(plan_s.handle, ps.dA, ps.dB, None, Ds, 1.0, 0.0, ws,
                                         stream)
            ft = lambda: migemm.gemm_run(plan_t.handle, ps.dA, ps.dB, None, Ds, 1.0, 0.0, None,
                                         stream)
            settle(fw, stream, 0.2)
            ms_w = statistics.median(per_launch_ms(fw, max(20, args.steps), stream))
            settle(ft, stream, 0.2)
            ms_t = statistics.median(per_launch_ms(ft, max(20, args.steps), stream))
            settle(fs, stream, 0.2)
            ms_s = statistics.median(per_launch_ms(fs, max(20, args.steps), stream))
            extra[key + "_whole_tiles_tflops"] = round(flops_s / (ms_w * 1e-3) / 1e12, 1)
            extra[key + "_tile_m192_tflops"] = round(flops_s / (ms_t * 1e-3) / 1e12, 1)
            extra[key + "_stream_k_tflops"] = round(flops_s / (ms_s * 1e-3) / 1e12, 1)
            extra[key + "_stream_k_tiles"] = int(plan_s.info.stream_k_tiles)
            extra[key + "_stream_k_plan_tile_m"] = int(plan_s.info.tile_m)
            del ps, Ds, ws

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
            "tile_consumer": True,
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
