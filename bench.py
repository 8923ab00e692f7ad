#!/usr/bin/env python3
"""SGEMM benchmark on one MI355X: GFLOP/s and fraction of the fp32 peak.

    python bench.py [--steps K] [--warmup W]            # headline line (4096^3)
    python bench.py --workload mlp_up                   # another named workload
    python bench.py --sweep sweep.json                  # every workload, table
                                                        # (memory-bound shapes rotate over
                                                        # operand copies > the 256 MB MALL)
    python bench.py --copy-bytes 1073741824              # plain copy (counter calibration)

A step is one C = alpha*(A*B) + beta*C call on the resident, seeded synthetic
inputs of the workload (workloads.py).  GFLOP/s counts 2*M*N*K per call, the
convention of the pages' ladder table ("The GEMM Scrapbook"), and divides by
wall-clock time over the timed steps; the kernel's own average duration comes
from HIP events recorded on the stream the kernel is launched on, and is also
set against the rate of a register-only MFMA loop measured in the same run.
The CPU oracle is timed on a bounded sample of the same workload as a
reported baseline (rank 0, N = 1 only); the rows it computes also check the
GPU's output of one more call on the original C.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGEMM GFLOP/s at 4096³ fp32 and % of MI355X fp32 peak (1 GPU)"
PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 (matrix and packed vector)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TILE_DIRECT = 0x2  # sgemm_tile_desc.flags bit of the direct-load MFMA tiles
TILE_TRANS_B = 0x4  # ... of those compiled with edges (they also read B stored transposed)
TILE_TRANS_A = 0x8  # ... of those that read A stored transposed
KERNEL_SOURCES = {
    1: ["mfma_gemm.hip", "gemm_internal.hpp"],
    "direct": ["mfma_direct.hip", "direct_kernel.hpp", "gemm_internal.hpp"],
    "direct_ta": ["mfma_direct_ta.hip", "direct_kernel.hpp", "gemm_internal.hpp"],
    2: ["valu_gemm.hip", "gemm_internal.hpp"],
    3: ["skinny_gemm.hip", "gemm_internal.hpp"],
    6: ["small_gemm.hip", "gemm_internal.hpp"],
}


def kernel_source_hash(variant: int, desc: dict | None = None) -> str:
    h = hashlib.sha256()
    key = variant
    if variant == 1 and desc and desc.get("flags", 0) & TILE_DIRECT:
        key = "direct_ta" if desc["flags"] & TILE_TRANS_A else "direct"
    for f in KERNEL_SOURCES.get(key, []):
        with open(os.path.join(ROOT, "fp32_sgemm_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_name(variant: int, desc: dict) -> str:
    """A name for the compiled kernel that does not depend on table order."""
    fam = {1: "mfma", 2: "valu", 3: "skinny", 6: "small"}.get(variant, f"v{variant}")
    if not desc:
        return fam
    if variant == 1 and desc.get("flags", 0) & TILE_DIRECT:
        fam = "mfma_direct_ta" if desc["flags"] & TILE_TRANS_A else "mfma_direct"
    edges = "_edges" if variant == 1 and desc.get("flags", 0) & TILE_TRANS_B else ""
    return (f"{fam}_{desc['bm']}x{desc['bn']}x{desc['bk']}_w{desc['wm']}x{desc['wn']}"
            f"_s{desc.get('stages', 0)}_t{desc['threads']}{edges}")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square4096")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 MFMA, 2 VALU, 3 skinny")
    ap.add_argument("--tile", type=int, default=-1)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--op", default="NN", choices=["NN", "NT", "TN", "TT"],
                    help="storage of A and B: N as given, T transposed (sgemm_op)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock with amd-smi (for runs under a "
                         "profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--sweep", metavar="JSON_OUT", default=None)
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    default=None,
                    help="write the HBM traffic record of the workload's kernel from two "
                         "rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE) of this same command")
    ap.add_argument("--traffic-out", default=None,
                    help="traffic record file to update (default: profiles/traffic.json)")
    ap.add_argument("--probes", action="store_true",
                    help="measure the MFMA-f32 and VALU-FMA ceilings with register-only loops, "
                         "and the HBM read rate of a plain streaming read")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_sclk_mhz() -> float | None:
    """The mean of the GPU's graphics clocks (one per XCD) now, in MHz, from
    `amd-smi metric -g 0 -c --json`; None when the tool is not there."""
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                             text=True, timeout=10).stdout
        data = json.loads(out)
        gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
        clocks = [v["clk"]["value"] for k, v in gpu["clock"].items()
                  if k.startswith("gfx") and isinstance(v, dict) and "clk" in v]
        vals = [float(c) for c in clocks if isinstance(c, (int, float))]
        return sum(vals) / len(vals) if vals else None
    except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
        return None


def sustained_sclk(torch, call, seconds: float = 1.5) -> dict:
    """SCLK sampled (amd-smi, one sample about every 0.2 s) while `call` runs
    back to back for about `seconds`: the clock the kernel runs at."""
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is not None:
                samples.append(v)
            stop.wait(0.2)
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            call()
        n += 20
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return {"sclk_mhz": None, "samples": 0}
    return {"sclk_mhz": round(statistics.median(samples), 1), "samples": len(samples),
            "calls": n}


def cpu_baseline(w, A, B, C0, target_s: float):
    """Time the CPU oracle on a bounded band of rows of the same workload.
    Returns (the baseline record, the oracle's rows 0..R-1 of C)."""
    import numpy as np
    import oracle

    threads = oracle.default_threads()
    rows = 1 if w.M < 1 else min(w.M, 8)
    while True:
        a = np.ascontiguousarray(A[:rows])
        c = None if C0 is None else np.ascontiguousarray(C0[:rows])
        t0 = time.perf_counter()
        ref = oracle.sgemm(a, B, c, w.alpha, w.beta if c is not None else 0.0, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= 0.6 * target_s or rows >= w.M:
            break
        rows = min(w.M, max(rows + 1, int(rows * target_s / max(dt, 1e-3))))
    flops = 2.0 * rows * w.N * w.K
    out = {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
           "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
           "sample": f"rows 0..{rows - 1} of {w.name} ({rows} x {w.N} x {w.K}, "
                     f"{flops / 1e9:.2f} GFLOP), fp64-accumulating C oracle on {threads} threads"}
    return out, ref


def cpu_baseline_one_core(target: str = "square256") -> dict:
    """The oracle on one core for a small workload, as a per-core reference."""
    import oracle
    import workloads

    w = workloads.WORKLOADS[target]
    A, B, C0 = workloads.inputs(w)
    t0 = time.perf_counter()
    oracle.sgemm(A, B, None if C0 is None else C0.copy(), w.alpha,
                 w.beta if C0 is not None else 0.0, nthreads=1)
    dt = time.perf_counter() - t0
    return {"workload": w.name, "value": round(w.flops / dt / 1e9, 3), "unit": "GFLOP/s",
            "cores": 1, "seconds": round(dt, 4)}


def time_each(torch, call, steps, per: int = 1):
    """Device times (ms per call) of `steps` samples, each sample `per` calls
    back to back bracketed by its own pair of events on torch's current
    stream (the stream the library launches on).  Short kernels take several
    calls per sample, so that the events' own cost and the host's launch
    path stay small beside the sample."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for s, e in ev:
        s.record()
        for _ in range(per):
            call()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) / per for s, e in ev]


def time_calls(torch, call, steps, warmup):
    """(wall seconds for `steps` back-to-back calls, mean device time per call
    in ms).  One pair of HIP events brackets the whole timed region on torch's
    current stream, the stream the library launches on, so the mean is the
    average launch duration (plus whatever gaps the host leaves between
    launches) without per-call events between the kernels."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


MALL_BYTES = 256 * 1024 * 1024     # MI355X Infinity Cache


def operand_sets(torch, w, A, B, C0, dev, rotate: bool):
    """Device copies (A, B, C) of a workload's operands.  With `rotate`, enough
    copies that consecutive calls never find their operands in the 256 MB
    Infinity Cache (each call's inputs were last touched more than 256 MB of
    traffic earlier), so memory-bound shapes are timed against HBM."""
    per_set = 4 * (w.M * w.K + w.K * w.N + w.M * w.N)
    n = 1 if not rotate else max(2, -(-2 * MALL_BYTES // per_set) + 1)
    sets = []
    for _ in range(n):
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
        dC = (torch.from_numpy(C0).to(dev) if C0 is not None
              else torch.empty((w.M, w.N), device=dev))
        sets.append((dA, dB, dC))
    return sets


def time_rotating(torch, call_i, steps, warmup):
    """Per-call event durations (ms) of call_i(0), call_i(1), ... back to back."""
    for i in range(warmup):
        call_i(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (s, e) in enumerate(ev):
        s.record()
        call_i(warmup + i)
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def traffic_for(variant_used: int, kernel: str, desc: dict | None = None):
    """Measured HBM bytes per launch, if recorded for this exact kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(kernel)
    if not entry or entry.get("source_hash") != kernel_source_hash(variant_used, desc):
        return None
    return entry.get("bytes_per_launch")


def headline(args):
    import numpy as np
    import torch
    import fp32_sgemm_02_amd as sg
    import workloads

    w = workloads.WORKLOADS[args.workload]
    A, B, C0 = workloads.inputs(w)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # memory-bound workloads rotate over operand copies larger than the MALL
    sets = operand_sets(torch, w, A, B, C0, dev, rotate=(w.bound == "hbm"))
    trans_a, trans_b = args.op[0] == "T", args.op[1] == "T"
    if trans_a or trans_b:
        # A stored K x M and/or B stored N x K
        sets = [(a.t().contiguous() if trans_a else a, b.t().contiguous() if trans_b else b, c)
                for a, b, c in sets]
    dA, dB, dC = sets[0]
    kw = dict(trans_a=trans_a, trans_b=trans_b)
    if args.variant or args.tile >= 0 or args.group_m:
        kw.update(variant=args.variant, tile=args.tile, group_m=args.group_m)
    counter = [0]
    # the timed calls go straight to the C ABI (sgemm_op_ex) with arguments
    # prepared once per operand set: the binding's per-call checks cost more
    # host time than the memory-bound kernels run, which would leave the GPU
    # idle between launches and time the host instead of the kernel
    import ctypes
    lib = sg._load()
    cfg = (sg.SgemmConfig(kw["variant"], kw["tile"], 0, kw["group_m"]) if "variant" in kw
           else None)
    cfg_ref = ctypes.byref(cfg) if cfg is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    prepared = [(int(trans_a), int(trans_b), w.M, w.N, w.K, float(w.alpha), a.data_ptr(),
                 a.stride(0), b.data_ptr(), b.stride(0), float(w.beta), c.data_ptr(), c.stride(0),
                 stream, cfg_ref) for a, b, c in sets]

    def call():
        st = lib.sgemm_op_ex(*prepared[counter[0] % len(prepared)])
        counter[0] += 1
        if st != 0:
            raise sg.SgemmError(st)

    chosen = sg.select(w.M, w.N, w.K, dA.data_ptr(), dA.stride(0), dB.data_ptr(), dB.stride(0),
                       dC.data_ptr(), w.N, trans_a=trans_a, trans_b=trans_b)
    variant = args.variant or chosen.variant
    tile = args.tile if args.tile >= 0 else chosen.tile
    if args.variant and args.tile < 0:
        tile = -1
    # The register-only MFMA probe runs first: it is reported beside the
    # kernel's rate, and its ~35 ms of matrix work brings the graphics clock
    # from idle (~160 MHz) to its working value, so that the timed steps
    # measure the kernel rather than the clock ramp (measured: with only the
    # warm-up steps before them, the first timed 4096^3 launches took up to
    # 1.12 ms against a 0.93 ms median).
    probe = measure_probe(torch, "mfma_f32")
    if variant == 2:
        probe = measure_probe(torch, "valu_fma_f32")
    wall, kern_ms = time_calls(torch, call, args.steps, args.warmup)
    torch.cuda.synchronize()
    # after the timed region: per-call durations, and the clock the kernel runs at
    each = time_each(torch, call, args.steps, per=max(1, math.ceil(0.2 / kern_ms)))
    clock = {"sclk_mhz": None} if args.no_clock else sustained_sclk(torch, call)

    flops = w.flops
    value = flops * args.steps / wall / 1e9
    kern_s = kern_ms / 1e3
    desc = sg.tile_info(variant, tile) if tile >= 0 else {}
    kernel = kernel_name(variant, desc)
    bound = w.bound
    if bound == "hbm":
        achieved = w.min_bytes / kern_s / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        # the VALU family runs on the vector ALUs: the same 157.3 TFLOP/s
        # (256 CUs x 2.4 GHz x 256 FLOP per clock per CU), priced as "alu"
        bound = "alu" if variant == 2 else bound
        achieved = flops / kern_s / 1e12
        peak, unit = PEAK_FP32_TFLOPS, "TFLOP/s"
    traffic = traffic_for(variant, kernel, desc)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "pct_of_peak": round(100 * value / (PEAK_FP32_TFLOPS * 1e3), 2),
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha,
                   "beta": w.beta, "dist": w.dist, "seed": w.seed, "op": args.op,
                   "variant": variant,
                   "tile": tile, "tile_desc": desc},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kernel, "kernel_ms_mean": round(kern_s * 1e3, 4),
                     "kernel_ms_median": round(statistics.median(each), 4),
                     "kernel_ms_min": round(min(each), 4)},
    }
    if bound != "hbm":
        out["roofline"]["probe_tflops"] = probe["tflops"]
        out["roofline"]["frac_of_probe"] = round(achieved / probe["tflops"], 4)
        if "implied_clock_ghz" in probe:
            # the clock at which the probe's matrix work meets the spec rate
            out["roofline"]["probe_implied_clock_ghz"] = probe["implied_clock_ghz"]
        # amd-smi's graphics clock under ~1.5 s of back-to-back calls after the
        # timed region: power-limited, so lower than during the short timed
        # region (a ceiling for long runs, not a denominator for this one)
        out["roofline"]["sclk_mhz_sustained"] = clock["sclk_mhz"]
    if not args.no_cpu_baseline:
        base, ref = cpu_baseline(w, A, B, C0, args.cpu_seconds)
        # the GPU's rows of one more call on the original C, against the oracle's
        dCv = torch.from_numpy(C0).to(dev) if C0 is not None else torch.empty((w.M, w.N), device=dev)
        sg.gemm(dA, dB, dCv, w.alpha, w.beta, **kw)
        got = dCv[:ref.shape[0]].cpu().numpy()
        tol = (2e-5 * w.K * abs(w.alpha) * float(np.abs(A).max()) * float(np.abs(B).max())
               + (1e-6 * abs(w.beta) * np.abs(C0[:ref.shape[0]]) if C0 is not None else 0.0))
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        base["checked_rows"] = int(ref.shape[0])
        base["max_err_over_tol"] = float(np.max(err / tol)) if err.size else 0.0
        base["one_core"] = cpu_baseline_one_core()
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


def sweep(args):
    """Every named workload through automatic dispatch.  `kernel_ms_median` is
    the device time per call from HIP-graph replay (calls back to back with no
    host launch gaps); `eager_call_ms_median` brackets single eager calls with
    events and includes the host launch path, which dominates small shapes.
    Plans that keep partial sums also record `noalloc_kernel_ms_median`, the
    same plan replayed through sgemm_op_ex_noalloc (a captured sgemm call
    records an allocation and a free node, the no-alloc entry point none).
    Each workload's oracle is timed on a bounded band of rows
    (`oracle_gflops`, on `oracle_cores` threads of the host CPU)."""
    import numpy as np
    import torch
    import fp32_sgemm_02_amd as sg
    from fp32_sgemm_02_amd.tune import time_graph
    import workloads

    torch.cuda.set_device(0)
    dev = "cuda:0"
    rows = [{"host_cpu": cpu_model(), "sclk_mhz_idle": read_sclk_mhz()}]
    print(json.dumps(rows[0]), flush=True)
    names = [n for n in workloads.WORKLOADS if n != "probe256"]
    for name in names:
        w = workloads.WORKLOADS[name]
        A, B, C0 = workloads.inputs(w)
        hbm = w.bound == "hbm"
        sets = operand_sets(torch, w, A, B, C0, dev, rotate=hbm)
        variants = [0] + ([2] if name == "square4096" else [])
        for v in variants:
            kw = dict(variant=v) if v else {}
            call_i = lambda i, kw=kw: sg.gemm(*sets[i % len(sets)], w.alpha, w.beta, **kw)
            eager = statistics.median(time_rotating(torch, call_i, 30 if hbm else 20, 5)) / 1e3
            calls = max(len(sets), 20 if w.flops < 1e11 else 5)
            med = statistics.median(time_graph(torch, call_i, calls)) / 1e3
            cfg, erows, ecols = sg.plan(w.M, w.N, w.K)
            row = {"workload": name, "M": w.M, "N": w.N, "K": w.K,
                   "variant": v or cfg.variant, "tile": cfg.tile if v == 0 else -1,
                   "group_m": cfg.group_m if v == 0 else 0, "edge_rows": erows,
                   "kernel_ms_median": round(med * 1e3, 4),
                   "eager_call_ms_median": round(eager * 1e3, 4),
                   "gflops": round(w.flops / med / 1e9, 1),
                   "gbs": round(w.min_bytes / med / 1e9, 1),
                   "bound": "alu" if v == 2 else w.bound,
                   "operand_copies": len(sets)}
            keeps_sums = v == 0 and (cfg.flags & sg.FLAG_STREAMK or erows or
                                     (cfg.variant == sg.VARIANT_SKINNY and cfg.group_m > 1))
            if keeps_sums:
                call_n = lambda i: sg.gemm(*sets[i % len(sets)], w.alpha, w.beta, noalloc=True)
                row["noalloc_kernel_ms_median"] = round(
                    statistics.median(time_graph(torch, call_n, calls)), 4)
            if v == 0:
                base, _ = cpu_baseline(w, A, B, C0, 1.5)
                row.update(oracle_gflops=base["value"], oracle_cores=base["cores"],
                           oracle_sample=base["sample"])
            if hbm:
                row["pct_roofline"] = round(100 * row["gbs"] / PEAK_HBM_GBS, 2)
            else:
                row["pct_roofline"] = round(100 * row["gflops"] / (PEAK_FP32_TFLOPS * 1e3), 2)
            rows.append(row)
            print(json.dumps(row), flush=True)
        if name in TRANSPOSED_SWEEP:
            rows.extend(sweep_transposed(torch, sg, time_graph, w, sets[0]))
        if name in WEIGHT_NT_SWEEP:
            rows.append(sweep_weight_nt(torch, sg, time_graph, w, sets))
        if name in EPILOGUE_SWEEP:
            rows.extend(sweep_epilogue(torch, sg, time_graph, w, sets))
        del sets
        torch.cuda.empty_cache()
    rows.extend(sweep_streamk(torch, sg, time_graph))
    rows.extend(sweep_batched(torch, sg, time_graph))
    rows.extend(sweep_mixed(torch, sg, time_graph))
    with open(args.sweep, "w") as fh:
        json.dump(rows, fh, indent=1)


TRANSPOSED_SWEEP = ("square4096", "mlp_up", "mlp_down")


def sweep_transposed(torch, sg, time_graph, w, operands):
    """The workload with A and/or B stored transposed (sgemm_op through
    automatic dispatch), graph-replay device time per call."""
    A, B, C = operands
    out = []
    for ta, tb in ((False, True), (True, False), (True, True)):
        As = A.t().contiguous() if ta else A
        Bs = B.t().contiguous() if tb else B
        call_i = lambda i: sg.gemm(As, Bs, C, w.alpha, w.beta, trans_a=ta, trans_b=tb)
        med = statistics.median(time_graph(torch, call_i, 5)) / 1e3
        op = ("T" if ta else "N") + ("T" if tb else "N")
        cfg = sg.select(w.M, w.N, w.K, As.data_ptr(), As.stride(0), Bs.data_ptr(), Bs.stride(0),
                        C.data_ptr(), C.stride(0), trans_a=ta, trans_b=tb)
        row = {"workload": f"{w.name}_{op}", "M": w.M, "N": w.N, "K": w.K, "op": op,
               "variant": cfg.variant, "tile": cfg.tile,
               "kernel_ms_median": round(med * 1e3, 4),
               "gflops": round(w.flops / med / 1e9, 1), "bound": w.bound,
               "pct_roofline": round(100 * w.flops / med / 1e9 / (PEAK_FP32_TFLOPS * 1e3), 2)}
        print(json.dumps(row), flush=True)
        out.append(row)
        del As, Bs
    return out


WEIGHT_NT_SWEEP = ("row_1x4096x4096", "mlp_decode16")


def sweep_weight_nt(torch, sg, time_graph, w, sets):
    """A memory-bound workload with B stored N x K (a linear layer's weight,
    C = A W^T: decode), rotated over the same operand copies, through the
    entry point that allocates nothing; graph-replay device time per call."""
    ops = [(A, B.t().contiguous(), C) for A, B, C in sets]
    call_i = lambda i: sg.gemm(*ops[i % len(ops)], w.alpha, w.beta, trans_b=True, noalloc=True)
    med = statistics.median(time_graph(torch, call_i, max(len(ops), 20))) / 1e3
    A, Bt, C = ops[0]
    cfg = sg.select(w.M, w.N, w.K, A.data_ptr(), A.stride(0), Bt.data_ptr(), Bt.stride(0),
                    C.data_ptr(), C.stride(0), trans_b=True)
    gbs = w.min_bytes / med / 1e9
    row = {"workload": f"{w.name}_NT", "M": w.M, "N": w.N, "K": w.K, "op": "NT",
           "variant": cfg.variant, "tile": cfg.tile, "group_m": cfg.group_m,
           "kernel_ms_median": round(med * 1e3, 4), "gflops": round(w.flops / med / 1e9, 1),
           "gbs": round(gbs, 1), "bound": "hbm",
           "pct_roofline": round(100 * gbs / PEAK_HBM_GBS, 2), "operand_copies": len(ops)}
    print(json.dumps(row), flush=True)
    del ops
    return row


EPILOGUE_SWEEP = ("mlp_up", "mlp_decode16")


def sweep_epilogue(torch, sg, time_graph, w, sets):
    """The workload as a linear layer, C = act(X W^T + bias) with W stored
    N x K, for each activation (sgemm_epilogue, automatic dispatch), rotating
    over the operand copies like the plain rows."""
    ops = [(A, B.t().contiguous(), C) for A, B, C in sets]
    bias = torch.rand(w.N, device=ops[0][0].device) * 2 - 1
    out = []
    for act, label in ((None, "plain"), (sg.ACT_NONE, "bias"), (sg.ACT_RELU, "relu"),
                       (sg.ACT_SILU, "silu"), (sg.ACT_GELU_ERF, "gelu"),
                       (sg.ACT_GELU_TANH, "gelu_tanh")):
        def call_i(i, act=act):
            A, Wt, C = ops[i % len(ops)]
            if act is None:   # the product alone, W stored N x K
                sg.gemm(A, Wt, C, 1.0, 0.0, trans_b=True)
            else:
                sg.gemm(A, Wt, C, 1.0, 0.0, trans_b=True, bias=bias, act=act)
        calls = max(len(ops), 5 if w.flops > 1e11 else 20)
        med = statistics.median(time_graph(torch, call_i, calls)) / 1e3
        row = {"workload": f"{w.name}_NT_{label}", "M": w.M, "N": w.N, "K": w.K, "op": "NT",
               "epilogue": label, "operand_copies": len(ops),
               "kernel_ms_median": round(med * 1e3, 4),
               "gflops": round(w.flops / med / 1e9, 1), "bound": w.bound}
        if w.bound == "hbm":
            row["gbs"] = round((w.min_bytes + (4 * w.N if act is not None else 0)) / med / 1e9, 1)
            row["pct_roofline"] = round(100 * row["gbs"] / PEAK_HBM_GBS, 2)
        else:
            row["pct_roofline"] = round(100 * w.flops / med / 1e9 / (PEAK_FP32_TFLOPS * 1e3), 2)
        print(json.dumps(row), flush=True)
        out.append(row)
    return out


# batched shapes: (name, batch, M, N, K, trans_b) -- attention over 32 heads
# of 2048 positions with head dimension 128 (scores Q K^T and the weighted
# sum P V), and many small products
BATCHED_SWEEP = (("attn_scores_32x2048x2048x128", 32, 2048, 2048, 128, True),
                 ("attn_values_32x2048x128x2048", 32, 2048, 128, 2048, False),
                 ("small_512x128x128x64", 512, 128, 128, 64, True),
                 ("small_4096x32x32x32", 4096, 32, 32, 32, False))


# Few tiles of C with a long K: the automatic plan runs them as stream-K
# (M, N, K, A stored transposed, B stored transposed).
STREAMK_SWEEP = ((512, 512, 32768, False, False), (768, 768, 65536, False, True),
                 (1536, 1536, 8192, False, False), (3000, 3000, 3000, True, False))


def sweep_streamk(torch, sg, time_graph):
    """Shapes whose automatic plan is stream-K, beside the fastest compiled
    MFMA tile run one workgroup per tile (every applicable tile timed, no
    stream-K flag); graph-replay device time per call."""
    out = []
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(13)
    for M, N, K, ta, tb in STREAMK_SWEEP:
        A = torch.rand((K, M) if ta else (M, K), device="cuda:0", generator=gen) * 2 - 1
        B = torch.rand((N, K) if tb else (K, N), device="cuda:0", generator=gen) * 2 - 1
        C = torch.empty((M, N), device="cuda:0")
        cfg = sg.plan(M, N, K, trans_a=ta, trans_b=tb)[0]
        op = ("T" if ta else "N") + ("T" if tb else "N")
        flops = 2.0 * M * N * K

        def timed(**kw):
            call_i = lambda i: sg.gemm(A, B, C, trans_a=ta, trans_b=tb, **kw)
            return statistics.median(time_graph(torch, call_i, 10, replays=3)) / 1e3
        best = None
        for t in range(sg.tile_count(sg.VARIANT_MFMA)):
            try:
                sec = timed(variant=sg.VARIANT_MFMA, tile=t)
            except sg.SgemmError:
                continue   # the tile does not serve this transposition
            if best is None or sec < best[1]:
                best = (t, sec)
        for label, tile, sec, sk in (("auto", cfg.tile, timed(), bool(cfg.flags & sg.FLAG_STREAMK)),
                                     ("fastest tile, one per workgroup", best[0], best[1], False)):
            row = {"workload": f"longk_{M}x{N}x{K}_{op}", "M": M, "N": N, "K": K, "op": op,
                   "plan": label, "variant": sg.VARIANT_MFMA, "tile": tile, "streamk": sk,
                   "kernel_ms_median": round(sec * 1e3, 4),
                   "gflops": round(flops / sec / 1e9, 1), "bound": "mfma",
                   "pct_roofline": round(100 * flops / sec / 1e12 / PEAK_FP32_TFLOPS, 2)}
            print(json.dumps(row), flush=True)
            out.append(row)
        del A, B, C
    return out


def sweep_batched(torch, sg, time_graph):
    """Strided-batched products (sgemm_strided_batched), graph-replay device
    time per call."""
    out = []
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    for name, batch, M, N, K, tb in BATCHED_SWEEP:
        A = torch.rand((batch, M, K), device="cuda:0", generator=gen) * 2 - 1
        B = torch.rand((batch, N, K) if tb else (batch, K, N), device="cuda:0", generator=gen)
        C = torch.empty((batch, M, N), device="cuda:0")
        call_i = lambda i: sg.gemm_batched(A, B, C, 1.0, 0.0, trans_b=tb)
        flops = 2.0 * batch * M * N * K
        med = statistics.median(time_graph(torch, call_i, 5 if flops > 1e11 else 20)) / 1e3
        byts = 4.0 * batch * (M * K + K * N + M * N)
        ai = flops / byts
        bound = "mfma" if ai > PEAK_FP32_TFLOPS * 1e3 / PEAK_HBM_GBS else "hbm"
        row = {"workload": name, "batch": batch, "M": M, "N": N, "K": K,
               "op": "NT" if tb else "NN", "kernel_ms_median": round(med * 1e3, 4),
               "gflops": round(flops / med / 1e9, 1), "gbs": round(byts / med / 1e9, 1),
               "bound": bound}
        row["pct_roofline"] = round(100 * (row["gflops"] / (PEAK_FP32_TFLOPS * 1e3)
                                           if bound == "mfma" else row["gbs"] / PEAK_HBM_GBS), 2)
        print(json.dumps(row), flush=True)
        out.append(row)
        del A, B, C
    return out


PEAK_16BIT_TFLOPS = 2500.0     # MI355X dense bf16 / fp16 matrix peak
MIXED_SWEEP = ((4096, 4096, 4096), (8192, 14336, 4096), (8192, 4096, 14336), (16, 14336, 4096))


def sweep_mixed(torch, sg, time_graph):
    """16-bit inputs (sgemm_mixed) as a linear layer, C = X W^T with W stored
    N x K, fp32 C; graph-replay device time per call.  The decode shape
    rotates over operand copies larger than the Infinity Cache."""
    out = []
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(11)
    for M, N, K in MIXED_SWEEP:
        for label, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
            per_set = 2 * (M * K + N * K) + 4 * M * N
            copies = 1 if M > 16 else max(2, -(-2 * MALL_BYTES // per_set) + 1)
            ops = [((torch.rand((M, K), device="cuda:0", generator=gen) * 2 - 1).to(dt),
                    (torch.rand((N, K), device="cuda:0", generator=gen) * 2 - 1).to(dt),
                    torch.empty((M, N), device="cuda:0")) for _ in range(copies)]

            def call_i(i):
                A, W, C = ops[i % len(ops)]
                sg.gemm_mixed(A, W, C, trans_b=True)
            flops = 2.0 * M * N * K
            med = statistics.median(time_graph(torch, call_i, max(copies, 5))) / 1e3
            byts = per_set
            bound = "mfma" if flops / byts > PEAK_16BIT_TFLOPS * 1e3 / PEAK_HBM_GBS else "hbm"
            row = {"workload": f"mixed_{label}_{M}x{N}x{K}_NT", "M": M, "N": N, "K": K,
                   "op": "NT", "inputs": label, "kernel_ms_median": round(med * 1e3, 4),
                   "gflops": round(flops / med / 1e9, 1), "gbs": round(byts / med / 1e9, 1),
                   "bound": bound, "operand_copies": copies}
            row["pct_roofline"] = round(100 * (row["gflops"] / (PEAK_16BIT_TFLOPS * 1e3)
                                               if bound == "mfma" else row["gbs"] / PEAK_HBM_GBS),
                                        2)
            print(json.dumps(row), flush=True)
            out.append(row)
            del ops
    return out


# FETCH_SIZE / WRITE_SIZE counter bytes -> true bytes, from a 1 GiB device
# copy of known size (profiles/hbm_counter_calibration_copy1GiB.md)
FETCH_FACTOR, WRITE_FACTOR = 2.0, 1.0


def read_counter_csv(path: str) -> dict:
    """{kernel name: (dispatches, mean counter KiB per dispatch, summed
    duration ns)} from a rocprofv3 counter_collection.csv with one counter."""
    import csv

    acc = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            name = row["Kernel_Name"]
            d = acc.setdefault(name, {})
            disp = row["Dispatch_Id"]
            v, dur = float(row["Counter_Value"]), int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            prev = d.get(disp, (0.0, dur))
            d[disp] = (prev[0] + v, dur)
    out = {}
    for name, d in acc.items():
        vals = [v for v, _ in d.values()]
        out[name] = (len(vals), sum(vals) / len(vals), sum(t for _, t in d.values()))
    return out


def record_traffic(args):
    """The HBM traffic record of the kernel this command times: the dominant
    library kernel (largest summed duration; probes, and torch's kernels that
    prepare operands such as the transposed copies of --op, excluded) of two
    counter runs,
    scaled by the copy calibration, keyed by the kernel's name and the hash
    of its source files, so that bench.py reports it only while the source is
    unchanged."""
    import fp32_sgemm_02_amd as sg
    import workloads

    w = workloads.WORKLOADS[args.workload]
    trans_a, trans_b = args.op[0] == "T", args.op[1] == "T"
    chosen = sg.select(w.M, w.N, w.K, trans_a=trans_a, trans_b=trans_b)
    variant = args.variant or chosen.variant
    tile = args.tile if args.tile >= 0 else chosen.tile
    desc = sg.tile_info(variant, tile) if tile >= 0 else {}
    fetch, write = (read_counter_csv(f) for f in args.record_traffic)
    names = [n for n in fetch if "probe_" not in n and "sg::" in n]
    main = max(names, key=lambda n: fetch[n][2])
    f_kib, w_kib = fetch[main][1], write[main][1]
    rec = {"kernel": main, "workload": w.name, "source_hash": kernel_source_hash(variant, desc),
           "dispatches": fetch[main][0], "fetch_kib_per_dispatch": round(f_kib, 1),
           "write_kib_per_dispatch": round(w_kib, 1), "fetch_factor": FETCH_FACTOR,
           "write_factor": WRITE_FACTOR, "fetch_bytes": int(f_kib * 1024 * FETCH_FACTOR),
           "write_bytes": int(w_kib * 1024 * WRITE_FACTOR),
           "bytes_per_launch": int(f_kib * 1024 * FETCH_FACTOR + w_kib * 1024 * WRITE_FACTOR),
           "algorithmic_bytes": w.min_bytes}
    path = args.traffic_out or TRAFFIC_FILE
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        data = {}
    data.setdefault("_about", "HBM/fabric bytes per launch from rocprofv3 --pmc FETCH_SIZE and "
                              "WRITE_SIZE (KiB per dispatch), each scaled by the factor that maps "
                              "the same counter onto a 1 GiB device copy of known size. "
                              "source_hash covers the kernel's source files; bench.py reports "
                              "traffic only while it matches.")
    data[kernel_name(variant, desc)] = rec
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1)
    print(json.dumps({kernel_name(variant, desc): rec}), flush=True)


def copy_calibration(args):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch

    torch.cuda.set_device(0)
    n = args.copy_bytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    wall, ms = time_calls(torch, lambda: dst.copy_(src), args.steps, args.warmup)
    print(json.dumps({"copy_bytes": n * 4, "read_bytes": n * 4, "write_bytes": n * 4,
                      "kernel_ms_mean": round(ms, 4),
                      "gbs": round(2 * n * 4 / (ms / 1e3) / 1e9, 1)}), flush=True)


def measure_probe(torch, name: str, steps: int = 10, warmup: int = 3) -> dict:
    """A register-only loop of fp32 MFMAs ("mfma_f32") or plain FMAs
    ("valu_fma_f32") on every SIMD: the rate this machine sustains."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "fp32_sgemm_02_amd", "libfp32probes.so"))
    kind = name.split("_")[0]
    getattr(lib, f"probe_{kind}_flops").restype = ctypes.c_double
    getattr(lib, f"probe_{kind}_flops").argtypes = [ctypes.c_int, ctypes.c_int]
    getattr(lib, f"probe_{kind}_f32").restype = ctypes.c_int
    getattr(lib, f"probe_{kind}_f32").argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                 ctypes.c_void_p]
    blocks = 256 * 8
    iters = 2000 if kind == "mfma" else 20000
    peak = PEAK_FP32_TFLOPS
    out = torch.empty(blocks * 256, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    flops = getattr(lib, f"probe_{kind}_flops")(blocks, iters)
    launch = getattr(lib, f"probe_{kind}_f32")
    _, ms = time_calls(torch, lambda: launch(blocks, iters, out.data_ptr(), stream), steps, warmup)
    tf = flops / (ms / 1e3) / 1e12
    out = {"probe": name, "tflops": round(tf, 2), "peak_tflops": peak,
           "frac": round(tf / peak, 4), "kernel_ms_mean": round(ms, 4)}
    if kind == "mfma":
        # the matrix cores retire 256 FP32 FLOP per clock per CU
        out["implied_clock_ghz"] = round(tf * 1e12 / (256 * 256) / 1e9, 3)
    return out


def measure_read_probe(torch, floats: int, blocks: int) -> dict:
    """The streaming-read probe over `floats` floats with `blocks` workgroups,
    graph-replayed back to back over copies larger than twice the Infinity
    Cache (so every launch reads HBM)."""
    import ctypes
    from fp32_sgemm_02_amd.tune import time_graph

    lib = ctypes.CDLL(os.path.join(ROOT, "fp32_sgemm_02_amd", "libfp32probes.so"))
    lib.probe_read_f32.restype = ctypes.c_int
    lib.probe_read_f32.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    copies = max(2, -(-2 * MALL_BYTES // (4 * floats)) + 1)
    bufs = [torch.ones(floats, device="cuda:0") for _ in range(copies)]
    out = torch.empty(blocks * 256, device="cuda:0")

    def call_i(i):
        st = lib.probe_read_f32(bufs[i % copies].data_ptr(), floats, blocks, out.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"probe_read_f32: {st}")
    ms = statistics.median(time_graph(torch, call_i, 2 * copies))
    del bufs
    return {"probe": "read_f32", "MB": round(4 * floats / 1e6, 1), "workgroups": blocks,
            "us": round(ms * 1e3, 2), "TBs": round(4 * floats / (ms / 1e3) / 1e12, 3),
            "frac_of_8TBs": round(4 * floats / (ms / 1e3) / 8e12, 4)}


def probes(args):
    """Register-only MFMA and FMA loops: the rates the chip sustains on this
    box; and a streaming read of 67 MB (one 4096 x 4096 operand) and 235 MB
    (the 4096 x 14336 weight of the decode shape) with 224 .. 2048
    workgroups: what a memory-bound kernel can reach, and how many
    workgroups it takes."""
    import torch

    torch.cuda.set_device(0)
    for name in ("mfma_f32", "valu_fma_f32"):
        print(json.dumps(measure_probe(torch, name)), flush=True)
    for floats in (4096 * 4096, 4096 * 14336):
        for blocks in (224, 256, 512, 1024, 2048):
            if floats % (4 * blocks) == 0:
                print(json.dumps(measure_read_probe(torch, floats, blocks)), flush=True)
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(args)
    elif args.probes:
        probes(args)
    elif args.copy_bytes:
        copy_calibration(args)
    elif args.sweep:
        sweep(args)
    else:
        headline(args)


if __name__ == "__main__":
    main()
