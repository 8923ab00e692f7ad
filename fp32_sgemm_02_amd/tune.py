"""Offline tuner: the fastest compiled configuration per problem shape.

    python -m fp32_sgemm_02_amd.tune --workloads square4096,mlp_up --out tune.json
    python -m fp32_sgemm_02_amd.tune --shapes 4097x1000x3001 --write-table

For every shape it times each applicable (kernel family, tile, group_m)
candidate on the GPU with HIP events (median of `--reps` calls after
`--warmup`), keeps the fastest, and optionally rewrites csrc/tuned_table.inc
with one exact-shape row per tuned shape (rebuild the library afterwards).
Autotuning tile sizes per GPU is the rung "The GEMM Scrapbook" fine print
credits with most of the gap before warptiling; here the candidates are the
compiled template instances of include/fp32_sgemm.h's families.

Correctness of every compiled configuration is established by the GPU parity
tests against the CPU oracle; as a guard against a mis-tuned table the tuner
also requires each candidate's output to agree with the automatic
configuration's output on the same inputs (same tolerance rule as the
tests) before it may win.

Graph-replayed timing (--graph) runs every candidate through
sgemm_op_ex_noalloc, so plans that keep partial sums (K-split skinny tiles,
stream-K) are not charged the allocation and free nodes a captured sgemm
call records; those the static scratch cannot hold (stream-K) are timed
eagerly after a warm-up call instead, and the cost of the nodes is reported
beside them as `graph_with_alloc_ms`.

    python -m fp32_sgemm_02_amd.tune --mixed bf16 --shapes 4096x4096x4096 --graph

times every 16-bit-input tile (sgemm_mixed, W stored N x K) instead; its
`eff_pct` (percent of the 2.5 PFLOP/s 16-bit matrix peak) is what the
16-bit tile table's efficiencies are read from.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TABLE = os.path.join(HERE, "csrc", "tuned_table.inc")

GROUPS = (1, 2, 4, 8, 16)


def parse_shape(text: str):
    m, n, k = (int(x) for x in text.lower().split("x"))
    return m, n, k


SLICES = (1, 2, 4, 8, 16, 32)   # K slices of the few-rows skinny tiles


def candidates(sg, M, N, K, sweep_groups: bool):
    """(variant, tile, group_m, flags) to time.  The first is the automatic
    plan without the tuned table (the cost model, edge strips included); when
    it wins, the shape needs no table row.  Then every MFMA tile (and its
    stream-K form where it has one), every VALU tile, every small-product
    tile, and for skinny shapes every skinny tile (the few-rows ones at each
    K-slice count)."""
    out = [(sg.VARIANT_AUTO, -1, 0, sg.FLAG_UNTUNED)]
    for tile in range(sg.tile_count(sg.VARIANT_MFMA)):
        groups = GROUPS if sweep_groups else (0,)
        for g in groups:
            out.append((sg.VARIANT_MFMA, tile, g, 0))
        if sg.tile_info(sg.VARIANT_MFMA, tile)["flags"] & sg.TILE_STREAMK:
            out.append((sg.VARIANT_MFMA, tile, 0, sg.FLAG_STREAMK))
    for tile in range(sg.tile_count(sg.VARIANT_VALU)):
        out.append((sg.VARIANT_VALU, tile, 0, 0))
    for tile in range(sg.tile_count(sg.VARIANT_SMALL)):
        out.append((sg.VARIANT_SMALL, tile, 0, 0))
    if M <= 16 or N <= 16:
        for tile in range(sg.tile_count(sg.VARIANT_SKINNY)):
            rows_kind = sg.tile_info(sg.VARIANT_SKINNY, tile)["tm"] == 0
            for g in (SLICES if rows_kind else (0,)):
                out.append((sg.VARIANT_SKINNY, tile, g, 0))
    return out


def agree(torch, C, ref, K, amax, bmax) -> bool:
    tol = 2e-5 * K * amax * bmax
    return bool(torch.isfinite(C).all()) and float((C - ref).abs().max()) <= tol


def time_graph(torch, call_i, calls: int, replays: int = 5):
    """Device time per call (ms) with no host gaps: `calls` consecutive calls
    call_i(0), call_i(1), ... captured in one HIP graph on a side stream, the
    graph replayed `replays` times; returns one per-call time per replay.
    The library's launches go to torch's current stream, which inside the
    capture is the capture stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(calls, 3)):
            call_i(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            call_i(i)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(replays):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / calls)
    del g
    return out


def tune_shape(sg, torch, M, N, K, warmup, reps, sweep_groups, seed=0, rotate=False,
               graph=False):
    """Time every candidate on (M, N, K).  With `rotate`, consecutive timed
    calls use different copies of A and B whose total exceeds the 256 MB
    Infinity Cache, so memory-bound shapes read their operands from HBM."""
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    per_set = 4 * (M * K + K * N)
    copies = max(2, -(-2 * 256 * 1024 * 1024 // per_set) + 1) if rotate else 1
    As = [torch.rand((M, K), device=dev, generator=gen) * 2 - 1 for _ in range(copies)]
    Bs = [torch.rand((K, N), device=dev, generator=gen) * 2 - 1 for _ in range(copies)]
    A, B = As[0], Bs[0]
    C = torch.empty((M, N), device=dev)
    ref = torch.empty((M, N), device=dev)
    sg.gemm(A, B, ref)
    torch.cuda.synchronize()
    # bring the clock back up after the host-side set-up before the first
    # (automatic) candidate is timed: ~20 ms of the product itself
    warm = max(1, int(0.02 / max(2.0 * M * N * K / 100e12, 5e-6)))
    for _ in range(min(warm, 4000)):
        sg.gemm(A, B, C)
    torch.cuda.synchronize()
    results = []
    for variant, tile, group, flags in candidates(sg, M, N, K, sweep_groups):
        try:
            call = lambda: sg.gemm(A, B, C, variant=variant, tile=tile, group_m=group, flags=flags)
            C.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
        except sg.SgemmError:
            continue                      # configuration does not apply to this shape
        if not agree(torch, C, ref, K, 1.0, 1.0):
            print(f"  rejected v{variant} t{tile} g{group}: output differs", flush=True)
            continue
        kw = dict(variant=variant, tile=tile, group_m=group, flags=flags)
        call_i = lambda i, kw=kw: sg.gemm(As[i % copies], Bs[i % copies], C, **kw)
        call_n = lambda i, kw=kw: sg.gemm(As[i % copies], Bs[i % copies], C, noalloc=True, **kw)
        timing = "eager"
        alloc_ms = None
        if graph:
            try:
                call_n(0)
                fits = True
            except sg.SgemmError as ex:
                if ex.status != -31:
                    raise
                fits = False   # partial sums beyond the static scratch: time eagerly
            if fits:
                ms = statistics.median(time_graph(torch, call_n, max(reps, copies)))
                timing = "graph, no allocation"
                if keeps_partial_sums(sg, M, N, K, variant, tile, group, flags):
                    alloc_ms = round(statistics.median(
                        time_graph(torch, call_i, max(reps, copies))), 5)
        if timing == "eager":
            for i in range(warmup):
                call_i(i)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for i, (s, e) in enumerate(ev):
                s.record()
                call_i(warmup + i)
                e.record()
            torch.cuda.synchronize()
            ms = statistics.median(s.elapsed_time(e) for s, e in ev)
        gf = 2.0 * M * N * K / (ms / 1e3) / 1e9
        if variant == sg.VARIANT_AUTO:
            main, rows, cols = sg.plan(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)
            desc = {"model": True, "variant": main.variant, "tile": main.tile,
                    "edge_rows": rows, "edge_cols": cols}
        else:
            desc = sg.tile_info(variant, tile)
        results.append({"variant": variant, "tile": tile, "group_m": group, "flags": flags,
                        "ms": round(ms, 5), "gflops": round(gf, 1), "timing": timing,
                        "graph_with_alloc_ms": alloc_ms, "desc": desc})
        print(f"  v{variant} t{tile} g{group} f{flags}: {ms:.4f} ms  {gf:,.0f} GFLOP/s", flush=True)
    results.sort(key=lambda r: r["ms"])
    return results


def keeps_partial_sums(sg, M, N, K, variant, tile, group, flags) -> bool:
    """Whether a candidate's plan keeps partial sums in device memory: a
    stream-K launch, or a few-rows skinny launch split over K (the automatic
    plan as sgemm_plan reports it)."""
    if flags & sg.FLAG_STREAMK:
        return True
    if variant == sg.VARIANT_AUTO:
        cfg, rows, _ = sg.plan(M, N, K)
        return bool(cfg.flags & sg.FLAG_STREAMK or rows or
                    (cfg.variant == sg.VARIANT_SKINNY and cfg.group_m > 1))
    return (variant == sg.VARIANT_SKINNY and sg.tile_info(variant, tile)["tm"] == 0 and
            group != 1)


PEAK_16BIT_GFLOPS = 2.5e6   # MI355X dense bf16 / fp16 matrix peak


def tune_mixed(sg, torch, M, N, K, dtype: str, reps: int, seed: int = 0):
    """Every 16-bit-input configuration (sgemm_mixed with W stored N x K: the
    automatic choice, each 16-bit MFMA tile, the generic kernel) on
    (M, N, K), graph-replayed; `eff_pct` is the percent of the 16-bit matrix
    peak, the figure the 16-bit tile table's cost model uses."""
    dev = "cuda:0"
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    A = (torch.rand((M, K), device=dev, generator=gen) * 2 - 1).to(dt)
    W = (torch.rand((N, K), device=dev, generator=gen) * 2 - 1).to(dt)
    C = torch.empty((M, N), device=dev)
    ref = torch.empty((M, N), device=dev)
    sg.gemm_mixed(A, W, ref, trans_b=True)
    torch.cuda.synchronize()
    cands = [(sg.VARIANT_AUTO, -1)] + [(sg.VARIANT_MFMA16, t)
                                       for t in range(sg.tile_count(sg.VARIANT_MFMA16))]
    cands.append((sg.VARIANT_GENERIC16, 0))
    results = []
    for variant, tile in cands:
        kw = {} if variant == sg.VARIANT_AUTO else dict(variant=variant, tile=tile)
        try:
            C.fill_(float("nan"))
            sg.gemm_mixed(A, W, C, trans_b=True, **kw)
            torch.cuda.synchronize()
        except sg.SgemmError:
            continue
        if not agree(torch, C, ref, K, 1.0, 1.0):
            print(f"  rejected v{variant} t{tile}: output differs", flush=True)
            continue
        call_i = lambda i, kw=kw: sg.gemm_mixed(A, W, C, trans_b=True, **kw)
        # the first timing of a process runs slower (clock and power ramp):
        # one untimed graph replay first
        time_graph(torch, call_i, reps, replays=1)
        ms = statistics.median(time_graph(torch, call_i, reps))
        gf = 2.0 * M * N * K / (ms / 1e3) / 1e9
        results.append({"variant": variant, "tile": tile, "inputs": dtype, "ms": round(ms, 5),
                        "gflops": round(gf, 1), "eff_pct": round(100 * gf / PEAK_16BIT_GFLOPS, 1),
                        "desc": (sg.tile_info(variant, tile) if variant == sg.VARIANT_MFMA16
                                 else {})})
        print(f"  v{variant} t{tile}: {ms:.4f} ms  {gf:,.0f} GFLOP/s  "
              f"{100 * gf / PEAK_16BIT_GFLOPS:.1f} %", flush=True)
    results.sort(key=lambda r: r["ms"])
    return results


def read_table(path: str = TABLE) -> dict:
    """The rows of an existing table, {(M, N, K): {variant, tile, group_m, gflops}}."""
    import re

    rows = {}
    if not os.path.exists(path):
        return rows
    pat = re.compile(r"\{(\d+), (\d+), (\d+), \{(\d+), (\d+), (\d+)\}\},\s*// ([\d,.]+) GFLOP/s")
    for line in open(path):
        m = pat.search(line)
        if m and int(m.group(1)) > 0:
            M, N, K, v, t, g = (int(m.group(i)) for i in range(1, 7))
            rows[(M, N, K)] = {"variant": v, "tile": t, "group_m": g,
                               "gflops": float(m.group(7).replace(",", ""))}
    return rows


def write_table(best: dict, path: str = TABLE, merge: bool = True):
    """Rewrite the table with `best`; rows for other shapes are kept when `merge`.
    A shape whose best candidate is the untuned automatic plan (variant 0)
    gets no row, and loses any row it had."""
    if merge:
        best = {**read_table(path), **best}
    best = {k: v for k, v in best.items() if v["variant"] != 0}
    rows = []
    for (M, N, K), r in sorted(best.items()):
        rows.append(f"    {{{M}, {N}, {K}, {{{r['variant']}, {r['tile']}, {r['group_m']}}}}},"
                    f"   // {r['gflops']:,.0f} GFLOP/s")
    text = f"""// tuned_table.inc -- measured best configurations per shape (written by
// fp32_sgemm_02_amd/tune.py; edit by re-running it).  Each row: the exact
// (M, N, K) it was tuned on, then variant, tile, group_m.  Shapes not listed
// fall back to the tile-count rule in auto_select().
static const struct {{ int M, N, K; Tuned t; }} kTuned[] = {{
    {{0, 0, 0, {{0, 0, 0}}}},   // sentinel (never matches: M == 0 returns early)
{chr(10).join(rows)}
}};

static bool lookup_tuned(int M, int N, int K, Tuned &out) {{
    for (const auto &e : kTuned)
        if (e.M == M && e.N == N && e.K == K) {{ out = e.t; return true; }}
    return false;
}}
"""
    with open(path, "w") as fh:
        fh.write(text)


def main():
    sys.path.insert(0, ROOT)
    import torch

    import fp32_sgemm_02_amd as sg
    import workloads

    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="")
    ap.add_argument("--shapes", default="")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--groups", action="store_true", help="also sweep group_m")
    ap.add_argument("--rotate", action="store_true",
                    help="rotate over operand copies larger than the 256 MB Infinity Cache "
                         "(memory-bound shapes)")
    ap.add_argument("--graph", action="store_true",
                    help="time calls replayed from a HIP graph (no host launch gaps; for "
                         "shapes whose kernels are shorter than the host launch path)")
    ap.add_argument("--mixed", choices=["bf16", "f16"], default=None,
                    help="time the 16-bit-input tiles (sgemm_mixed, W stored N x K) instead")
    ap.add_argument("--out", default=None)
    ap.add_argument("--write-table", action="store_true")
    ap.add_argument("--from-json", default=None,
                    help="write the table from a saved --out report instead of timing")
    args = ap.parse_args()
    if args.from_json:
        report = json.load(open(args.from_json))
        best = {parse_shape(k): v[0] for k, v in report.items() if v}
        write_table(best)
        for k, r in sorted(best.items()):
            print(k, r["variant"], r["tile"], r["group_m"], r["gflops"])
        return

    shapes = []
    for name in filter(None, args.workloads.split(",")):
        w = workloads.WORKLOADS[name]
        shapes.append((w.M, w.N, w.K))
    shapes += [parse_shape(s) for s in filter(None, args.shapes.split(","))]
    torch.cuda.set_device(0)
    report, best = {}, {}
    for (M, N, K) in shapes:
        print(f"shape {M}x{N}x{K}", flush=True)
        if args.mixed:
            report[f"{M}x{N}x{K}"] = tune_mixed(sg, torch, M, N, K, args.mixed, args.reps)
            torch.cuda.empty_cache()
            continue
        res = tune_shape(sg, torch, M, N, K, args.warmup, args.reps, args.groups,
                         rotate=args.rotate, graph=args.graph)
        report[f"{M}x{N}x{K}"] = res
        if res:
            best[(M, N, K)] = res[0]
            print(f"  best: v{res[0]['variant']} t{res[0]['tile']} g{res[0]['group_m']} "
                  f"{res[0]['gflops']:,.0f} GFLOP/s", flush=True)
        torch.cuda.empty_cache()
    if args.out:
        with open(args.out, "w") as fh:
            json.dump(report, fh, indent=1)
    if args.write_table and not args.mixed:
        write_table(best)


if __name__ == "__main__":
    main()
