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


def candidates(sg, M, N, K, sweep_groups: bool):
    """(variant, tile, group_m, flags) to time.  The first is the automatic
    plan without the tuned table (the cost model, edge strips included); when
    it wins, the shape needs no table row."""
    out = [(sg.VARIANT_AUTO, -1, 0, sg.FLAG_UNTUNED)]
    for tile in range(sg.tile_count(sg.VARIANT_MFMA)):
        groups = GROUPS if sweep_groups else (0,)
        for g in groups:
            out.append((sg.VARIANT_MFMA, tile, g, 0))
    if M <= 16 or N <= 16:
        for tile in range(sg.tile_count(sg.VARIANT_SKINNY)):
            out.append((sg.VARIANT_SKINNY, tile, 0, 0))
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
        call_i = lambda i: sg.gemm(As[i % copies], Bs[i % copies], C, variant=variant, tile=tile,
                                   group_m=group, flags=flags)
        if graph:
            ms = statistics.median(time_graph(torch, call_i, max(reps, copies)))
        else:
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
                        "ms": round(ms, 5), "gflops": round(gf, 1), "desc": desc})
        print(f"  v{variant} t{tile} g{group} f{flags}: {ms:.4f} ms  {gf:,.0f} GFLOP/s", flush=True)
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
    if args.write_table:
        write_table(best)


if __name__ == "__main__":
    main()
