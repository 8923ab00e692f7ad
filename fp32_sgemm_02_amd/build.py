"""Build libfp32sgemm.so (gfx950) from csrc/ with hipcc, in-tree.

    python -m fp32_sgemm_02_amd.build            # build
    python -m fp32_sgemm_02_amd.build --resources  # also print VGPR/AGPR/LDS/spill use

Every HIP source is compiled for gfx950 only, with packed fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
one shared library next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp32sgemm.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "workspace.cpp", "scale.hip", "mfma_gemm.hip", "mfma_direct.hip", "mfma_direct_epi.hip",
           "mfma_direct_sk.hip",
           "mfma_direct_ta.hip", "mfma_direct_ta_epi.hip", "mfma_gemm16.hip", "valu_gemm.hip",
           "skinny_gemm.hip", "small_gemm.hip"]
PROBE_SOURCES = ["peak_probes.hip"]
PROBE_LIB = os.path.join(HERE, "libfp32probes.so")

COMMON_FLAGS = [
    "-x", "hip", "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, resources: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if resources:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(resources: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libfp32sgemm.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    allsrc = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(allsrc), max(1, (os.cpu_count() or 2) - 1), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = dict(zip(allsrc, ex.map(lambda s: _compile(s, resources), allsrc)))
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        objs = [results[s][0] for s in srcs]
        tmp = lib + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
    if resources:
        for (_, log) in results.values():
            for line in summarize_resources(log):
                print(line)
    return LIB


def summarize_resources(log: str) -> list[str]:
    """One line per kernel from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = [], {}
    for line in log.splitlines():
        m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)", line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            if cur:
                out.append(cur)
            cur = {"name": val}
        else:
            cur[key] = val
    if cur:
        out.append(cur)
    lines = []
    for k in out:
        lines.append(f"{k.get('name')[:90]:90s} vgpr={k.get('VGPRs')} agpr={k.get('AGPRs')} "
                     f"spill={k.get('VGPRs Spill')} scratch={k.get('ScratchSize [bytes/lane]')} "
                     f"occ={k.get('Occupancy [waves/SIMD]')} lds={k.get('LDS Size [bytes/block]')}")
    return lines


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--resources", action="store_true")
    args = ap.parse_args()
    print(build(resources=args.resources))
    sys.exit(0)
