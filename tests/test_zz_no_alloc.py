"""sgemm_op_ex_noalloc: the entry point for callers that cannot allocate.

Its plans keep partial sums in the library's static scratch array instead of
a workspace, so its results must equal sgemm_op_ex's (same kernels, same
split, same summation order: bit for bit) and the oracle's (tolerance;
integer inputs bit-exact).  Consecutive calls reuse the array (the second
call here is smaller than the first), graph replays reuse it, and a plan
whose partial sums exceed it is refused before anything runs.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import fp32_sgemm_02_amd as sg
import workloads
from parity import max_err_ratio

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32 = np.float32
SCRATCH_BYTES = 16 << 20


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def call(entry, ta, tb, M, N, K, alpha, A, B, beta, C, cfg=None):
    """One raw C-ABI call (entry: sg.sgemm_op or sg.sgemm_op_noalloc)."""
    stream = torch.cuda.current_stream().cuda_stream
    return entry(int(ta), int(tb), M, N, K, alpha, A.data_ptr(), A.stride(0), B.data_ptr(),
                 B.stride(0), beta, C.data_ptr(), C.stride(0), stream, cfg=cfg)


def stored(A, B, ta, tb):
    return (np.ascontiguousarray(A.T) if ta else A), (np.ascontiguousarray(B.T) if tb else B)


# (M, N, K, trans_a, trans_b, config or None, inputs, seed); consecutive pairs
# run back to back, the second smaller than the first
CASES = [
    ((1, 4096, 4096, False, False, None, "uniform", 11),
     (3, 1000, 3001, False, False, None, "uniform", 12)),
    ((2, 2048, 8192, False, False, (sg.VARIANT_SKINNY, 3, 0, 16), "int4", 13),
     (1, 300, 1000, False, False, (sg.VARIANT_SKINNY, 3, 0, 5), "int4", 14)),
    ((16, 14336, 4096, False, True, None, "uniform", 15),
     (5, 700, 1024, True, False, None, "uniform", 16)),
    ((300, 520, 777, False, False, None, "uniform", 17),
     (64, 64, 16, False, False, None, "int4", 18)),
]


def run_pair(pair, oracle_mod):
    for M, N, K, ta, tb, cfgt, dist, seed in pair:
        lab = f"{(M, N, K)} ta={ta} tb={tb} cfg={cfgt}"
        print(lab, flush=True)
        A, B, C0 = workloads.draw(M, N, K, dist, seed, True)
        As, Bs = stored(A, B, ta, tb)
        cfg = sg.SgemmConfig(*cfgt) if cfgt else None
        dA, dB = dev(As), dev(Bs)
        C_ref, C_na = dev(C0), dev(C0)
        assert call(sg.sgemm_op, ta, tb, M, N, K, 0.5, dA, dB, -1.25, C_ref, cfg) == 0, lab
        st = call(sg.sgemm_op_noalloc, ta, tb, M, N, K, 0.5, dA, dB, -1.25, C_na, cfg)
        assert st == 0, f"{lab}: {sg.status_string(st)}"
        torch.cuda.synchronize()
        got, want = C_na.cpu().numpy(), C_ref.cpu().numpy()
        assert np.array_equal(got, want), f"{lab}: differs from sgemm_op_ex"
        ref = oracle_mod.sgemm(As, Bs, C0.copy(), 0.5, -1.25, trans_a=ta, trans_b=tb)
        if dist == "int4":
            assert np.array_equal(got, ref), f"{lab}: integer inputs not bit-exact"
        else:
            r = max_err_ratio(got, ref, K, 0.5, -1.25, As, Bs, C0)
            assert r <= 1.0, f"{lab}: max err/tol {r}"


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_matches_sgemm_op(pair, oracle_mod):
    run_pair(CASES[pair], oracle_mod)


def test_noalloc_split_plan_uses_scratch():
    """The automatic plan of 1 x 4096 x 4096 is split over K (partial sums),
    so the calls above went through the static scratch."""
    cfg, _, _ = sg.plan(1, 4096, 4096)
    assert cfg.variant == sg.VARIANT_SKINNY and cfg.group_m > 1


def test_noalloc_graph_replays(oracle_mod):
    """Captured in a HIP graph (no allocation nodes: the scratch is static),
    replayed several times with eager calls in between, each replay equal to
    the eager result."""
    M, N, K = 4, 1024, 8192
    A, B, C0 = workloads.draw(M, N, K, "int4", 19, True)
    dA, dB = dev(A), dev(B)
    want = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
    C = dev(C0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert call(sg.sgemm_op_noalloc, 0, 0, M, N, K, 0.5, dA, dB, -1.25, C) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    C0d = dev(C0)
    with torch.cuda.graph(g):
        C.copy_(C0d)
        assert call(sg.sgemm_op_noalloc, 0, 0, M, N, K, 0.5, dA, dB, -1.25, C) == 0
    other = dev(C0)
    for r in range(4):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), want), f"replay {r}"
        # eager work on the same scratch between replays
        other.copy_(C0d)
        assert call(sg.sgemm_op_noalloc, 0, 0, M, N, K, 0.5, dA, dB, -1.25, other) == 0
        torch.cuda.synchronize()
        assert np.array_equal(other.cpu().numpy(), want), f"eager call after replay {r}"
    del g


def test_noalloc_refuses_plans_beyond_the_scratch():
    """An explicit stream-K configuration keeps 64 MiB or more of partial
    sums: refused with -31 before any launch (C untouched)."""
    tiles = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
             if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_STREAMK
             and not sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_TRANS_A]
    assert tiles
    M, N, K = 512, 512, 8192
    rng = np.random.default_rng(20)
    dA = dev(rng.uniform(-1, 1, (M, K)).astype(F32))
    dB = dev(rng.uniform(-1, 1, (K, N)).astype(F32))
    C = torch.full((M, N), 7.0, device=DEV)
    cfg = sg.SgemmConfig(sg.VARIANT_MFMA, tiles[0], sg.FLAG_STREAMK, 0)
    st = call(sg.sgemm_op_noalloc, 0, 0, M, N, K, 1.0, dA, dB, 0.0, C, cfg)
    assert st == -31, sg.status_string(st)
    assert "static scratch" in sg.status_string(st)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
    # the same explicit plan through sgemm_op_ex allocates and runs
    assert call(sg.sgemm_op, 0, 0, M, N, K, 1.0, dA, dB, 0.0, C, cfg) == 0
    # a split asking for more slices than fit: 16 rows x 65536 columns x 64
    # slices = 256 MiB of partial sums
    M2, N2, K2 = 16, 65536, 4096
    A2 = torch.zeros((M2, K2), device=DEV)
    B2 = torch.zeros((K2, N2), device=DEV)
    C2 = torch.full((M2, N2), 3.0, device=DEV)
    cfg2 = sg.SgemmConfig(sg.VARIANT_SKINNY, 2, 0, 64)
    assert 64 * M2 * N2 * 4 > SCRATCH_BYTES
    st = call(sg.sgemm_op_noalloc, 0, 0, M2, N2, K2, 1.0, A2, B2, 0.0, C2, cfg2)
    torch.cuda.synchronize()
    # 1024 strips of 64 columns: within the 4096 counters, so the split is real
    assert st == -31, sg.status_string(st)
    assert bool((C2 == 3.0).all())
