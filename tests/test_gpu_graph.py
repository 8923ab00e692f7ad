"""The library's launches inside a captured HIP graph.

The benchmark's sweep times small shapes by replaying captured calls, so the
calls must behave identically when replayed: every replay, with the
program's own eager work and synchronisations in between, must reproduce the
eager result bit for bit (the kernels are deterministic).
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def test_graph_replays_match_eager():
    whole = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
             if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_WHOLE][0]
    cases = [  # (M, N, K, alpha, beta, gemm kwargs)
        (512, 512, 64, 1.0, 0.0, dict(variant=sg.VARIANT_MFMA, tile=whole)),
        (300, 257, 129, 0.5, -1.25, {}),
        (1, 1000, 300, 1.0, 0.5, {}),
        (1000, 3, 300, 2.0, 0.0, {}),
        (70, 90, 30, 0.0, 0.5, {}),          # alpha = 0: the beta-scale kernel
    ]
    ops = []
    for i, (M, N, K, alpha, beta, kw) in enumerate(cases):
        A, B, C0 = workloads.draw(M, N, K, "uniform", 900 + i, True)
        ops.append((_dev(A), _dev(B), _dev(C0), torch.empty((M, N), device=DEV), alpha, beta, kw))

    def run_all():
        for A, B, C0, C, alpha, beta, kw in ops:
            C.copy_(C0)
            sg.gemm(A, B, C, alpha, beta, **kw)

    run_all()
    torch.cuda.synchronize()
    eager = [op[3].clone() for op in ops]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for rep in range(3):
        for op in ops:
            op[3].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (op, ref) in enumerate(zip(ops, eager)):
            assert torch.equal(op[3], ref), f"replay {rep}, case {cases[i][:5]}"
        # the program's own eager work between replays
        x = torch.randn(1000, device=DEV)
        float((x * x).sum())



def test_graph_edge_strips(oracle_mod):
    """A plan with edge strips (4097 x 1000 x 301: the last row by the skinny
    family in a second launch) captured in a graph: every replay, with eager work between replays, reproduces the
    eager result, which matches the oracle bit for bit (integer inputs)."""
    M, N, K = 4097, 1000, 301
    A, B, C0 = workloads.draw(M, N, K, "int4", 960, True)
    dA, dB, dC0 = _dev(A), _dev(B), _dev(C0)
    assert sg.plan(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC0.data_ptr(), N)[1] == 1
    ref = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
    C = dC0.clone()
    sg.gemm(dA, dB, C, 0.5, -1.25)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref), "eager"
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        C.copy_(dC0)
        sg.gemm(dA, dB, C, 0.5, -1.25)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        C.copy_(dC0)
        sg.gemm(dA, dB, C, 0.5, -1.25)
    for rep in range(3):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), ref), f"replay {rep}"
        x = torch.randn(1000, device=DEV)
        float((x * x).sum())
    del g
