"""GPU parity of the fused bias/activation epilogue (sgemm_epilogue) against
the CPU oracle's epilogue entry point.

Every test is marked ``gpu``.  Floating-point inputs are held to
parity.epilogue_err_ratio's tolerance; integer inputs with ReLU or no
activation and an integer bias must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
import workloads
from parity import epilogue_err_ratio, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"
ACTS = [sg.ACT_NONE, sg.ACT_RELU, sg.ACT_SILU, sg.ACT_GELU_ERF, sg.ACT_GELU_TANH]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run_gpu(As, Bs, C0, alpha, beta, bias, act, trans_a=False, trans_b=False, **kw):
    M = As.shape[1] if trans_a else As.shape[0]
    N = Bs.shape[0] if trans_b else Bs.shape[1]
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(As), dev(Bs), C, alpha, beta, trans_a=trans_a, trans_b=trans_b,
            bias=None if bias is None else dev(bias), act=act, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check(As, Bs, C0, alpha, beta, bias, act, C, oracle_mod, trans_a=False, trans_b=False,
          exact=False, label="", rows=None):
    if rows is not None:
        As = np.ascontiguousarray(As[:, rows] if trans_a else As[rows])
        C0 = None if C0 is None else np.ascontiguousarray(C0[rows])
        C = C[rows]
    b0 = beta if C0 is not None else 0.0
    ref = oracle_mod.sgemm(As, Bs, None if C0 is None else C0.copy(), alpha, b0,
                           trans_a=trans_a, trans_b=trans_b, bias=bias, act=act)
    if exact:
        assert np.array_equal(C, ref), f"{label}: not bit-exact"
        return 0.0
    x = oracle_mod.sgemm(As, Bs, None if C0 is None else C0.copy(), alpha, b0, trans_a=trans_a,
                         trans_b=trans_b, bias=bias, act=sg.ACT_NONE)
    K = As.shape[0] if trans_a else As.shape[1]
    r = epilogue_err_ratio(C, ref, x, K, alpha, b0, As, Bs, C0, bias, act)
    assert r <= 1.0, f"{label}: max err/tol = {r}"
    return r


SHAPES = [(300, 520, 77), (256, 256, 64), (1000, 300, 5), (129, 1031, 200), (16, 700, 300),
          (700, 9, 300), (1, 1, 1)]


@pytest.mark.parametrize("act", ACTS)
def test_epilogue_automatic(act, oracle_mod):
    """Automatic dispatch (direct-load tiles, skinny shapes, ragged edges)
    with and without bias, beta = 0 over NaN and alpha/beta, and both
    transpositions of B."""
    rng = np.random.default_rng(act)
    for i, (M, N, K) in enumerate(SHAPES):
        A, B, C0 = workloads.draw(M, N, K, "uniform", 2000 + i, True)
        bias = rng.uniform(-1, 1, N).astype(F32)
        for tb in (False, True):
            Bs = np.ascontiguousarray(B.T) if tb else B
            lab = f"act {act} {(M, N, K)} tb={tb}"
            C = run_gpu(A, Bs, C0, 0.5, -1.25, bias, act, trans_b=tb)
            check(A, Bs, C0, 0.5, -1.25, bias, act, C, oracle_mod, trans_b=tb, label=lab)
            C = run_gpu(A, Bs, None, 1.0, 0.0, None if tb else bias, act, trans_b=tb)
            check(A, Bs, None, 1.0, 0.0, None if tb else bias, act, C, oracle_mod, trans_b=tb,
                  label=lab + " b0")


@pytest.mark.parametrize("act", [sg.ACT_NONE, sg.ACT_RELU])
def test_epilogue_integer_bit_exact(act, oracle_mod):
    """Integer inputs and bias: every partial sum, the bias add and ReLU are
    exact, so every kernel path must give the oracle's bits."""
    rng = np.random.default_rng(7)
    for i, (M, N, K) in enumerate(SHAPES):
        A, B, C0 = workloads.draw(M, N, K, "int4", 2100 + i, True)
        bias = rng.integers(-64, 65, N).astype(F32)
        for ta in (False, True):
            As = np.ascontiguousarray(A.T) if ta else A
            C = run_gpu(As, B, C0, 0.5, -1.25, bias, act, trans_a=ta)
            check(As, B, C0, 0.5, -1.25, bias, act, C, oracle_mod, trans_a=ta, exact=True,
                  label=f"int act {act} {(M, N, K)} ta={ta}")


def _configs():
    out = [(sg.VARIANT_VALU, 0), (sg.VARIANT_MFMA, 0), (sg.VARIANT_MFMA, 5)]
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        f = sg.tile_info(sg.VARIANT_MFMA, t)["flags"]
        if f & sg.TILE_DIRECT and not f & (sg.TILE_WHOLE | sg.TILE_TRANS_A):
            out.append((sg.VARIANT_MFMA, t))
    return out


@pytest.mark.parametrize("act", [sg.ACT_SILU, sg.ACT_GELU_ERF])
def test_epilogue_every_family(act, oracle_mod):
    """Explicit configurations: the VALU family and the general MFMA tiles
    (stored product plus an elementwise pass), every direct-load tile with
    edges (fused), the skinny family, and 4-byte I/O."""
    rng = np.random.default_rng(11)
    M, N, K = 300, 520, 77
    A, B, C0 = workloads.draw(M, N, K, "uniform", 2200, True)
    bias = rng.uniform(-1, 1, N).astype(F32)
    for variant, tile in _configs():
        for flags in (0, sg.FLAG_SCALAR_IO):
            kw = dict(variant=variant, tile=tile, flags=flags)
            C = run_gpu(A, B, C0, 0.5, -1.25, bias, act, **kw)
            check(A, B, C0, 0.5, -1.25, bias, act, C, oracle_mod,
                  label=f"v{variant} t{tile} f{flags} act {act}")
    for M, N in ((7, 700), (700, 7)):
        A, B, C0 = workloads.draw(M, N, K, "uniform", 2300, True)
        bias = rng.uniform(-1, 1, N).astype(F32)
        C = run_gpu(A, B, C0, 0.5, -1.25, bias, act, variant=sg.VARIANT_SKINNY)
        check(A, B, C0, 0.5, -1.25, bias, act, C, oracle_mod, label=f"skinny {(M, N)}")


def test_epilogue_special_cases(oracle_mod):
    """alpha == 0 and K == 0 give act(beta C + bias) without reading A or B
    (NaN-poisoned); beta == 0 never reads C; beta == 1 with an epilogue is
    not a no-op."""
    rng = np.random.default_rng(3)
    M, N, K = 77, 130, 40
    C0 = rng.uniform(-2, 2, (M, N)).astype(F32)
    bias = rng.uniform(-1, 1, N).astype(F32)
    An = np.full((M, K), np.nan, F32)
    Bn = np.full((K, N), np.nan, F32)
    for act in ACTS:
        for beta in (0.0, 1.0, -0.5):
            C = run_gpu(An, Bn, C0, 0.0, beta, bias, act)
            check(An, Bn, C0, 0.0, beta, bias, act, C, oracle_mod, label=f"alpha0 {act} {beta}")
        Cz = torch.full((M, N), float("nan"), device=DEV)
        sg.gemm(torch.empty((M, 0), device=DEV), torch.empty((0, N), device=DEV), Cz, 1.0, 0.0,
                bias=dev(bias), act=act)
        torch.cuda.synchronize()
        check(np.zeros((M, 0), F32), np.zeros((0, N), F32), None, 1.0, 0.0, bias, act,
              Cz.cpu().numpy(), oracle_mod, exact=act in (sg.ACT_NONE, sg.ACT_RELU),
              label=f"K == 0 act {act}")


@pytest.mark.parametrize("name,act,tb", [("mlp_up", sg.ACT_SILU, True),
                                         ("mlp_up", sg.ACT_GELU_TANH, False),
                                         ("mlp_decode16", sg.ACT_GELU_ERF, True),
                                         ("mlp_down", sg.ACT_NONE, True)])
def test_epilogue_mlp_full_size(name, act, tb, oracle_mod):
    """The feed-forward shapes at full size (bias and activation as a linear
    layer applies them; B as the layer's weight, N x K, when tb), sampled
    rows against the oracle."""
    w = workloads.WORKLOADS[name]
    A, B, _ = workloads.inputs(w)
    bias = np.random.default_rng(5).uniform(-1, 1, w.N).astype(F32)
    Bs = np.ascontiguousarray(B.T) if tb else B
    C = run_gpu(A, Bs, None, 1.0, 0.0, bias, act, trans_b=tb)
    rows = sample_rows(w.M, 16)
    check(A, Bs, None, 1.0, 0.0, bias, act, C, oracle_mod, trans_b=tb, rows=rows,
          label=f"{name} act {act}")
