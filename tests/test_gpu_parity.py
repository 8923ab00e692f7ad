"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every test here is marked ``gpu`` and needs an MI355X.  Shapes span several
tiles with ragged tails; the full-size workloads are checked on sampled rows
that the oracle computes one by one.  Floating-point inputs are held to the
tolerance in parity.py; integer-valued inputs must match bit for bit.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
import workloads
from parity import epilogue_err_ratio, max_err_ratio, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def run_gpu(A, B, C0, alpha, beta, **kw):
    """C on the GPU through the C ABI; C0 None means a NaN-poisoned C (beta must be 0)."""
    M, N = A.shape[0], B.shape[1]
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(A), dev(B), C, alpha, beta, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check(A, B, C0, alpha, beta, C, oracle_mod, rows=None, exact=False, label=""):
    if rows is not None:
        ref = oracle_mod.sgemm(np.ascontiguousarray(A[rows]), B,
                               None if C0 is None else np.ascontiguousarray(C0[rows]),
                               alpha, beta if C0 is not None else 0.0)
        got = C[rows]
        c0 = None if C0 is None else C0[rows]
    else:
        ref = oracle_mod.sgemm(A, B, None if C0 is None else C0.copy(), alpha,
                               beta if C0 is not None else 0.0)
        got, c0 = C, C0
    if exact:
        assert np.array_equal(got, ref), f"{label}: not bit-exact " \
            f"(max diff {np.nanmax(np.abs(got - ref))})"
        return 0.0
    r = max_err_ratio(got, ref, A.shape[1], alpha, beta, A, B, c0)
    assert r <= 1.0, f"{label}: max err/tol = {r}"
    return r


def tiles(variant):
    return list(range(sg.tile_count(variant)))


def uniform(M, N, K, seed, with_c=True):
    return workloads.draw(M, N, K, "uniform", seed, with_c)


# ---------------------------------------------------------------- per tile --
SMALL_SHAPES = [(300, 520, 77), (257, 129, 33), (64, 64, 16), (1000, 300, 5), (129, 1031, 200)]


@pytest.mark.parametrize("variant,tile", [(sg.VARIANT_MFMA, t) for t in range(8)] +
                         [(sg.VARIANT_VALU, t) for t in range(3)])
def test_tile_parity_ragged(variant, tile, oracle_mod):
    if tile >= sg.tile_count(variant):
        pytest.skip("tile not compiled")
    for i, (M, N, K) in enumerate(SMALL_SHAPES):
        A, B, C0 = uniform(M, N, K, 100 + i)
        C = run_gpu(A, B, C0, 0.5, -1.25, variant=variant, tile=tile)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, label=f"v{variant} t{tile} {(M, N, K)}")
        C = run_gpu(A, B, None, 1.0, 0.0, variant=variant, tile=tile)
        check(A, B, None, 1.0, 0.0, C, oracle_mod, label=f"v{variant} t{tile} {(M, N, K)} b0")


@pytest.mark.parametrize("variant,tile", [(sg.VARIANT_MFMA, t) for t in range(8)] +
                         [(sg.VARIANT_VALU, t) for t in range(3)])
def test_tile_integer_bit_exact(variant, tile, oracle_mod):
    if tile >= sg.tile_count(variant):
        pytest.skip("tile not compiled")
    A, B, C0 = workloads.draw(333, 271, 1001, "int4", 7, True)
    C = run_gpu(A, B, C0, 0.5, -1.25, variant=variant, tile=tile)
    check(A, B, C0, 0.5, -1.25, C, oracle_mod, exact=True, label=f"v{variant} t{tile} int")
    # the scalar (4-byte) I/O path of the same tile
    C = run_gpu(A, B, C0, 0.5, -1.25, variant=variant, tile=tile, flags=sg.FLAG_SCALAR_IO)
    check(A, B, C0, 0.5, -1.25, C, oracle_mod, exact=True, label=f"v{variant} t{tile} int scalar")


# ------------------------------------------------------ whole-tile MFMA --
def whole_tiles():
    return [t for t in tiles(sg.VARIANT_MFMA)
            if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_WHOLE]


@pytest.mark.parametrize("slot", range(12))
def test_whole_tile_parity(slot, oracle_mod):
    """Direct-load tiles on shapes made of whole tiles: 1, 2, 3, 5 and 17
    K-steps (fewer than the LDS ring, odd and even counts, many), alpha/beta,
    beta = 0 over a NaN C, integer inputs bit-exact, and padded rows."""
    wt = whole_tiles()
    if slot >= len(wt):
        pytest.skip("no such whole-tile configuration")
    tile = wt[slot]
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
    for i, (mt, nt, kt) in enumerate(((1, 1, 1), (2, 1, 2), (1, 3, 3), (2, 2, 5), (3, 2, 17))):
        M, N, K = mt * bm, nt * bn, kt * bk
        lab = f"whole t{tile} {(M, N, K)}"
        A, B, C0 = uniform(M, N, K, 400 + i)
        C = run_gpu(A, B, C0, 0.5, -1.25, **kw)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, label=lab)
        C = run_gpu(A, B, None, 1.0, 0.0, **kw)
        check(A, B, None, 1.0, 0.0, C, oracle_mod, label=lab + " b0")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 500 + i, True)
        C = run_gpu(Ai, Bi, Ci, 0.5, -1.25, **kw)
        check(Ai, Bi, Ci, 0.5, -1.25, C, oracle_mod, exact=True, label=lab + " int")
    # rows padded by multiples of 4 floats keep every row 16-byte aligned
    M, N, K = 2 * bm, bn, 4 * bk
    rng = np.random.default_rng(tile)
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
    As = torch.full((M, K + 4), float("nan"), device=DEV)
    Bs = torch.full((K, N + 8), float("nan"), device=DEV)
    Cs = torch.full((M, N + 4), 777.0, device=DEV)
    As[:, :K] = dev(A)
    Bs[:, :N] = dev(B)
    Cs[:, :N] = dev(C0)
    sg.gemm(As[:, :K], Bs[:, :N], Cs[:, :N], 0.5, -1.25, **kw)
    torch.cuda.synchronize()
    Ch = Cs.cpu().numpy()
    assert np.all(Ch[:, N:] == 777.0), "C padding written"
    check(A, B, C0, 0.5, -1.25, Ch[:, :N].copy(), oracle_mod, label=f"whole t{tile} padded")


# ---------------------------------------------- direct-load tiles, edges --
def direct_edge_tiles():
    """Direct-load tiles with edges that read A untransposed."""
    out = []
    for t in tiles(sg.VARIANT_MFMA):
        f = sg.tile_info(sg.VARIANT_MFMA, t)["flags"]
        if f & sg.TILE_DIRECT and not f & (sg.TILE_WHOLE | sg.TILE_TRANS_A):
            out.append(t)
    return out


@pytest.mark.parametrize("slot", range(10))
def test_direct_tile_edges(slot, oracle_mod):
    """Direct-load tiles on ragged shapes: M, N, K not tile multiples, K under
    one stage, odd K and N (4-byte loads of A and B), alpha/beta, beta = 0 over
    a NaN C, integer inputs bit-exact, the 4-byte I/O flag, and padded rows
    of odd length (unaligned rows for every operand)."""
    et = direct_edge_tiles()
    if slot >= len(et):
        pytest.skip("no such direct-load tile with edges")
    tile = et[slot]
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
    shapes = [(bm + 1, bn + 3, 17), (2 * bm - 5, bn - 4, 3 * bk + 5), (37, 45, 5),
              (bm, bn, bk), (3 * bm + 16, 2 * bn + 4, 64), (300, 520, 77), (1, 1, 1)]
    for i, (M, N, K) in enumerate(shapes):
        lab = f"direct t{tile} {(M, N, K)}"
        A, B, C0 = uniform(M, N, K, 700 + i)
        C = run_gpu(A, B, C0, 0.5, -1.25, **kw)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, label=lab)
        C = run_gpu(A, B, None, 1.0, 0.0, **kw)
        check(A, B, None, 1.0, 0.0, C, oracle_mod, label=lab + " b0")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 800 + i, True)
        C = run_gpu(Ai, Bi, Ci, 0.5, -1.25, **kw)
        check(Ai, Bi, Ci, 0.5, -1.25, C, oracle_mod, exact=True, label=lab + " int")
        C = run_gpu(Ai, Bi, Ci, 0.5, -1.25, flags=sg.FLAG_SCALAR_IO, **kw)
        check(Ai, Bi, Ci, 0.5, -1.25, C, oracle_mod, exact=True, label=lab + " int scalar")
    rng = np.random.default_rng(tile)
    for (M, N, K), (pa, pb, pc) in (((bm + 7, bn + 9, 40), (3, 5, 1)),
                                    ((2 * bm, bn, 2 * bk), (4, 4, 4))):
        A = rng.uniform(-1, 1, (M, K)).astype(F32)
        B = rng.uniform(-1, 1, (K, N)).astype(F32)
        C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
        As = torch.full((M, K + pa), float("nan"), device=DEV)
        Bs = torch.full((K, N + pb), float("nan"), device=DEV)
        Cs = torch.full((M, N + pc), 777.0, device=DEV)
        As[:, :K] = dev(A)
        Bs[:, :N] = dev(B)
        Cs[:, :N] = dev(C0)
        sg.gemm(As[:, :K], Bs[:, :N], Cs[:, :N], 0.5, -1.25, **kw)
        torch.cuda.synchronize()
        Ch = Cs.cpu().numpy()
        assert np.all(Ch[:, N:] == 777.0), "C padding written"
        check(A, B, C0, 0.5, -1.25, Ch[:, :N].copy(), oracle_mod,
              label=f"direct t{tile} padded {(pa, pb, pc)}")


@pytest.mark.parametrize("shape", [(2049, 2048, 64), (2048, 2051, 70), (4112, 1000, 48),
                                   (4097, 1000, 301)])
def test_automatic_plan_with_edge_strips(shape, oracle_mod):
    """Automatic dispatch that hands edge rows / columns to the skinny family:
    every row of C against the oracle, integer inputs bit-exact."""
    M, N, K = shape
    A, B, C0 = workloads.draw(M, N, K, "int4", 950, True)
    dA, dB, dC = dev(A), dev(B), dev(C0)
    cfg, rows, cols = sg.plan(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N)
    assert rows or cols, "shape no longer exercises an edge strip"
    sg.gemm(dA, dB, dC, 0.5, -1.25)
    torch.cuda.synchronize()
    check(A, B, C0, 0.5, -1.25, dC.cpu().numpy(), oracle_mod, exact=True,
          label=f"plan {shape} strips {(rows, cols)}")


# ------------------------------------------------------- transposed B --
def trans_b_tiles():
    """Tiles that serve untransposed A with B stored transposed."""
    out = []
    for t in tiles(sg.VARIANT_MFMA):
        f = sg.tile_info(sg.VARIANT_MFMA, t)["flags"]
        if f & sg.TILE_TRANS_B and not f & sg.TILE_TRANS_A:
            out.append(t)
    return out


def run_gpu_tb(A, Bt, C0, alpha, beta, **kw):
    """C = alpha * A @ Bt^T + beta * C on the GPU, B stored transposed (N x K)."""
    M, N = A.shape[0], Bt.shape[0]
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(A), dev(Bt), C, alpha, beta, trans_b=True, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_tb(A, Bt, C0, alpha, beta, C, oracle_mod, exact=False, label=""):
    ref = oracle_mod.sgemm(A, Bt, None if C0 is None else C0.copy(), alpha,
                           beta if C0 is not None else 0.0, trans_b=True)
    if exact:
        assert np.array_equal(C, ref), f"{label}: not bit-exact"
        return
    r = max_err_ratio(C, ref, A.shape[1], alpha, beta, A, Bt, C0)
    assert r <= 1.0, f"{label}: max err/tol = {r}"


@pytest.mark.parametrize("slot", range(10))
def test_transposed_b_tiles(slot, oracle_mod):
    """Every tile that serves B stored transposed (N x K, a linear layer's
    weight): ragged and whole shapes, K under one stage and odd K (4-byte
    loads), alpha/beta, beta = 0 over NaN, integer bit-exact, 4-byte I/O."""
    tb = trans_b_tiles()
    if slot >= len(tb):
        pytest.skip("no such tile")
    tile = tb[slot]
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
    for i, (M, N, K) in enumerate(((bm, bn, 4 * bk), (bm + 3, bn - 5, 3 * bk + 7), (37, 45, 5),
                                   (2 * bm, 2 * bn + 4, 64), (1, 1, 1))):
        lab = f"tb t{tile} {(M, N, K)}"
        A, B, C0 = uniform(M, N, K, 1000 + i)
        Bt = np.ascontiguousarray(B.T)
        check_tb(A, Bt, C0, 0.5, -1.25, run_gpu_tb(A, Bt, C0, 0.5, -1.25, **kw), oracle_mod,
                 label=lab)
        check_tb(A, Bt, None, 1.0, 0.0, run_gpu_tb(A, Bt, None, 1.0, 0.0, **kw), oracle_mod,
                 label=lab + " b0")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 1100 + i, True)
        Bit = np.ascontiguousarray(Bi.T)
        check_tb(Ai, Bit, Ci, 0.5, -1.25, run_gpu_tb(Ai, Bit, Ci, 0.5, -1.25, **kw), oracle_mod,
                 exact=True, label=lab + " int")
        check_tb(Ai, Bit, Ci, 0.5, -1.25,
                 run_gpu_tb(Ai, Bit, Ci, 0.5, -1.25, flags=sg.FLAG_SCALAR_IO, **kw), oracle_mod,
                 exact=True, label=lab + " int scalar")
    # padded rows of the transposed B (NaN padding must not leak)
    M, N, K = bm + 7, bn + 9, 40
    rng = np.random.default_rng(tile)
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    Bt = rng.uniform(-1, 1, (N, K)).astype(F32)
    Bs = torch.full((N, K + 3), float("nan"), device=DEV)
    Bs[:, :K] = dev(Bt)
    C = torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(A), Bs[:, :K], C, 1.0, 0.0, trans_b=True, **kw)
    torch.cuda.synchronize()
    check_tb(A, Bt, None, 1.0, 0.0, C.cpu().numpy(), oracle_mod, label=f"tb t{tile} padded")


@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (8192, 14336, 4096), (4097, 1000, 3001),
                                   (300, 257, 129)])
def test_transposed_b_automatic(shape, oracle_mod):
    """Automatic dispatch of C = X W^T (W stored N x K) at benchmark sizes,
    sampled rows against the oracle; integer inputs bit-exact."""
    M, N, K = shape
    A, B, C0 = workloads.draw(M, N, K, "int4", 1200, True)
    Bt = np.ascontiguousarray(B.T)
    dA, dBt, dC = dev(A), dev(Bt), dev(C0)
    sg.gemm(dA, dBt, dC, 0.5, -1.25, trans_b=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, 24)
    got = dC.cpu().numpy()[rows]
    ref = oracle_mod.sgemm(np.ascontiguousarray(A[rows]), Bt, np.ascontiguousarray(C0[rows]),
                           0.5, -1.25, trans_b=True)
    assert np.array_equal(got, ref), f"transposed B {shape}"


# ------------------------------------------------------- transposed A --
def trans_a_tiles():
    return [t for t in tiles(sg.VARIANT_MFMA)
            if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_TRANS_A]


def run_gpu_op(As, Bs, C0, alpha, beta, trans_a, trans_b, **kw):
    """C = alpha * op(As) @ op(Bs) + beta * C on the GPU, operands as stored
    (A as K x M when trans_a, B as N x K when trans_b)."""
    M = As.shape[1] if trans_a else As.shape[0]
    N = Bs.shape[0] if trans_b else Bs.shape[1]
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(As), dev(Bs), C, alpha, beta, trans_a=trans_a, trans_b=trans_b, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_op(As, Bs, C0, alpha, beta, C, trans_a, trans_b, oracle_mod, exact=False, label=""):
    ref = oracle_mod.sgemm(As, Bs, None if C0 is None else C0.copy(), alpha,
                           beta if C0 is not None else 0.0, trans_a=trans_a, trans_b=trans_b)
    if exact:
        assert np.array_equal(C, ref), f"{label}: not bit-exact " \
            f"(max diff {np.nanmax(np.abs(C - ref))})"
        return
    K = As.shape[0] if trans_a else As.shape[1]
    r = max_err_ratio(C, ref, K, alpha, beta, As, Bs, C0)
    assert r <= 1.0, f"{label}: max err/tol = {r}"


def stored(A, B, trans_a, trans_b):
    return (np.ascontiguousarray(A.T) if trans_a else A,
            np.ascontiguousarray(B.T) if trans_b else B)


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("slot", range(8))
def test_transposed_a_tiles(slot, trans_b, oracle_mod):
    """Every tile that serves A stored transposed (K x M), with B either way:
    whole and ragged shapes, M not a multiple of 4 (4-byte loads of A), K
    under one stage and odd K, alpha/beta, beta = 0 over NaN, integer inputs
    bit-exact, 4-byte I/O, and a NaN-padded A."""
    ta = trans_a_tiles()
    if slot >= len(ta):
        pytest.skip("no such tile")
    tile = ta[slot]
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
    shapes = [(bm, bn, 4 * bk), (bm + 3, bn - 5, 3 * bk + 7), (37, 45, 5),
              (2 * bm + 4, 2 * bn, 64), (3 * bm - 16, bn + 4, 2 * bk), (1, 1, 1)]
    for i, (M, N, K) in enumerate(shapes):
        lab = f"ta t{tile} tb={trans_b} {(M, N, K)}"
        A0, B0, C0 = uniform(M, N, K, 1300 + i)
        A, B = stored(A0, B0, True, trans_b)
        args = (True, trans_b)
        check_op(A, B, C0, 0.5, -1.25, run_gpu_op(A, B, C0, 0.5, -1.25, *args, **kw), *args,
                 oracle_mod, label=lab)
        check_op(A, B, None, 1.0, 0.0, run_gpu_op(A, B, None, 1.0, 0.0, *args, **kw), *args,
                 oracle_mod, label=lab + " b0")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 1400 + i, True)
        Ai, Bi = stored(Ai, Bi, True, trans_b)
        check_op(Ai, Bi, Ci, 0.5, -1.25, run_gpu_op(Ai, Bi, Ci, 0.5, -1.25, *args, **kw), *args,
                 oracle_mod, exact=True, label=lab + " int")
        check_op(Ai, Bi, Ci, 0.5, -1.25,
                 run_gpu_op(Ai, Bi, Ci, 0.5, -1.25, *args, flags=sg.FLAG_SCALAR_IO, **kw),
                 *args, oracle_mod, exact=True, label=lab + " int scalar")
    # A stored K x M inside wider rows (lda = M + 3 and M + 4); NaN padding must not leak
    rng = np.random.default_rng(tile)
    for M, N, K, pad in ((bm + 7, bn + 9, 40, 3), (2 * bm, bn, 2 * bk, 4)):
        At = rng.uniform(-1, 1, (K, M)).astype(F32)
        B = rng.uniform(-1, 1, (N, K) if trans_b else (K, N)).astype(F32)
        As = torch.full((K, M + pad), float("nan"), device=DEV)
        As[:, :M] = dev(At)
        C = torch.full((M, N), float("nan"), device=DEV)
        sg.gemm(As[:, :M], dev(B), C, 1.0, 0.0, trans_a=True, trans_b=trans_b, **kw)
        torch.cuda.synchronize()
        check_op(At, B, None, 1.0, 0.0, C.cpu().numpy(), True, trans_b, oracle_mod,
                 label=f"ta t{tile} tb={trans_b} padded {pad}")


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (4097, 1000, 3001), (300, 257, 129),
                                   (64, 64, 64)])
def test_transposed_a_automatic(shape, trans_b, oracle_mod):
    """Automatic dispatch of C = A^T B and C = A^T B^T (A stored K x M) at
    benchmark and ragged sizes, sampled rows against the oracle; integer
    inputs bit-exact."""
    M, N, K = shape
    A, B, C0 = workloads.draw(M, N, K, "int4", 1500, True)
    As, Bs = stored(A, B, True, trans_b)
    dA, dB, dC = dev(As), dev(Bs), dev(C0)
    sg.gemm(dA, dB, dC, 0.5, -1.25, trans_a=True, trans_b=trans_b)
    torch.cuda.synchronize()
    rows = sample_rows(M, 24)
    got = dC.cpu().numpy()[rows]
    ref = oracle_mod.sgemm(np.ascontiguousarray(As[:, rows]), Bs, np.ascontiguousarray(C0[rows]),
                           0.5, -1.25, trans_a=True, trans_b=trans_b)
    assert np.array_equal(got, ref), f"transposed A {shape} trans_b={trans_b}"


# ------------------------------------------------------- CBLAS order --
@pytest.mark.parametrize("order", [101, 102])
@pytest.mark.parametrize("ta,tb", [(111, 111), (111, 112), (112, 111), (113, 113)])
def test_cblas_orders(order, ta, tb, oracle_mod):
    """sgemm_cblas in both storage orders and every transposition: the stored
    matrices are built from the logical A (M x K), B (K x N), C (M x N) and
    the result read back through the same order; integer inputs bit-exact."""
    def store(X, trans):
        # the matrix the caller stores (X, or X^T when trans) in the given
        # order, as a row-major array, and its leading dimension
        S = X.T if trans else X
        S = S if order == 101 else S.T
        S = np.ascontiguousarray(S)
        return S, S.shape[1]

    for i, (M, N, K) in enumerate(((300, 257, 129), (1000, 777, 333), (64, 64, 64), (1, 1, 1),
                                   (5, 3, 4100))):
        for dist in ("uniform", "int4"):
            A, B, C0 = workloads.draw(M, N, K, dist, 1600 + i, True)
            As, lda = store(A, ta != 111)
            Bs, ldb = store(B, tb != 111)
            Cs, ldc = store(C0, False)
            dA, dB, dC = dev(As), dev(Bs), dev(Cs)
            torch.cuda.synchronize()
            st = sg.sgemm_cblas(order, ta, tb, M, N, K, 0.5, dA.data_ptr(), lda, dB.data_ptr(),
                                ldb, -1.25, dC.data_ptr(), ldc,
                                torch.cuda.current_stream().cuda_stream)
            assert st == 0, sg.status_string(st)
            torch.cuda.synchronize()
            got = dC.cpu().numpy()
            got = got if order == 101 else np.ascontiguousarray(got.T)
            lab = f"cblas order={order} {ta}/{tb} {(M, N, K)} {dist}"
            check(A, B, C0, 0.5, -1.25, got, oracle_mod, exact=(dist == "int4"), label=lab)


SKINNY_CASES = {
    0: [(1, 1000, 3001), (16, 4100, 333), (7, 77, 4097), (3, 5, 9)],
    1: [(1000, 1, 3001), (513, 3, 1000), (77, 16, 4097), (5, 2, 9),
        # one column, K a multiple of 4: the row-streaming kernel (two or
        # three rows per wave at 5000 rows)
        (1000, 1, 3000), (5000, 1, 1024), (3, 1, 4)],
}


@pytest.mark.parametrize("tile", range(16))
def test_skinny_tiles(tile, oracle_mod):
    if tile >= sg.tile_count(sg.VARIANT_SKINNY):
        pytest.skip("tile not compiled")
    desc = sg.tile_info(sg.VARIANT_SKINNY, tile)
    kind = desc["tm"]
    for i, (M, N, K) in enumerate(SKINNY_CASES[kind]):
        if kind == 1 and N > desc["bn"]:
            continue
        A, B, C0 = uniform(M, N, K, 200 + i)
        kw = dict(variant=sg.VARIANT_SKINNY, tile=tile)
        C = run_gpu(A, B, C0, 0.5, -1.25, **kw)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, label=f"skinny t{tile} {(M, N, K)}")
        C = run_gpu(A, B, C0, 0.5, -1.25, flags=sg.FLAG_SCALAR_IO, **kw)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, label=f"skinny t{tile} {(M, N, K)} scalar")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 300 + i, True)
        C = run_gpu(Ai, Bi, Ci, 0.5, -1.25, **kw)
        check(Ai, Bi, Ci, 0.5, -1.25, C, oracle_mod, exact=True, label=f"skinny t{tile} int")


def test_one_column_stream(oracle_mod):
    """One column of C with A in 16-byte rows and a contiguous column of B:
    the row-streaming kernel (rows handed to the waves in turn), through
    automatic dispatch.  Integer inputs bit for bit: more rows than waves,
    beta reading C, B stored as a column and as a row (transposed), padded
    16-byte rows of A, a batch, and bias + ReLU; a padded row length that is
    not a multiple of 4 takes the general few-columns kernel.  Also one row
    of C with W stored N x K, which runs as that column problem transposed."""
    rng = np.random.default_rng(77)
    for (M, K) in ((9000, 512), (4096, 4096), (7, 4), (2049, 1000)):
        A, B, C0 = workloads.draw(M, 1, K, "int4", M + K, True)
        lab = f"one column {(M, K)}"
        C = run_gpu(A, B, C0, 0.5, -1.25)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, exact=True, label=lab)
        Bt = np.ascontiguousarray(B.T)
        C = run_gpu_op(A, Bt, C0, 0.5, -1.25, False, True)
        check_op(A, Bt, C0, 0.5, -1.25, C, False, True, oracle_mod, exact=True, label=lab + " B^T")
        for pad in (4, 1):
            Ap = torch.full((M, K + pad), float("nan"), device=DEV)
            Ap[:, :K] = dev(A)
            Cd = dev(C0)
            sg.gemm(Ap[:, :K], dev(B), Cd, 0.5, -1.25)
            torch.cuda.synchronize()
            check(A, B, C0, 0.5, -1.25, Cd.cpu().numpy(), oracle_mod, exact=True,
                  label=f"{lab} lda={K + pad}")
    bat, M, K = 3, 3000, 256
    A = rng.integers(-4, 5, (bat, M, K)).astype(F32)
    B = rng.integers(-4, 5, (bat, K, 1)).astype(F32)
    C0 = rng.integers(-4, 5, (bat, M, 1)).astype(F32)
    ref = oracle_mod.sgemm_batched(A, B, C0.copy(), 0.5, -1.25)
    C = dev(C0)
    sg.gemm_batched(dev(A), dev(B), C, 0.5, -1.25)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref), "one column, batched"
    # a batch of single rows times W^T (one W per entry): the transposed form
    W = rng.integers(-4, 5, (bat, 700, K)).astype(F32)
    X = rng.integers(-4, 5, (bat, 1, K)).astype(F32)
    C0 = rng.integers(-4, 5, (bat, 1, 700)).astype(F32)
    ref = oracle_mod.sgemm_batched(X, W, C0.copy(), 0.5, -1.25, trans_b=True)
    C = dev(C0)
    sg.gemm_batched(dev(X), dev(W), C, 0.5, -1.25, trans_b=True)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref), "one row x W^T, batched"
    # one row with B stored transposed (x W^T): run as the column W x^T when
    # there is no bias; with a bias, or a K split asked for, the few-rows path
    for (N, K) in ((14336, 4096), (1000, 3000), (257, 8)):
        A, B, C0 = workloads.draw(1, N, K, "int4", N + K, True)
        Bt = np.ascontiguousarray(B.T)
        lab = f"one row x W^T {(N, K)}"
        C = run_gpu_op(A, Bt, C0, 0.5, -1.25, False, True)
        check_op(A, Bt, C0, 0.5, -1.25, C, False, True, oracle_mod, exact=True, label=lab)
        for kw in (dict(act=sg.ACT_RELU), dict(bias=np.full(N, 2.0, F32), act=sg.ACT_RELU)):
            ref = oracle_mod.sgemm(A, Bt, C0.copy(), 1.0, 0.5, trans_b=True, **kw)
            C = dev(C0)
            b = kw.get("bias")
            sg.gemm(dev(A), dev(Bt), C, 1.0, 0.5, trans_b=True, act=kw["act"],
                    bias=None if b is None else dev(b))
            torch.cuda.synchronize()
            assert np.array_equal(C.cpu().numpy(), ref), f"{lab} {sorted(kw)}"
        C = run_gpu_op(A, Bt, C0, 0.5, -1.25, False, True, variant=sg.VARIANT_SKINNY,
                       tile=staged_tile(), group_m=2)
        check_op(A, Bt, C0, 0.5, -1.25, C, False, True, oracle_mod, exact=True,
                 label=lab + " split asked for")
    A, B, C0 = workloads.draw(5000, 1, 512, "int4", 78, True)
    bias = np.array([3.0], dtype=F32)
    ref = oracle_mod.sgemm(A, B, C0.copy(), 1.0, 0.5, bias=bias, act=sg.ACT_RELU)
    C = dev(C0)
    sg.gemm(dev(A), dev(B), C, 1.0, 0.5, bias=dev(bias), act=sg.ACT_RELU)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref), "one column, bias + ReLU"


def staged_tile():
    """The few-rows tile of 64 columns, 4 waves and 4 chunks per round: with B
    stored transposed and 16-byte rows of A and B it runs the LDS-staged kernel."""
    for t in tiles(sg.VARIANT_SKINNY):
        d = sg.tile_info(sg.VARIANT_SKINNY, t)
        if d["tm"] == 0 and d["bn"] == 64 and d["threads"] == 256 and d["bk"] == 64:
            return t
    return None


@pytest.mark.parametrize("slices", [1, 0, 3, 8])
def test_skinny_staged_transposed_b(slices, oracle_mod):
    """Few rows with B stored N x K through the LDS-staged kernel: ragged
    strips (N not a multiple of 64), K not a multiple of the 64-k round, one
    to sixteen rows, split over K or not; integer inputs bit for bit,
    uniform inputs within tolerance, bias + activation, and two calls alike."""
    tile = staged_tile()
    if tile is None:
        pytest.skip("no 64-column 4-wave tile with 4 chunks per round")
    for i, (M, N, K) in enumerate([(16, 4100, 336), (1, 1000, 3004), (7, 64, 4096),
                                   (16, 2048, 4096), (3, 200, 68), (11, 130, 1028)]):
        kw = dict(variant=sg.VARIANT_SKINNY, tile=tile, group_m=slices)
        lab = f"staged t{tile} s{slices} {(M, N, K)}"
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 3100 + i, True)
        Bt = np.ascontiguousarray(Bi.T)
        C = run_gpu_op(Ai, Bt, Ci, 0.5, -1.25, False, True, **kw)
        check_op(Ai, Bt, Ci, 0.5, -1.25, C, False, True, oracle_mod, exact=True, label=lab + " int")
        C2 = run_gpu_op(Ai, Bt, Ci, 0.5, -1.25, False, True, **kw)
        assert np.array_equal(C, C2), f"{lab}: two calls differ"
        A, B, C0 = uniform(M, N, K, 3200 + i)
        Bt = np.ascontiguousarray(B.T)
        check_op(A, Bt, C0, 1.0, 0.0, run_gpu_op(A, Bt, None, 1.0, 0.0, False, True, **kw),
                 False, True, oracle_mod, label=lab)
    M, N, K = 9, 300, 512
    A, B, C0 = uniform(M, N, K, 3300)
    Bt = np.ascontiguousarray(B.T)
    bias = np.random.default_rng(3301).uniform(-1, 1, N).astype(F32)
    C = dev(C0)
    sg.gemm(dev(A), dev(Bt), C, 1.0, 0.5, trans_b=True, bias=dev(bias), act=sg.ACT_SILU,
            variant=sg.VARIANT_SKINNY, tile=tile, group_m=slices)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm(A, Bt, C0.copy(), 1.0, 0.5, trans_b=True, bias=bias, act=sg.ACT_SILU)
    x = oracle_mod.sgemm(A, Bt, C0.copy(), 1.0, 0.5, trans_b=True, bias=bias, act=sg.ACT_NONE)
    r = epilogue_err_ratio(C.cpu().numpy(), ref, x, K, 1.0, 0.5, A, Bt, C0, bias, sg.ACT_SILU)
    assert r <= 1.0, f"staged epilogue: {r}"


def test_skinny_balanced_strips(oracle_mod):
    """Few-rows products with B stored N x K, large (32 MB or more), whose
    natural strips times K slices fall short of the 256 CUs run narrower
    strips (a multiple of 4 rows of B^T, not the tile's 64) so that every CU
    streams.  Through the LDS-staged kernel: 16 x 9001 x 4096 as 251 strips
    of 36 rows (the last one row), in fp32 and bfloat16; 8 x 6000 x 8192 as
    125 strips of 48 rows and 2 K slices; one row with a bias (not the
    one-column route) as 256 strips of 56 rows.  With K = 4097 (4-byte
    loads, the register kernel) 6 x 9000 x 4097 as 250 strips of 36 rows.
    Integer inputs, beta reading C: the whole of C bit for bit."""
    for i, (M, N, K) in enumerate([(16, 9001, 4096), (8, 6000, 8192), (6, 9000, 4097)]):
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 3400 + i, True)
        Bt = np.ascontiguousarray(Bi.T)
        C = run_gpu_op(Ai, Bt, Ci, 0.5, -1.25, False, True)
        check_op(Ai, Bt, Ci, 0.5, -1.25, C, False, True, oracle_mod, exact=True,
                 label=f"balanced strips {(M, N, K)}")
    rng = np.random.default_rng(3410)
    M, N, K = 1, 14336, 4096
    x = rng.integers(-4, 5, (M, K)).astype(F32)
    w = rng.integers(-4, 5, (N, K)).astype(F32)
    C0 = rng.integers(-4, 5, (M, N)).astype(F32)
    bias = rng.integers(-8, 9, N).astype(F32)
    C = dev(C0)
    sg.gemm(dev(x), dev(w), C, 0.5, -1.25, trans_b=True, bias=dev(bias), act=sg.ACT_RELU)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm(x, w, C0.copy(), 0.5, -1.25, trans_b=True, bias=bias, act=sg.ACT_RELU)
    assert np.array_equal(C.cpu().numpy(), ref), "balanced strips, one row with bias"
    M, N, K = 16, 9001, 4096
    x = rng.integers(-4, 5, (M, K)).astype(F32)
    w = rng.integers(-4, 5, (N, K)).astype(F32)
    C0 = rng.integers(-4, 5, (M, N)).astype(F32)
    C = dev(C0)
    sg.gemm_mixed(dev(x).to(torch.bfloat16), dev(w).to(torch.bfloat16), C, 0.5, -1.25,
                  trans_b=True)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm(x, w, C0.copy(), 0.5, -1.25, trans_b=True)
    assert np.array_equal(C.cpu().numpy(), ref), "balanced strips, bfloat16 x W^T"


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
@pytest.mark.parametrize("tile", range(16))
def test_skinny_tiles_transposed(tile, ta, tb, oracle_mod):
    """The skinny family on transposed storage: few rows with A and/or B
    transposed (B stored N x K is the decode layout of a linear layer), few
    columns with B transposed; 16-byte and 4-byte paths, integers bit-exact."""
    if tile >= sg.tile_count(sg.VARIANT_SKINNY):
        pytest.skip("tile not compiled")
    desc = sg.tile_info(sg.VARIANT_SKINNY, tile)
    kind = desc["tm"]
    if kind == 1 and ta:
        pytest.skip("the few-columns kernel does not read A transposed")
    cases = SKINNY_CASES[kind] + [(9, 300, 64) if kind == 0 else (300, 9, 64)]
    for i, (M, N, K) in enumerate(cases):
        if kind == 1 and N > desc["bn"]:
            continue
        kw = dict(variant=sg.VARIANT_SKINNY, tile=tile)
        A0, B0, C0 = uniform(M, N, K, 250 + i)
        As, Bs = stored(A0, B0, ta, tb)
        lab = f"skinny t{tile} ta={ta} tb={tb} {(M, N, K)}"
        check_op(As, Bs, C0, 0.5, -1.25, run_gpu_op(As, Bs, C0, 0.5, -1.25, ta, tb, **kw), ta,
                 tb, oracle_mod, label=lab)
        check_op(As, Bs, C0, 0.5, -1.25,
                 run_gpu_op(As, Bs, C0, 0.5, -1.25, ta, tb, flags=sg.FLAG_SCALAR_IO, **kw), ta,
                 tb, oracle_mod, label=lab + " scalar")
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 350 + i, True)
        Ai, Bi = stored(Ai, Bi, ta, tb)
        check_op(Ai, Bi, Ci, 0.5, -1.25, run_gpu_op(Ai, Bi, Ci, 0.5, -1.25, ta, tb, **kw), ta,
                 tb, oracle_mod, exact=True, label=lab + " int")


# ------------------------------------------------------------ tiny shapes --
def test_tiny_shapes_brute_force(oracle_mod):
    """Every (M, N, K) from a set of tiny sizes, through automatic dispatch,
    bit-exact on integer inputs."""
    sizes = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 33]
    for M, N, K in itertools.product(sizes, sizes, sizes):
        A, B, C0 = workloads.draw(M, N, K, "int4", M * 10007 + N * 101 + K, True)
        C = run_gpu(A, B, C0, 0.5, -1.25)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, exact=True, label=f"tiny {(M, N, K)}")
        ta, tb = bool((M + K) % 2), bool((N + K) % 2)
        if ta or tb:
            As, Bs = stored(A, B, ta, tb)
            check_op(As, Bs, C0, 0.5, -1.25, run_gpu_op(As, Bs, C0, 0.5, -1.25, ta, tb), ta, tb,
                     oracle_mod, exact=True, label=f"tiny {(M, N, K)} ta={ta} tb={tb}")


# ------------------------------------------------------- full-size shapes --
FULL = [n for n in workloads.WORKLOADS if n != "probe256"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size(name, oracle_mod):
    """Each named workload at its full size, automatic dispatch (the launch
    configuration the benchmark times), sampled rows against the oracle."""
    w = workloads.WORKLOADS[name]
    A, B, C0 = workloads.inputs(w)
    C = run_gpu(A, B, C0, w.alpha, w.beta)
    exact = w.dist == "int4"
    # the whole of C: the largest (mlp_up, mlp_down, sweep8192, ~1 TFLOP each)
    # take the multithreaded oracle about ten seconds on the GPU machine's host
    r = check(A, B, C0, w.alpha, w.beta, C, oracle_mod, exact=exact, label=name)
    print(f"{name}: max err/tol = {r:.3g} on all {w.M} rows", flush=True)
    assert np.all(np.isfinite(C))


def test_valu_family_full_size(oracle_mod):
    w = workloads.WORKLOADS["square4096"]
    A, B, _ = workloads.inputs(w)
    C = run_gpu(A, B, None, 1.0, 0.0, variant=sg.VARIANT_VALU)
    check(A, B, None, 1.0, 0.0, C, oracle_mod, rows=sample_rows(w.M, 48), label="valu 4096")


def test_integer_full_size_every_mfma_tile(oracle_mod):
    """Every MFMA tile at 4096^3 (the transposed-A tiles on A stored K x M)."""
    A, B, C0 = workloads.inputs("int4096_blas")
    rows = sample_rows(4096, 24)
    At = np.ascontiguousarray(A.T)
    for tile in tiles(sg.VARIANT_MFMA):
        kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
        if sg.tile_info(sg.VARIANT_MFMA, tile)["flags"] & sg.TILE_TRANS_A:
            C = run_gpu_op(At, B, C0, 0.5, -1.25, True, False, **kw)
        else:
            C = run_gpu(A, B, C0, 0.5, -1.25, **kw)
        check(A, B, C0, 0.5, -1.25, C, oracle_mod, rows=rows, exact=True, label=f"tile {tile}")


# ------------------------------------------------------------ edge cases --
def test_fp32_probe_bit_exact(oracle_mod):
    """17-significant-bit inputs: exact in fp32, wrong under any narrower input format."""
    A, B, _ = workloads.inputs("probe256")
    for variant in (sg.VARIANT_AUTO, sg.VARIANT_MFMA, sg.VARIANT_VALU):
        C = run_gpu(A, B, None, 1.0, 0.0, variant=variant)
        check(A, B, None, 1.0, 0.0, C, oracle_mod, exact=True, label=f"probe v{variant}")


def probe_inputs(M, N, K, seed):
    """The precision probe's draws at another shape: A = n * 2^-16 with
    |n| <= 2^16 (17 significant bits), B in {-1, 0, 1}.  With K <= 256 every
    partial sum is a multiple of 2^-16 below 2^8 in magnitude, exact in fp32
    whatever the order, and inexact if either input were rounded to a format
    with fewer significant bits (tf32, bf16, fp16)."""
    assert K <= 256
    return workloads.draw(M, N, K, "probe", seed, False)[:2]


def test_fp32_probe_every_kernel(oracle_mod):
    """The probe through every compiled fp32 kernel, bit for bit: each MFMA
    tile (the transposed-A tiles on A stored K x M, the others also with B
    stored N x K where they serve it), forced stream-K, each VALU tile, each
    few-rows skinny tile (split over K and not), each few-columns tile and
    each small-product tile."""
    M, N, K = 512, 512, 256
    A, B = probe_inputs(M, N, K, 41)
    ref = oracle_mod.sgemm(A, B)
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    for tile in tiles(sg.VARIANT_MFMA):
        d = sg.tile_info(sg.VARIANT_MFMA, tile)
        kw = dict(variant=sg.VARIANT_MFMA, tile=tile)
        ta = bool(d["flags"] & sg.TILE_TRANS_A)
        for tb in (False, True):
            if tb and not d["flags"] & (sg.TILE_TRANS_B | sg.TILE_TRANS_A):
                continue
            C = run_gpu_op(At if ta else A, Bt if tb else B, None, 1.0, 0.0, ta, tb, **kw)
            assert np.array_equal(C, ref), f"probe: MFMA tile {tile} ta={ta} tb={tb}"
            if d["flags"] & sg.TILE_STREAMK:
                # 8 tiles of 256 x 128 (or 4 of 256 x 256), 16 k-steps each,
                # cut into 256 runs: every tile is split and fixed up
                C = run_gpu_op(At if ta else A, Bt if tb else B, None, 1.0, 0.0, ta, tb,
                               flags=sg.FLAG_STREAMK, **kw)
                assert np.array_equal(C, ref), f"probe: stream-K tile {tile} ta={ta} tb={tb}"
    for tile in tiles(sg.VARIANT_VALU):
        C = run_gpu(A, B, None, 1.0, 0.0, variant=sg.VARIANT_VALU, tile=tile)
        assert np.array_equal(C, ref), f"probe: VALU tile {tile}"
    for tile in tiles(sg.VARIANT_SKINNY):
        d = sg.tile_info(sg.VARIANT_SKINNY, tile)
        if d["tm"] == 0:
            Ar, Br = probe_inputs(16, 1000, 256, 42)
            refr = oracle_mod.sgemm(Ar, Br)
            for tb in (False, True):
                for slices in (1, 0, 4):
                    kw = dict(variant=sg.VARIANT_SKINNY, tile=tile, group_m=slices)
                    C = run_gpu_op(Ar, np.ascontiguousarray(Br.T) if tb else Br, None, 1.0, 0.0,
                                   False, tb, **kw)
                    assert np.array_equal(C, refr), \
                        f"probe: skinny tile {tile} tb={tb} slices={slices}"
        else:
            n = min(d["bn"], 16)
            Ac, Bc = probe_inputs(777, n, 256, 43)
            refc = oracle_mod.sgemm(Ac, Bc)
            C = run_gpu(Ac, Bc, None, 1.0, 0.0, variant=sg.VARIANT_SKINNY, tile=tile)
            assert np.array_equal(C, refc), f"probe: few-columns tile {tile} N={n}"
    for tile in tiles(sg.VARIANT_SMALL):
        for tb in (False, True):
            C = run_gpu_op(A, Bt if tb else B, None, 1.0, 0.0, False, tb,
                           variant=sg.VARIANT_SMALL, tile=tile)
            assert np.array_equal(C, ref), f"probe: small tile {tile} tb={tb}"


def test_beta_zero_never_reads_c(oracle_mod):
    for (M, N, K) in ((300, 500, 70), (1, 300, 50), (300, 1, 50)):
        A, B, _ = uniform(M, N, K, 11, False)
        C = run_gpu(A, B, None, 1.0, 0.0)        # C starts as NaN
        assert np.all(np.isfinite(C))
        check(A, B, None, 1.0, 0.0, C, oracle_mod, label=f"beta0 {(M, N, K)}")


def test_alpha_zero_never_reads_a_b():
    M, N, K = 100, 70, 30
    A = np.full((M, K), np.nan, F32)
    B = np.full((K, N), np.nan, F32)
    C0 = np.random.default_rng(1).uniform(-1, 1, (M, N)).astype(F32)
    C = run_gpu(A, B, C0, 0.0, 0.5)
    assert np.array_equal(C, C0 * F32(0.5))
    C = run_gpu(A, B, C0, 0.0, 0.0)
    assert np.all(C == 0)
    C = run_gpu(A, B, C0, 0.0, 1.0)
    assert np.array_equal(C, C0)


def test_k_zero_and_empty():
    C0 = np.arange(12, dtype=F32).reshape(3, 4)
    C = dev(C0)
    sg.gemm(torch.empty((3, 0), device=DEV), torch.empty((0, 4), device=DEV), C, 1.0, 2.0)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), C0 * 2)
    out = sg.gemm(torch.empty((0, 5), device=DEV), torch.ones((5, 4), device=DEV))
    assert out.shape == (0, 4)


def test_leading_dimension_padding(oracle_mod):
    """NaN in the row padding of A and B never reaches C; C's padding is untouched."""
    rng = np.random.default_rng(5)
    for (M, N, K) in ((300, 257, 129), (5, 1000, 300), (1000, 3, 300), (64, 64, 64)):
        for pa, pb, pc in ((4, 4, 4), (3, 5, 1)):
            A = rng.uniform(-1, 1, (M, K)).astype(F32)
            B = rng.uniform(-1, 1, (K, N)).astype(F32)
            C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
            As = torch.full((M, K + pa), float("nan"), device=DEV)
            Bs = torch.full((K, N + pb), float("nan"), device=DEV)
            Cs = torch.full((M, N + pc), 777.0, device=DEV)
            As[:, :K] = dev(A)
            Bs[:, :N] = dev(B)
            Cs[:, :N] = dev(C0)
            sg.gemm(As[:, :K], Bs[:, :N], Cs[:, :N], 1.0, 1.0)
            torch.cuda.synchronize()
            Ch = Cs.cpu().numpy()
            assert np.all(Ch[:, N:] == 777.0), "C padding written"
            check(A, B, C0, 1.0, 1.0, Ch[:, :N].copy(), oracle_mod,
                  label=f"ld {(M, N, K)} pad {(pa, pb, pc)}")


def test_unaligned_pointers_use_scalar_io(oracle_mod):
    """Operands starting 4 bytes past a 16-byte boundary are valid (4-byte aligned)."""
    rng = np.random.default_rng(6)
    M, N, K = 333, 290, 157
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
    a = torch.zeros(M * K + 1, device=DEV); a[1:] = dev(A).reshape(-1)
    b = torch.zeros(K * N + 1, device=DEV); b[1:] = dev(B).reshape(-1)
    c = torch.zeros(M * N + 1, device=DEV); c[1:] = dev(C0).reshape(-1)
    cfg = sg.select(M, N, K, a[1:].data_ptr(), K, b[1:].data_ptr(), N, c[1:].data_ptr(), N)
    # general tiles fall back to 4-byte I/O; direct-load and skinny tiles
    # choose the width per operand themselves
    d = sg.tile_info(cfg.variant, cfg.tile)
    if cfg.variant == sg.VARIANT_MFMA and not d["flags"] & sg.TILE_DIRECT:
        assert cfg.flags & sg.FLAG_SCALAR_IO
    sg.gemm(a[1:].view(M, K), b[1:].view(K, N), c[1:].view(M, N), 0.5, -1.25)
    torch.cuda.synchronize()
    check(A, B, C0, 0.5, -1.25, c[1:].view(M, N).cpu().numpy(), oracle_mod, label="unaligned")


def test_closed_forms_ragged():
    """Identity, permutation and all-ones products are exact at ragged shapes."""
    rng = np.random.default_rng(8)
    for K in (33, 300, 1031):
        I = np.eye(K, dtype=F32)
        for N in (1, 17, 257):
            Bm = rng.uniform(-1, 1, (K, N)).astype(F32)
            assert np.array_equal(run_gpu(I, Bm, None, 1.0, 0.0), Bm)
        for M in (1, 19, 500):
            Am = rng.uniform(-1, 1, (M, K)).astype(F32)
            assert np.array_equal(run_gpu(Am, I, None, 1.0, 0.0), Am)
            perm = rng.permutation(K)
            P = np.zeros((K, K), F32)
            P[perm, np.arange(K)] = 1
            assert np.array_equal(run_gpu(Am, P, None, 1.0, 0.0), Am[:, perm])
    for (M, N, K) in ((129, 65, 4096), (1, 300, 4096), (300, 1, 4096), (4097, 1000, 3001)):
        C = run_gpu(np.ones((M, K), F32), np.ones((K, N), F32), None, 1.0, 0.0)
        assert np.all(C == K)


def test_deterministic_and_scaling():
    A, B, _ = uniform(1000, 1000, 1000, 12, False)
    for variant in (sg.VARIANT_MFMA, sg.VARIANT_VALU):
        C1 = run_gpu(A, B, None, 1.0, 0.0, variant=variant)
        C2 = run_gpu(A, B, None, 1.0, 0.0, variant=variant)
        assert np.array_equal(C1, C2)
        C3 = run_gpu(A * F32(2), B, None, 1.0, 0.0, variant=variant)
        assert np.array_equal(C3, C1 * F32(2))
    for (M, N, K) in ((1, 4096, 4096), (4096, 1, 4096), (16, 14336, 512)):
        A, B, _ = uniform(M, N, K, 13, False)
        assert np.array_equal(run_gpu(A, B, None, 1.0, 0.0), run_gpu(A, B, None, 1.0, 0.0))
