"""GPU parity of the 16-bit-input GEMM (sgemm_mixed: bfloat16 / float16 A and
B, fp32 accumulation and C) against the oracle's 16-bit entry point, which
decodes the same bit patterns exactly.

Every test is marked ``gpu``.  Every product of two 16-bit values is exact
in fp32 and the sums are accumulated in fp32, so the fp32 tolerance of
parity.py applies (with max|A|, max|B| of the decoded values); small-integer
inputs are bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
from parity import max_err_ratio, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"
DTYPES = [(sg.DTYPE_BF16, "bfloat16"), (sg.DTYPE_F16, "float16")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def to16(x: np.ndarray, tname: str) -> np.ndarray:
    """Round float values to the 16-bit format (round to nearest even) and
    return the bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=F32)).to(getattr(torch, tname))
    return t.view(torch.int16).numpy().view(np.uint16)


def decoded(bits: np.ndarray, tname: str) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(getattr(torch, tname)).float().numpy()


def dev16(bits: np.ndarray, tname: str):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        getattr(torch, tname)).to(DEV)


def draw(rng, shape, integer, tname):
    x = rng.integers(-4, 5, shape) if integer else rng.uniform(-1, 1, shape)
    return to16(x, tname)


def run_check(rng, dtype, tname, M, N, K, ta, tb, integer, oracle_mod, label, alpha=0.5,
              beta=-1.25, rows=None, **kw):
    Ab = draw(rng, (K, M) if ta else (M, K), integer, tname)
    Bb = draw(rng, (N, K) if tb else (K, N), integer, tname)
    C0 = (rng.integers(-4, 5, (M, N)) if integer else rng.uniform(-1, 1, (M, N))).astype(F32)
    C = torch.from_numpy(C0).to(DEV) if beta != 0 else \
        torch.full((M, N), float("nan"), device=DEV)
    sg.gemm_mixed(dev16(Ab, tname), dev16(Bb, tname), C, alpha, beta, trans_a=ta, trans_b=tb,
                  **kw)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    Ar = Ab if rows is None else np.ascontiguousarray(Ab[:, rows] if ta else Ab[rows])
    Cr = C0 if rows is None else np.ascontiguousarray(C0[rows])
    got = got if rows is None else got[rows]
    ref = oracle_mod.gemm_mixed(dtype, Ar, Bb, Cr.copy() if beta != 0 else None, alpha,
                                beta, trans_a=ta, trans_b=tb)
    if integer:
        assert np.array_equal(got, ref), f"{label}: not bit-exact"
        return
    Ad, Bd = decoded(Ar, tname), decoded(Bb, tname)
    r = max_err_ratio(got, ref, K, alpha, beta, Ad, Bd, Cr if beta != 0 else None)
    assert r <= 1.0, f"{label}: max err/tol = {r}"


@pytest.mark.parametrize("dtype,tname", DTYPES)
@pytest.mark.parametrize("tile", range(8))
def test_mfma16_tiles(tile, dtype, tname, oracle_mod):
    """Every 16-bit matrix-core tile on C = X W^T (W stored N x K): whole
    tiles, ragged M/N/K, K a multiple of 2 but not of 8 (4-byte loads),
    alpha/beta and beta = 0 over NaN, integers bit-exact."""
    if tile >= sg.tile_count(sg.VARIANT_MFMA16):
        pytest.skip("no such tile")
    d = sg.tile_info(sg.VARIANT_MFMA16, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    rng = np.random.default_rng(tile * 10 + dtype)
    kw = dict(variant=sg.VARIANT_MFMA16, tile=tile)
    for M, N, K in ((bm, bn, 4 * bk), (bm + 3, bn - 5, 3 * bk + 2), (37, 45, 6),
                    (2 * bm + 4, 2 * bn, 64), (1, 1, 2), (bm, bn + 16, 70)):
        lab = f"{tname} t{tile} {(M, N, K)}"
        run_check(rng, dtype, tname, M, N, K, False, True, False, oracle_mod, lab, **kw)
        run_check(rng, dtype, tname, M, N, K, False, True, False, oracle_mod, lab + " b0",
                  alpha=1.0, beta=0.0, **kw)
        run_check(rng, dtype, tname, M, N, K, False, True, True, oracle_mod, lab + " int", **kw)


@pytest.mark.parametrize("dtype,tname", DTYPES)
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_mixed_automatic_every_layout(ta, tb, dtype, tname, oracle_mod):
    """Automatic dispatch for every transposition (the generic kernel for all
    but NT), odd K and ragged shapes, integers bit-exact."""
    rng = np.random.default_rng(int(ta) * 2 + int(tb) + 10 * dtype)
    for M, N, K in ((300, 257, 129), (64, 64, 64), (1000, 300, 77), (5, 700, 33), (1, 1, 1)):
        lab = f"{tname} auto ta={ta} tb={tb} {(M, N, K)}"
        run_check(rng, dtype, tname, M, N, K, ta, tb, False, oracle_mod, lab)
        run_check(rng, dtype, tname, M, N, K, ta, tb, True, oracle_mod, lab + " int")


@pytest.mark.parametrize("dtype,tname", DTYPES)
def test_mixed_few_rows(dtype, tname, oracle_mod):
    """Decode-like shapes (M <= 16) with W stored N x K: the few-rows skinny
    kernel in word form (M <= 8), 16-byte and 4-byte loads, and the k-group
    tiles above that; one row runs as the transposed one-column product
    (W's rows streamed, more rows than waves at 9000) where the word rows
    take 16-byte loads."""
    rng = np.random.default_rng(40 + dtype)
    for M, N, K in ((1, 5000, 4096), (8, 300, 64), (5, 4100, 66), (3, 17, 2), (16, 14336, 512),
                    (9, 300, 64), (1, 14336, 4096), (1, 9000, 1024), (1, 300, 24), (1, 77, 6)):
        lab = f"{tname} few rows {(M, N, K)}"
        run_check(rng, dtype, tname, M, N, K, False, True, False, oracle_mod, lab)
        run_check(rng, dtype, tname, M, N, K, False, True, True, oracle_mod, lab + " int")


@pytest.mark.parametrize("dtype,tname", DTYPES)
def test_mixed_generic_explicit_and_unaligned(dtype, tname, oracle_mod):
    """The generic kernel asked for explicitly on the matrix-core layout, and
    operands that are only 2-byte aligned (the matrix-core tiles cannot take
    them; automatic dispatch falls back)."""
    rng = np.random.default_rng(30 + dtype)
    run_check(rng, dtype, tname, 300, 257, 130, False, True, False, oracle_mod,
              f"{tname} generic", variant=sg.VARIANT_GENERIC16)
    M, N, K = 130, 70, 66
    Ab = draw(rng, (M, K + 1), False, tname)
    Bb = draw(rng, (N, K + 1), False, tname)
    dA, dB = dev16(Ab, tname), dev16(Bb, tname)
    C = torch.empty((M, N), device=DEV)
    sg.gemm_mixed(dA[:, 1:], dB[:, 1:], C, trans_b=True)     # 2-byte aligned views
    torch.cuda.synchronize()
    As, Bs = np.ascontiguousarray(Ab[:, 1:]), np.ascontiguousarray(Bb[:, 1:])
    ref = oracle_mod.gemm_mixed(dtype, As, Bs, None, 1.0, 0.0, trans_b=True)
    r = max_err_ratio(C.cpu().numpy(), ref, K, 1.0, 0.0, decoded(As, tname), decoded(Bs, tname),
                      None)
    assert r <= 1.0, f"{tname} unaligned: {r}"


@pytest.mark.parametrize("dtype,tname", DTYPES)
def test_mixed_special_cases(dtype, tname, oracle_mod):
    """alpha == 0 and K == 0 scale C without reading A or B; M or N == 0 does
    nothing."""
    M, N, K = 40, 30, 20
    C0 = np.random.default_rng(1).uniform(-1, 1, (M, N)).astype(F32)
    nan = 0x7FC0 if dtype == sg.DTYPE_BF16 else 0x7E00
    An, Bn = np.full((M, K), nan, np.uint16), np.full((K, N), nan, np.uint16)
    C = torch.from_numpy(C0).to(DEV)
    sg.gemm_mixed(dev16(An, tname), dev16(Bn, tname), C, 0.0, -0.5)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), (-0.5 * C0).astype(F32))
    C = torch.from_numpy(C0).to(DEV)
    st = sg.sgemm_mixed(dtype, 0, 1, 0, N, K, 1.0, None, K, None, K, 0.0, C.data_ptr(), N)
    assert st == 0 and np.array_equal(C.cpu().numpy(), C0)


@pytest.mark.parametrize("dtype,tname", DTYPES)
@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (8192, 14336, 4096), (16, 14336, 4096)])
def test_mixed_full_size(shape, dtype, tname, oracle_mod):
    """Linear-layer shapes at full size (W stored N x K), sampled rows
    against the oracle; integers bit-exact."""
    M, N, K = shape
    rng = np.random.default_rng(M + dtype)
    rows = sample_rows(M, 12)
    run_check(rng, dtype, tname, M, N, K, False, True, True, oracle_mod, f"{tname} {shape}",
              rows=rows)
