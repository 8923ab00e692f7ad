"""GPU parity of the small-product family (VARIANT_SMALL) against the CPU
oracle, every compiled tile asked for explicitly.

The shapes make each part of the kernel's indexing work: several workgroups
with ragged last tiles in M and N, K under one 16-wide chunk, K not a
multiple of 4 (4-byte loads of A), k-groups whose share of K is empty
(K = 33 with 8 k-groups), rows that are not 16-byte aligned (padded leading
dimensions, offset views), B stored transposed, alpha/beta with beta = 0
over a NaN-filled C, the fused bias/activation epilogue, and batches.
Integer-valued inputs must match bit for bit (every partial sum is exact in
fp32); uniform inputs are held to the tolerance in parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
import workloads
from parity import epilogue_err_ratio, max_err_ratio

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"
SHAPES = [(256, 256, 256), (777, 777, 33), (1, 1, 1), (17, 33, 5), (100, 64, 1000),
          (65, 130, 64), (48, 300, 18)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def small_tiles():
    return list(range(sg.tile_count(sg.VARIANT_SMALL)))


def to_dev(x):
    """x on the device with its row padding: a column-sliced view of a padded
    array (workloads.padded) keeps the padded leading dimension."""
    if x.flags.c_contiguous:
        return dev(x)
    return dev(x.base)[:x.shape[0], :x.shape[1]]


def run(A, B, C0, alpha, beta, tb, tile, **kw):
    """A (M x K) and B (K x N, or N x K with tb) as stored."""
    M = A.shape[0]
    N = B.shape[0] if tb else B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dA, dB, C, alpha, beta, trans_b=tb, variant=sg.VARIANT_SMALL, tile=tile, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


@pytest.mark.parametrize("tile", small_tiles())
def test_small_tile_integer_bit_exact(tile, oracle_mod):
    for (M, N, K) in SHAPES:
        A, B, C0 = workloads.draw(M, N, K, "int4", 7 + tile, True)
        for tb in (False, True):
            Bs = np.ascontiguousarray(B.T) if tb else B
            ref = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
            C = run(A, Bs, C0, 0.5, -1.25, tb, tile)
            assert np.array_equal(C, ref), f"tile {tile} {(M, N, K)} tb={tb}"


@pytest.mark.parametrize("tile", small_tiles())
def test_small_tile_uniform(tile, oracle_mod):
    for (M, N, K) in SHAPES:
        A, B, _ = workloads.draw(M, N, K, "uniform", 3, False)
        ref = oracle_mod.sgemm(A, B)
        C = run(A, B, None, 1.0, 0.0, False, tile)   # C starts as NaN: beta = 0 never reads it
        r = max_err_ratio(C, ref, K, 1.0, 0.0, A, B, None)
        assert r <= 1.0, f"tile {tile} {(M, N, K)}: {r}"


@pytest.mark.parametrize("tile", small_tiles())
def test_small_tile_unaligned_rows(tile, oracle_mod):
    """Leading dimensions that are not multiples of 4 and operands that start
    one float into their buffer: every load and store takes the 4-byte path."""
    M, N, K = 70, 90, 60
    A, B, C0 = workloads.draw(M, N, K, "int4", 5, True)
    Ap = workloads.padded(A, 3, np.nan)[:, :K]
    Bp = workloads.padded(B, 1, np.nan)[:, :N]
    ref = oracle_mod.sgemm(A, B, C0.copy(), 1.0, 1.0)
    C = run(Ap, Bp, C0, 1.0, 1.0, False, tile)
    assert np.array_equal(C, ref), f"tile {tile} padded"
    # offset views: row starts one float past a 16-byte boundary
    dA = dev(np.concatenate([np.zeros(1, F32), A.ravel()]))[1:].view(M, K)
    dB = dev(np.concatenate([np.zeros(1, F32), B.ravel()]))[1:].view(K, N)
    Cd = dev(C0)
    sg.gemm(dA, dB, Cd, 1.0, 1.0, variant=sg.VARIANT_SMALL, tile=tile)
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), ref), f"tile {tile} offset"


@pytest.mark.parametrize("tile", small_tiles())
def test_small_tile_epilogue(tile, oracle_mod):
    M, N, K = 100, 200, 48
    A, B, C0 = workloads.draw(M, N, K, "uniform", 9, True)
    bias = np.random.default_rng(4).uniform(-1, 1, N).astype(F32)
    x = oracle_mod.sgemm(A, B, C0.copy(), 1.0, 0.5, bias=bias, act=sg.ACT_NONE)
    for act in (sg.ACT_RELU, sg.ACT_GELU_TANH):
        ref = oracle_mod.sgemm(A, B, C0.copy(), 1.0, 0.5, bias=bias, act=act)
        C = dev(C0)
        sg.gemm(dev(A), dev(B), C, 1.0, 0.5, bias=dev(bias), act=act, variant=sg.VARIANT_SMALL,
                tile=tile)
        torch.cuda.synchronize()
        r = epilogue_err_ratio(C.cpu().numpy(), ref, x, K, 1.0, 0.5, A, B, C0, bias, act)
        assert r <= 1.0, f"tile {tile} act {act}: {r}"


@pytest.mark.parametrize("tile", small_tiles())
def test_small_tile_batched(tile, oracle_mod):
    bat, M, N, K = 5, 40, 72, 36
    rng = np.random.default_rng(12)
    A = rng.integers(-4, 5, (bat, M, K)).astype(F32)
    B = rng.integers(-4, 5, (bat, K, N)).astype(F32)
    ref = oracle_mod.sgemm_batched(A, B)
    C = sg.gemm_batched(dev(A), dev(B), variant=sg.VARIANT_SMALL, tile=tile)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), ref), f"tile {tile} batched"


def test_small_rejects_transposed_a():
    A = torch.ones((8, 8), device=DEV)
    with pytest.raises(sg.SgemmError):
        sg.gemm(A, A, trans_a=True, variant=sg.VARIANT_SMALL, tile=0)
