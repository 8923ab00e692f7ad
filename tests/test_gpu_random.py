"""GPU parity on seeded random problems: shapes, storage orders, padded
leading dimensions, operands starting 1-3 floats past a 16-byte boundary,
alpha and beta (0 and 1 among them), batches and 16-bit inputs, all through
automatic dispatch, against the CPU oracle.

Inputs are mostly integers in [-4, 4] and alpha, beta small dyadic
rationals, so every product and sum is exact in fp32 and the whole of C must
match the oracle bit for bit whatever kernel, tile, split or summation order
the library picks; a third of the single products take uniform [-1, 1]
inputs held to the fp32 tolerance.  With beta = 0, C starts as NaN (C is
never read).  The shape draws mix tiny problems, skinny ones (M or N up to
16, long K), mid-size ragged ones and a few that span many tiles, so that
every kernel family and its edge paths are reached.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
from parity import max_err_ratio

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"
SCALARS = (0.0, 1.0, -1.0, 0.5, -1.25, 2.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def draw_shape(rng):
    kind = rng.integers(0, 5)
    if kind == 0:   # tiny
        return tuple(int(v) for v in rng.integers(1, 40, 3))
    if kind == 1:   # few rows or few columns, long K
        small, wide = int(rng.integers(1, 17)), int(rng.integers(1, 3000))
        k = int(rng.integers(1, 6000))
        return (small, wide, k) if rng.integers(0, 2) else (wide, small, k)
    if kind == 2:   # mid-size, ragged
        return tuple(int(v) for v in rng.integers(40, 700, 3))
    if kind == 3:   # short K
        return int(rng.integers(100, 1500)), int(rng.integers(100, 1500)), int(rng.integers(1, 40))
    return int(rng.integers(500, 1300)), int(rng.integers(500, 1300)), int(rng.integers(200, 1200))


def placed(x: np.ndarray, pad: int, offset: int):
    """x (rows x cols) on the device inside a NaN-filled buffer with leading
    dimension cols + pad, its first element `offset` floats into the buffer."""
    rows, cols = x.shape
    ld = cols + pad
    buf = torch.full((offset + rows * ld + 1,), float("nan"), device=DEV)
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(DEV))
    return view


@pytest.mark.parametrize("block", range(8))
def test_random_problems(block, oracle_mod):
    """20 problems per block: random shape, storage order of A and B,
    padding (0-5 floats) and start offset (0-3 floats) of each operand and of
    C, alpha and beta.  Every third problem takes uniform [-1, 1] inputs,
    held to the fp32 tolerance instead of bit for bit."""
    rng = np.random.default_rng(9100 + block)
    for case in range(20):
        M, N, K = draw_shape(rng)
        ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        alpha = float(rng.choice(SCALARS[1:]))
        beta = float(rng.choice(SCALARS))
        exact = case % 3 != 2
        if exact:
            A = rng.integers(-4, 5, (M, K)).astype(F32)
            B = rng.integers(-4, 5, (K, N)).astype(F32)
            C0 = rng.integers(-4, 5, (M, N)).astype(F32)
        else:
            A = rng.uniform(-1, 1, (M, K)).astype(F32)
            B = rng.uniform(-1, 1, (K, N)).astype(F32)
            C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        pads = [int(v) for v in rng.integers(0, 6, 3)]
        offs = [int(v) for v in rng.integers(0, 4, 3)]
        dA, dB = placed(As, pads[0], offs[0]), placed(Bs, pads[1], offs[1])
        if beta == 0.0:
            dC = placed(np.full((M, N), np.nan, dtype=F32), pads[2], offs[2])
        else:
            dC = placed(C0, pads[2], offs[2])
        label = (f"block {block} case {case}: {(M, N, K)} ta={ta} tb={tb} alpha={alpha} "
                 f"beta={beta} pads={pads} offsets={offs}")
        print(label, flush=True)
        sg.gemm(dA, dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm(As, Bs, C0.copy(), alpha, beta, trans_a=ta, trans_b=tb)
        got = dC.cpu().numpy()
        if exact:
            assert np.array_equal(got, ref), \
                f"{label}: {int(np.sum(got != ref))} of {M * N} elements differ"
        else:
            r = max_err_ratio(got, ref, K, alpha, beta, A, B, C0 if beta != 0.0 else None)
            assert r <= 1.0, f"{label} (uniform): max err/tol = {r}"


@pytest.mark.parametrize("block", range(2))
def test_random_batches(block, oracle_mod):
    """Strided batches of random shapes and storage orders, B shared by the
    batch (batch stride 0) in half of them."""
    rng = np.random.default_rng(9200 + block)
    for case in range(10):
        M, N, K = (int(v) for v in rng.integers(1, 200, 3))
        bat = int(rng.integers(1, 40))
        ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        shared = bool(rng.integers(0, 2))
        alpha, beta = float(rng.choice(SCALARS[1:])), float(rng.choice(SCALARS[1:]))
        A = rng.integers(-4, 5, (bat, M, K)).astype(F32)
        B = rng.integers(-4, 5, (1 if shared else bat, K, N)).astype(F32)
        C0 = rng.integers(-4, 5, (bat, M, N)).astype(F32)
        As = np.ascontiguousarray(A.transpose(0, 2, 1)) if ta else A
        Bs = np.ascontiguousarray(B.transpose(0, 2, 1)) if tb else B
        dB = torch.from_numpy(Bs[0] if shared else Bs).to(DEV)
        dC = torch.from_numpy(C0).to(DEV)
        label = (f"batch block {block} case {case}: {bat} x {(M, N, K)} ta={ta} tb={tb} "
                 f"shared={shared}")
        print(label, flush=True)
        sg.gemm_batched(torch.from_numpy(As).to(DEV), dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm_batched(As, Bs[0] if shared else Bs, C0.copy(), alpha, beta,
                                       trans_a=ta, trans_b=tb)
        assert np.array_equal(dC.cpu().numpy(), ref), label


@pytest.mark.parametrize("tname", ["bfloat16", "float16"])
def test_random_16bit(tname, oracle_mod):
    """16-bit inputs (C = X W^T with W stored N x K, and other storage orders
    through the generic kernel) on random shapes; integers in [-4, 4] are
    exact in both formats and their products and sums exact in fp32."""
    dtype = getattr(torch, tname)
    rng = np.random.default_rng(9300 + (tname == "float16"))
    for case in range(16):
        M, N, K = draw_shape(rng)
        if case % 4 == 3:
            ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        else:
            ta, tb = False, True
        alpha, beta = float(rng.choice(SCALARS[1:])), float(rng.choice(SCALARS))
        A = rng.integers(-4, 5, (M, K)).astype(F32)
        B = rng.integers(-4, 5, (K, N)).astype(F32)
        C0 = rng.integers(-4, 5, (M, N)).astype(F32)
        As = np.ascontiguousarray(A.T) if ta else A
        Bs = np.ascontiguousarray(B.T) if tb else B
        dC = torch.from_numpy(C0 if beta != 0.0 else np.full((M, N), np.nan, dtype=F32)).to(DEV)
        label = f"{tname} case {case}: {(M, N, K)} ta={ta} tb={tb} alpha={alpha} beta={beta}"
        print(label, flush=True)
        dA = torch.from_numpy(As).to(DEV).to(dtype)
        dB = torch.from_numpy(Bs).to(DEV).to(dtype)
        sg.gemm_mixed(dA, dB, dC, alpha, beta, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm(As, Bs, C0.copy(), alpha, beta, trans_a=ta, trans_b=tb)
        assert np.array_equal(dC.cpu().numpy(), ref), label
