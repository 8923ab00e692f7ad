"""GPU parity of the direct-load tiles' split-tail loads.

A k-contiguous operand (A untransposed, B stored transposed) whose rows are
only 4-byte aligned, or whose K is not a multiple of 4, is read with 16-byte
loads from unaligned addresses, and its last k stage float by float so that
nothing past K enters a sum.  Each case is built so that a wrong tail fails:
the rows' padding is NaN (a 16-byte load that ran past K would bring NaN into
the product), K leaves every remainder 1..3 past the last whole chunk as well
as stages shorter than one chunk, the operands start 1-3 floats past a
16-byte boundary, and M and N are ragged so that rows outside the matrix
meet the tail stage.  Integer-valued inputs match the oracle bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def nan_padded(x: np.ndarray, pad: int, offset: int):
    """x (rows x cols) on the device inside a NaN-filled buffer: leading
    dimension cols + pad, first element `offset` floats into the buffer."""
    rows, cols = x.shape
    ld = cols + pad
    buf = torch.full((offset + rows * ld,), float("nan"), device=DEV)
    view = buf[offset:].view(rows, ld)[:, :cols]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to(DEV))
    return view


def direct_tiles(trans_b: bool):
    """Direct-load tiles with edges for untransposed A (that serve B^T too)."""
    out = []
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        f = sg.tile_info(sg.VARIANT_MFMA, t)["flags"]
        if f & sg.TILE_DIRECT and not f & (sg.TILE_WHOLE | sg.TILE_TRANS_A):
            if not trans_b or f & sg.TILE_TRANS_B:
                out.append(t)
    return out


def k_values(bk: int):
    """Stages shorter than one 4-float chunk, a remainder of 1..3 after whole
    chunks inside one stage, and after one or more whole stages."""
    return [1, 2, 3, 5, bk - 1, bk + 1, 2 * bk + 2, 3 * bk + 3]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("slot", range(12))
def test_split_tail_tiles(slot, trans_b, oracle_mod):
    tl = direct_tiles(trans_b)
    if slot >= len(tl):
        pytest.skip("no such tile")
    tile = tl[slot]
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    M, N = bm + 5, bn + 3
    rng = np.random.default_rng(100 * tile + int(trans_b))
    # (K, A's row padding, A's start offset, the same for B^T): every padding
    # and offset; with K a multiple of 4 one operand aligned and the other not
    cases = [(K, i % 4, (3 * i + 1) % 4, (i + 1) % 4, (3 * i + 3) % 4)
             for i, K in enumerate(k_values(bk))]
    cases += [(4 * bk + 8, 0, 0, 1, 2), (4 * bk + 8, 3, 1, 0, 0)]
    for K, pad, off, bpad, boff in cases:
        A = rng.integers(-4, 5, (M, K)).astype(F32)
        B = rng.integers(-4, 5, (K, N)).astype(F32)
        C0 = rng.integers(-4, 5, (M, N)).astype(F32)
        dA = nan_padded(A, pad, off)
        if trans_b:
            dB = nan_padded(np.ascontiguousarray(B.T), bpad, boff)
        else:
            dB = torch.from_numpy(B).to(DEV)
        C = torch.from_numpy(C0).to(DEV)
        sg.gemm(dA, dB, C, 0.5, -1.25, trans_b=trans_b, variant=sg.VARIANT_MFMA, tile=tile)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
        got = C.cpu().numpy()
        assert np.array_equal(got, ref), \
            f"tile {tile} tb={trans_b} K={K} A pad/off {pad}/{off} B^T {bpad}/{boff}: " \
            f"{int(np.sum(got != ref))} elements differ"


@pytest.mark.parametrize("shape", [(4097, 1000, 3001), (1000, 777, 1001), (300, 4100, 258)])
def test_split_tail_automatic(shape, oracle_mod):
    """Automatic dispatch of unaligned, odd-K products (the ragged workload's
    4097 x 1000 x 3001 among them): rows sampled through every row tile."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    A = rng.integers(-4, 5, (M, K)).astype(F32)
    B = rng.integers(-4, 5, (K, N)).astype(F32)
    for trans_b in (False, True):
        dA = nan_padded(A, 1, 3)
        dB = nan_padded(np.ascontiguousarray(B.T), 2, 1) if trans_b else \
            torch.from_numpy(B).to(DEV)
        C = torch.full((M, N), float("nan"), device=DEV)
        sg.gemm(dA, dB, C, trans_b=trans_b)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(0, M, 61), [M - 1]]))
        ref = oracle_mod.sgemm(np.ascontiguousarray(A[rows]), B)
        got = C.cpu().numpy()[rows]
        assert np.array_equal(got, ref), f"{shape} tb={trans_b}"


@pytest.mark.parametrize("tname", ["bfloat16", "float16"])
def test_split_tail_16bit(tname, oracle_mod):
    """16-bit inputs (C = X W^T): word rows that are 4-byte but not 16-byte
    aligned and K a multiple of 2 but not of 8, NaN in the row padding."""
    dtype = sg.DTYPE_BF16 if tname == "bfloat16" else sg.DTYPE_F16
    nan_bits = np.int16(0x7FC0) if tname == "bfloat16" else np.int16(0x7E00)
    tdt = getattr(torch, tname)
    rng = np.random.default_rng(7 + dtype)
    for i, (M, N, K) in enumerate(((300, 257, 130), (37, 45, 6), (256, 256, 66), (5, 700, 2),
                                   (513, 129, 258))):
        pad, off = 2 * (i % 3 + 1), 2 * (i % 2 + 1)   # in 16-bit elements: 4-byte aligned
        x = rng.integers(-4, 5, (M, K)).astype(F32)
        w = rng.integers(-4, 5, (N, K)).astype(F32)
        ops = []
        for v, p_, o_ in ((x, pad, off), (w, pad + 2, 2)):
            rows, cols = v.shape
            buf = torch.full((o_ + rows * (cols + p_),), int(nan_bits), dtype=torch.int16,
                             device=DEV)
            view = buf.view(tdt)[o_:].view(rows, cols + p_)[:, :cols]
            view.copy_(torch.from_numpy(v).to(DEV).to(tdt))
            ops.append(view)
        C = torch.full((M, N), float("nan"), device=DEV)
        sg.gemm_mixed(ops[0], ops[1], C, trans_b=True)
        torch.cuda.synchronize()
        xb = torch.from_numpy(x).to(tdt).view(torch.int16).numpy()
        wb = torch.from_numpy(w).to(tdt).view(torch.int16).numpy()
        ref = oracle_mod.gemm_mixed(dtype, xb.view(np.uint16), wb.view(np.uint16), None, 1.0,
                                    0.0, trans_b=True)
        assert np.array_equal(C.cpu().numpy(), ref), f"{tname} {(M, N, K)} pad={pad} off={off}"
