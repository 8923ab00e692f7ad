"""GPU parity of strided-batched SGEMM (sgemm_strided_batched) against the
CPU oracle's batched entry point.

Every test is marked ``gpu``.  Floating-point inputs are held to the
tolerance in parity.py per batch entry; integer inputs must match bit for bit.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def draw(rng, shape, integer):
    if integer:
        return rng.integers(-4, 5, shape).astype(F32)
    return rng.uniform(-1, 1, shape).astype(F32)


def stacks(rng, batch, M, N, K, ta, tb, integer=False, share=None):
    """Stored operands (A as batch x K x M when ta, ...), and logical copies."""
    A = draw(rng, (batch, M, K), integer)
    B = draw(rng, (batch, K, N), integer)
    C0 = draw(rng, (batch, M, N), integer)
    if share == "A":
        A = np.broadcast_to(A[:1], A.shape).copy()
    if share == "B":
        B = np.broadcast_to(B[:1], B.shape).copy()
    As = np.ascontiguousarray(np.transpose(A, (0, 2, 1)) if ta else A)
    Bs = np.ascontiguousarray(np.transpose(B, (0, 2, 1)) if tb else B)
    return A, B, C0, As, Bs


def check(A, B, C0, alpha, beta, C, ref, exact, label):
    if exact:
        assert np.array_equal(C, ref), f"{label}: not bit-exact"
        return
    for b in range(C.shape[0]):
        r = max_err_ratio(C[b], ref[b], A.shape[2], alpha, beta, A[b], B[b],
                          None if C0 is None else C0[b])
        assert r <= 1.0, f"{label} entry {b}: max err/tol = {r}"


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_batched_shapes(ta, tb, oracle_mod):
    """Stacks of ragged and tile-sized products, every transposition,
    alpha/beta and beta = 0 over NaN, integers bit-exact; batches of tiny
    products (the small-product family takes them, A untransposed)."""
    rng = np.random.default_rng(int(ta) * 2 + int(tb))
    for batch, (M, N, K) in ((3, (300, 257, 129)), (7, (64, 64, 64)), (5, (128, 96, 33)),
                             (2, (1000, 300, 77)), (1, (37, 45, 5)), (16, (128, 128, 64)),
                             (300, (32, 32, 32)), (64, (16, 64, 128)), (40, (5, 33, 17))):
        for integer in (False, True):
            A, B, C0, As, Bs = stacks(rng, batch, M, N, K, ta, tb, integer)
            lab = f"batch {batch} {(M, N, K)} ta={ta} tb={tb} int={integer}"
            C = dev(C0)
            sg.gemm_batched(dev(As), dev(Bs), C, 0.5, -1.25, trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            ref = oracle_mod.sgemm_batched(As, Bs, C0.copy(), 0.5, -1.25, trans_a=ta, trans_b=tb)
            check(A, B, C0, 0.5, -1.25, C.cpu().numpy(), ref, integer, lab)
            Cn = torch.full((batch, M, N), float("nan"), device=DEV)
            sg.gemm_batched(dev(As), dev(Bs), Cn, 1.0, 0.0, trans_a=ta, trans_b=tb)
            torch.cuda.synchronize()
            ref = oracle_mod.sgemm_batched(As, Bs, None, 1.0, 0.0, trans_a=ta, trans_b=tb)
            check(A, B, None, 1.0, 0.0, Cn.cpu().numpy(), ref, integer, lab + " b0")


@pytest.mark.parametrize("share", ["A", "B"])
def test_batched_shared_operand(share, oracle_mod):
    """A stride of 0 shares one operand across the batch (one weight matrix
    for many inputs, or one input for many weights)."""
    rng = np.random.default_rng(5)
    batch, M, N, K = 6, 200, 136, 96
    A, B, C0, As, Bs = stacks(rng, batch, M, N, K, False, True, True, share)
    dA = dev(As[0]) if share == "A" else dev(As)
    dB = dev(Bs[0]) if share == "B" else dev(Bs)
    C = dev(C0)
    sg.gemm_batched(dA, dB, C, 0.5, -1.25, trans_b=True)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm_batched(As[0] if share == "A" else As, Bs[0] if share == "B" else Bs,
                                   C0.copy(), 0.5, -1.25, trans_b=True)
    check(A, B, C0, 0.5, -1.25, C.cpu().numpy(), ref, True, f"shared {share}")


def test_batched_padded_strides(oracle_mod):
    """Batch strides with gaps (NaN in A's and B's gaps must not leak; C's
    gaps and row padding keep their sentinel), odd strides (4-byte paths)."""
    rng = np.random.default_rng(9)
    for (batch, M, N, K, ga, gb, gc, pad) in ((4, 130, 70, 50, 12, 8, 4, 4),
                                               (3, 65, 33, 17, 3, 5, 1, 1)):
        A, B, C0, As, Bs = stacks(rng, batch, M, N, K, False, False)
        sa, sb = M * K + ga, K * N + gb
        ldc = N + pad
        sc = M * ldc + gc
        a = torch.full((batch * sa,), float("nan"), device=DEV)
        b = torch.full((batch * sb,), float("nan"), device=DEV)
        c = torch.full((batch * sc,), 777.0, device=DEV)
        for i in range(batch):
            a[i * sa: i * sa + M * K] = dev(As[i].reshape(-1))
            b[i * sb: i * sb + K * N] = dev(Bs[i].reshape(-1))
            c[i * sc: i * sc + M * ldc].view(M, ldc)[:, :N] = dev(C0[i])
        st = sg.sgemm_strided_batched(0, 0, M, N, K, 0.5, a.data_ptr(), K, sa, b.data_ptr(), N,
                                      sb, -1.25, c.data_ptr(), ldc, sc, batch,
                                      torch.cuda.current_stream().cuda_stream)
        assert st == 0, sg.status_string(st)
        torch.cuda.synchronize()
        ch = c.cpu().numpy()
        got = np.stack([ch[i * sc: i * sc + M * ldc].reshape(M, ldc)[:, :N] for i in range(batch)])
        for i in range(batch):
            blk = ch[i * sc: (i + 1) * sc]
            assert np.all(blk[M * ldc:] == 777.0), "C gap written"
            assert np.all(blk[:M * ldc].reshape(M, ldc)[:, N:] == 777.0), "C padding written"
        ref = oracle_mod.sgemm_batched(As, Bs, C0.copy(), 0.5, -1.25)
        check(A, B, C0, 0.5, -1.25, got, ref, False, f"padded {(M, N, K)}")


def test_batched_every_family(oracle_mod):
    """Explicit configurations over a batch: general and direct-load MFMA
    tiles, the VALU family, 4-byte I/O, and the skinny family."""
    rng = np.random.default_rng(13)
    batch, M, N, K = 4, 150, 130, 70
    A, B, C0, As, Bs = stacks(rng, batch, M, N, K, False, False, True)
    ref = oracle_mod.sgemm_batched(As, Bs, C0.copy(), 0.5, -1.25)
    configs = [(sg.VARIANT_VALU, 0, 0), (sg.VARIANT_MFMA, 0, 0), (sg.VARIANT_MFMA, 7, 0)]
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        f = sg.tile_info(sg.VARIANT_MFMA, t)["flags"]
        if f & sg.TILE_DIRECT and not f & (sg.TILE_WHOLE | sg.TILE_TRANS_A):
            configs += [(sg.VARIANT_MFMA, t, 0), (sg.VARIANT_MFMA, t, sg.FLAG_SCALAR_IO)]
    for variant, tile, flags in configs:
        C = dev(C0)
        sg.gemm_batched(dev(As), dev(Bs), C, 0.5, -1.25, variant=variant, tile=tile, flags=flags)
        torch.cuda.synchronize()
        check(A, B, C0, 0.5, -1.25, C.cpu().numpy(), ref, True, f"v{variant} t{tile} f{flags}")
    for M, N in ((5, 300), (300, 5)):
        A, B, C0, As, Bs = stacks(rng, batch, M, N, K, False, False, True)
        C = dev(C0)
        sg.gemm_batched(dev(As), dev(Bs), C, 0.5, -1.25)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm_batched(As, Bs, C0.copy(), 0.5, -1.25)
        check(A, B, C0, 0.5, -1.25, C.cpu().numpy(), ref, True, f"skinny {(M, N)}")


def test_batched_more_than_one_launch(oracle_mod):
    """More entries than one launch's grid holds (65535): the batch is split
    over launches."""
    rng = np.random.default_rng(17)
    batch, M, N, K = 70001, 2, 3, 4
    A, B, C0, As, Bs = stacks(rng, batch, M, N, K, False, False, True)
    C = dev(C0)
    sg.gemm_batched(dev(As), dev(Bs), C, 0.5, -1.25)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm_batched(As, Bs, C0.copy(), 0.5, -1.25, nthreads=1)
    assert np.array_equal(C.cpu().numpy(), ref)


def test_batched_attention_shapes(oracle_mod):
    """The shapes of attention over heads: scores Q K^T (B stored
    transposed) and the weighted sum P V, 32 heads of 256 x 256 x 64."""
    rng = np.random.default_rng(19)
    heads, S, D = 32, 256, 64
    Q = rng.uniform(-1, 1, (heads, S, D)).astype(F32)
    Kt = rng.uniform(-1, 1, (heads, S, D)).astype(F32)
    V = rng.uniform(-1, 1, (heads, S, D)).astype(F32)
    scores = sg.gemm_batched(dev(Q), dev(Kt), None, 0.125, 0.0, trans_b=True)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm_batched(Q, Kt, None, 0.125, 0.0, trans_b=True)
    check(Q, np.transpose(Kt, (0, 2, 1)), None, 0.125, 0.0, scores.cpu().numpy(), ref, False,
          "scores")
    P = rng.uniform(0, 1.0 / S, (heads, S, S)).astype(F32)
    out = sg.gemm_batched(dev(P), dev(V), None, 1.0, 0.0)
    torch.cuda.synchronize()
    ref = oracle_mod.sgemm_batched(P, V, None, 1.0, 0.0)
    check(P, V, None, 1.0, 0.0, out.cpu().numpy(), ref, False, "weighted sum")


def test_batched_short_k_automatic(oracle_mod):
    """Attention scores at a size where the automatic plan takes the
    short-K rule (K = 128, two full rounds of 128 x 128 tiles): 8 heads of
    1024 x 1024 x 128 with B stored transposed, and the same through the
    persistent schedule of a 256-row tile; small-integer inputs, so every
    result must equal the oracle's bit for bit."""
    rng = np.random.default_rng(23)
    heads, S, D = 8, 1024, 128
    Q = rng.integers(-4, 5, (heads, S, D)).astype(F32)
    Kt = rng.integers(-4, 5, (heads, S, D)).astype(F32)
    ref = oracle_mod.sgemm_batched(Q, Kt, None, 0.5, 0.0, trans_b=True)
    got = sg.gemm_batched(dev(Q), dev(Kt), None, 0.5, 0.0, trans_b=True)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref), "automatic plan differs from the oracle"
    sk = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
          if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_STREAMK
          and not sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_TRANS_A]
    if sk:
        got = sg.gemm_batched(dev(Q), dev(Kt), None, 0.5, 0.0, trans_b=True,
                              variant=sg.VARIANT_MFMA, tile=sk[0], flags=sg.FLAG_STREAMK)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref), "persistent schedule differs"
