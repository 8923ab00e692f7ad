"""Helpers for comparing the GPU path with the CPU oracle.

Tolerance (elementwise, on the oracle's fp32 output C_ref):
    |C_gpu - C_ref| <= 2e-5 * K * |alpha| * max|A| * max|B| + 1e-6 * |beta| * |C0|
with max|A|, max|B| over the whole input matrices and C0 the initial C at the
same cell.  Integer-valued inputs (every partial sum exact in fp32) are
compared bit for bit instead.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def tolerance(K, alpha, beta, A, B, C0):
    if alpha == 0 or K == 0:
        tol = 0.0   # no product term (A and B are not read, and may hold NaN)
    else:
        amax = float(np.abs(A).max()) if A.size else 0.0
        bmax = float(np.abs(B).max()) if B.size else 0.0
        tol = 2e-5 * K * abs(alpha) * amax * bmax
    if beta != 0 and C0 is not None:
        return tol + 1e-6 * abs(beta) * np.abs(C0.astype(np.float64))
    return np.full(1, tol)


def max_err_ratio(C, Cref, K, alpha, beta, A, B, C0) -> float:
    """max over cells of |C - Cref| / tol (<= 1 passes); inf on NaN mismatch."""
    C = np.asarray(C, dtype=np.float64)
    Cref = np.asarray(Cref, dtype=np.float64)
    if C.shape != Cref.shape:
        raise AssertionError(f"shape {C.shape} vs {Cref.shape}")
    if not np.array_equal(np.isnan(C), np.isnan(Cref)):
        return float("inf")
    err = np.abs(np.nan_to_num(C) - np.nan_to_num(Cref))
    tol = tolerance(K, alpha, beta, A, B, C0)
    if C0 is not None and beta != 0:
        tol = np.broadcast_to(tol, C.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / np.maximum(tol, 1e-300))
    return float(r.max()) if r.size else 0.0


def sample_rows(M: int, count: int, seed: int = 99) -> np.ndarray:
    """First, last and random distinct rows (sorted), for checks at sizes the
    oracle cannot finish whole in seconds."""
    if M <= count:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1, M // 2])
    rows.update(rng.choice(M, count - len(rows), replace=False).tolist())
    while len(rows) < count:
        rows.add(int(rng.integers(M)))
    return np.array(sorted(rows))


# Largest slope of each activation (0 none, 1 ReLU, 2 SiLU, 3 GELU erf, 4
# GELU tanh): max |act'(x)| is 1 for the first two and about 1.100 and 1.129
# for SiLU and GELU.
ACT_LIPSCHITZ = {0: 1.0, 1: 1.0, 2: 1.1, 3: 1.13, 4: 1.13}
EPS32 = 2.0 ** -23


def epilogue_err_ratio(C, Cref, Xref, K, alpha, beta, A, B, C0, bias, act) -> float:
    """max |C - Cref| / tol for C = act(alpha AB + beta C0 + bias), with
        tol = L (tol_gemm + eps (|x| + |bias|)) + 5 eps |Cref|
    elementwise: the product's tolerance and the rounding of the bias add,
    carried through the activation's slope L, plus a few fp32 ulp of the
    activation's own evaluation.  Xref is the oracle's pre-activation sum."""
    C = np.asarray(C, dtype=np.float64)
    Cref = np.asarray(Cref, dtype=np.float64)
    X = np.abs(np.asarray(Xref, dtype=np.float64))
    if not np.array_equal(np.isnan(C), np.isnan(Cref)):
        return float("inf")
    tol = np.broadcast_to(tolerance(K, alpha, beta, A, B, C0), C.shape)
    b = 0.0 if bias is None else np.abs(bias.astype(np.float64))[None, :]
    tol = ACT_LIPSCHITZ[act] * (tol + EPS32 * (X + b)) + 5 * EPS32 * np.abs(Cref)
    err = np.abs(np.nan_to_num(C) - np.nan_to_num(Cref))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / np.maximum(tol, 1e-300))
    return float(r.max()) if r.size else 0.0
