"""Pins for the CPU oracle: checks that tie it to the mathematics, not to itself.

Each pin calls an oracle entry point through ``call(M, N, K, alpha, A, lda,
B, ldb, beta, C, ldc) -> status`` on flat float32 buffers, so the same pins run
against the real oracle and against deliberately broken copies of it (see
test_oracle.py).  The pins are:

  brute_force   exact rational arithmetic (fractions.Fraction) on every shape
                with M, N, K in 1..4, random fp32 entries and random alpha/beta:
                the oracle must equal the correctly rounded fp32 value of the
                exact result, up to the fp64 summation error bound.
  identity      A = I gives C = B, B = I gives C = A, exactly.
  ones          all-ones A and B give C = K exactly.
  permutation   B a permutation matrix gives an exact column shuffle of A.
  one_hot       a single 1 in A and in B gives a single 1 in C at (i, j).
  beta0_nan     beta = 0 never reads C: NaN-filled C gives a finite result.
  alpha0_nan    alpha = 0 never reads A or B: C = beta * C exactly.
  ld_padding    NaN in the row padding of A and B does not leak; C's padding
                is left untouched.
  transposed    (entry point with op(A), op(B)) exact rational brute force for
                every combination of transposed storage, a permutation stored
                transposed, padded rows of transposed operands, and the
                argument checks of the transposed leading dimensions.
  epilogue      (entry point with bias and activation) every cell against the
                activation of the exact rational sum plus bias, evaluated at
                40 significant digits (mpmath; GELU through mpmath's normal
                CDF, its tanh form and SiLU as printed in their papers) and
                rounded to fp32: within one fp32 ulp; ReLU and bias exact on
                integers; the alpha = 0 path; act codes checked.
  mixed         (16-bit inputs) the decoding of listed bfloat16 / float16 bit
                patterns against the values their formats define, every finite
                pattern against numpy's binary16 (float16) or the binary32
                embedding (bfloat16), and exact rational brute force on
                random 16-bit inputs for every transposition.
  batched       (strided-batched entry point) exact rational brute force on
                every matrix of a batch with padded, shared (stride 0) and
                transposed operands; batch = 0 touches nothing; stride and
                batch checks.

The definition pinned: C = alpha * (A * B) + beta * C, each cell a dot product
of a row of A and a column of B ("a CUDA matmul" section 00; "The GEMM
Scrapbook" introduction; "The 1% kernel" section 1).
"""
from __future__ import annotations

from fractions import Fraction

import mpmath
import numpy as np

F32 = np.float32


def rn32(x: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) float32 value of a rational."""
    if x == 0:
        return 0.0
    f = np.float32(float(x))
    best, best_key = None, None
    for c in (np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))):
        key = (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1)
        if best_key is None or key < best_key:
            best, best_key = float(c), key
    return best


def exact_cell(A, B, C0, i, j, alpha, beta):
    """(exact value, magnitude bound) of alpha * sum_k A[i,k] B[k,j] + beta * C0[i,j]."""
    K = A.shape[1]
    terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
    a = Fraction(float(alpha))
    b = Fraction(float(beta))
    if alpha == 0 or K == 0:
        val = Fraction(0) if beta == 0 else b * Fraction(float(C0[i, j]))
        return val, abs(val)
    val = a * sum(terms, Fraction(0))
    mag = abs(a) * sum((abs(t) for t in terms), Fraction(0))
    if beta != 0:
        bc = b * Fraction(float(C0[i, j]))
        val += bc
        mag += abs(bc)
    return val, mag


def within_fp64_rounding(r: float, exact: Fraction, mag: Fraction, K: int) -> bool:
    """r must lie between RN32(exact - d) and RN32(exact + d), where d bounds the
    error of summing K exact products and the epilogue in fp64."""
    d = Fraction(K + 4, 2 ** 52) * mag
    return rn32(exact - d) <= r <= rn32(exact + d)


def run(call, A, B, C0, alpha, beta, lda=None, ldb=None, ldc=None):
    """Call the oracle on dense copies; returns (status, C)."""
    M, K = A.shape
    N = B.shape[1]
    A_ = np.ascontiguousarray(A, dtype=F32).reshape(-1)
    B_ = np.ascontiguousarray(B, dtype=F32).reshape(-1)
    C = (np.ascontiguousarray(C0, dtype=F32).copy() if C0 is not None
         else np.full((M, N), np.nan, dtype=F32))
    st = call(M, N, K, alpha, A_, lda or max(K, 1), B_, ldb or max(N, 1), beta,
              C.reshape(-1), ldc or max(N, 1))
    return st, C


def pin_brute_force(call, rng, dims=range(1, 5)) -> list[str]:
    fails = []
    for M in dims:
        for N in dims:
            for K in dims:
                A = rng.uniform(-2, 2, (M, K)).astype(F32)
                B = rng.uniform(-2, 2, (K, N)).astype(F32)
                C0 = rng.uniform(-2, 2, (M, N)).astype(F32)
                for alpha, beta in ((1.0, 0.0), (float(F32(rng.uniform(-3, 3))),
                                                 float(F32(rng.uniform(-3, 3))))):
                    st, C = run(call, A, B, C0 if beta != 0 else None, alpha, beta)
                    if st != 0:
                        fails.append(f"brute_force status {st} at {(M, N, K)}")
                        continue
                    for i in range(M):
                        for j in range(N):
                            ex, mag = exact_cell(A, B, C0, i, j, alpha, beta)
                            if not within_fp64_rounding(float(C[i, j]), ex, mag, K):
                                fails.append(f"brute_force {(M, N, K)} cell {(i, j)}: "
                                             f"{C[i, j]!r} vs exact {float(ex)!r}")
                                break
    return fails


def pin_closed_forms(call, rng) -> list[str]:
    fails = []
    # identity on both sides, ragged shapes
    for (M, K) in ((5, 5), (17, 17), (33, 33)):
        I = np.eye(K, dtype=F32)
        for N in (1, 7, 40):
            B = rng.uniform(-1, 1, (K, N)).astype(F32)
            st, C = run(call, I, B, None, 1.0, 0.0)
            if st or not np.array_equal(C, B):
                fails.append(f"identity-left {(M, N, K)}")
            A = rng.uniform(-1, 1, (N, K)).astype(F32)
            st, C = run(call, A, I, None, 1.0, 0.0)
            if st or not np.array_equal(C, A):
                fails.append(f"identity-right {(N, K)}")
    # all ones: C = K
    for (M, N, K) in ((3, 5, 7), (16, 9, 100), (1, 1, 1000)):
        st, C = run(call, np.ones((M, K), F32), np.ones((K, N), F32), None, 1.0, 0.0)
        if st or not np.all(C == F32(K)):
            fails.append(f"ones {(M, N, K)}")
    # permutation: B = P with P[perm[j], j] = 1, so C[:, j] = A[:, perm[j]]
    for (M, K) in ((6, 11), (13, 29)):
        perm = rng.permutation(K)
        P = np.zeros((K, K), F32)
        P[perm, np.arange(K)] = 1.0
        A = rng.uniform(-1, 1, (M, K)).astype(F32)
        st, C = run(call, A, P, None, 1.0, 0.0)
        if st or not np.array_equal(C, A[:, perm]):
            fails.append(f"permutation {(M, K)}")
    # one-hot: A = e_i e_k^T, B = e_k e_j^T -> single 1 at (i, j)
    M, N, K = 7, 9, 5
    for (i, j, k) in ((0, 0, 0), (6, 8, 4), (3, 1, 2)):
        A = np.zeros((M, K), F32); A[i, k] = 1
        B = np.zeros((K, N), F32); B[k, j] = 1
        st, C = run(call, A, B, None, 1.0, 0.0)
        E = np.zeros((M, N), F32); E[i, j] = 1
        if st or not np.array_equal(C, E):
            fails.append(f"one_hot {(i, j, k)}")
    return fails


def pin_alpha_beta(call, rng) -> list[str]:
    fails = []
    M, N, K = 9, 11, 13
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    # beta == 0: C must not be read
    st, C = run(call, A, B, np.full((M, N), np.nan, F32), 1.5, 0.0)
    if st or not np.all(np.isfinite(C)):
        fails.append("beta0_nan")
    # alpha == 0: A and B must not be read; C = beta * C exactly (beta = 0.5)
    C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
    st, C = run(call, np.full((M, K), np.nan, F32), np.full((K, N), np.nan, F32),
                C0, 0.0, 0.5)
    if st or not np.array_equal(C, C0 * F32(0.5)):
        fails.append("alpha0_nan")
    # alpha == 0, beta == 0: zero fill without reading anything
    st, C = run(call, np.full((M, K), np.nan, F32), np.full((K, N), np.nan, F32),
                np.full((M, N), np.nan, F32), 0.0, 0.0)
    if st or not np.all(C == 0):
        fails.append("alpha0_beta0")
    # integer-valued alpha/beta case: exact
    Ai = rng.integers(-4, 5, (M, K)).astype(F32)
    Bi = rng.integers(-4, 5, (K, N)).astype(F32)
    Ci = rng.integers(-4, 5, (M, N)).astype(F32)
    st, C = run(call, Ai, Bi, Ci, 0.5, -1.25)
    want = (0.5 * (Ai.astype(np.int64) @ Bi.astype(np.int64)) - 1.25 * Ci).astype(F32)
    if st or not np.array_equal(C, want):
        fails.append("alpha_beta_integer")
    return fails


def pin_ld_padding(call, rng) -> list[str]:
    fails = []
    M, N, K = 7, 10, 6
    pa, pb, pc = 3, 5, 2
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
    As = np.full((M, K + pa), np.nan, F32); As[:, :K] = A
    Bs = np.full((K, N + pb), np.nan, F32); Bs[:, :N] = B
    Cs = np.full((M, N + pc), 777.0, F32); Cs[:, :N] = C0
    st = call(M, N, K, 1.0, As.reshape(-1), K + pa, Bs.reshape(-1), N + pb, 1.0,
              Cs.reshape(-1), N + pc)
    _, Ctight = run(call, A, B, C0, 1.0, 1.0)
    if st or not np.array_equal(Cs[:, :N], Ctight):
        fails.append("ld_padding values")
    if not np.all(Cs[:, N:] == 777.0):
        fails.append("ld_padding C pad written")
    return fails


def run_op(call_op, ta, tb, A, B, C0, alpha, beta, lda=None, ldb=None):
    """Call the op entry point on op(A) = A (M x K), op(B) = B (K x N) given in
    logical form; A is stored transposed when ta (K x M), B when tb (N x K)."""
    M, K = A.shape
    N = B.shape[1]
    As = np.ascontiguousarray(A.T if ta else A, dtype=F32)
    Bs = np.ascontiguousarray(B.T if tb else B, dtype=F32)
    C = (np.ascontiguousarray(C0, dtype=F32).copy() if C0 is not None
         else np.full((M, N), np.nan, dtype=F32))
    st = call_op(int(ta), int(tb), M, N, K, alpha, As.reshape(-1), lda or max(As.shape[1], 1),
                 Bs.reshape(-1), ldb or max(Bs.shape[1], 1), beta, C.reshape(-1), max(N, 1))
    return st, C


def pin_transposed(call_op, rng, dims=range(1, 4), square_only=False) -> list[str]:
    fails = []
    combos = ((0, 0), (1, 0), (0, 1), (1, 1))
    shapes = ([(n, n, n) for n in range(2, 5)] if square_only else
              [(M, N, K) for M in dims for N in dims for K in dims])
    for (M, N, K) in shapes:
        A = rng.uniform(-2, 2, (M, K)).astype(F32)
        B = rng.uniform(-2, 2, (K, N)).astype(F32)
        C0 = rng.uniform(-2, 2, (M, N)).astype(F32)
        alpha, beta = float(F32(rng.uniform(-3, 3))), float(F32(rng.uniform(-3, 3)))
        for ta, tb in combos:
            st, C = run_op(call_op, ta, tb, A, B, C0, alpha, beta)
            if st != 0:
                fails.append(f"transposed status {st} at {(ta, tb, M, N, K)}")
                continue
            for i in range(M):
                for j in range(N):
                    ex, mag = exact_cell(A, B, C0, i, j, alpha, beta)
                    if not within_fp64_rounding(float(C[i, j]), ex, mag, K):
                        fails.append(f"transposed {(ta, tb)} {(M, N, K)} cell {(i, j)}")
                        break
    if square_only:
        return fails
    # permutation stored transposed: op(B) = P, C = A[:, perm]
    M, K = 5, 9
    perm = rng.permutation(K)
    P = np.zeros((K, K), F32)
    P[perm, np.arange(K)] = 1.0
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    for ta in (0, 1):
        st, C = run_op(call_op, ta, 1, A, P, None, 1.0, 0.0)
        if st or not np.array_equal(C, A[:, perm]):
            fails.append(f"transposed permutation ta={ta}")
    # NaN padding of transposed storage never leaks
    M, N, K = 6, 7, 5
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    _, Cref = run_op(call_op, 0, 0, A, B, None, 1.0, 0.0)
    As = np.full((K, M + 3), np.nan, F32); As[:, :M] = A.T
    Bs = np.full((N, K + 2), np.nan, F32); Bs[:, :K] = B.T
    C = np.full((M, N), np.nan, F32)
    st = call_op(1, 1, M, N, K, 1.0, As.reshape(-1), M + 3, Bs.reshape(-1), K + 2, 0.0,
                 C.reshape(-1), N)
    if st or not np.array_equal(C, Cref):
        fails.append("transposed ld padding")
    # leading dimensions are checked against the stored shapes
    buf = np.zeros(64, F32)
    if call_op(1, 0, 4, 3, 2, 1.0, buf, 3, buf, 3, 0.0, buf, 3) != -8:      # lda < M
        fails.append("transposed lda check")
    if call_op(0, 1, 4, 3, 5, 1.0, buf, 5, buf, 4, 0.0, buf, 3) != -10:     # ldb < K
        fails.append("transposed ldb check")
    if call_op(2, 0, 1, 1, 1, 1.0, buf, 1, buf, 1, 0.0, buf, 1) != -1:
        fails.append("trans flag check")
    return fails


def all_pins(call, seed=1234, square_only=False, call_op=None, call_epi=None,
             call_batched=None, call_mixed=None) -> list[str]:
    """Every pin; square_only restricts brute force to M = N = K (used for
    broken copies whose indexing is only memory-safe on square shapes).
    call_op, call_epi, call_batched, when given, are the entry points with
    transposed operands, with bias and activation, and strided-batched."""
    rng = np.random.default_rng(seed)
    fails = []
    if square_only:
        fails = _square_brute(call, rng)
        if call_op is not None:
            fails += pin_transposed(call_op, rng, square_only=True)
        return fails
    fails += pin_brute_force(call, rng)
    fails += pin_closed_forms(call, rng)
    fails += pin_alpha_beta(call, rng)
    fails += pin_ld_padding(call, rng)
    if call_op is not None:
        fails += pin_transposed(call_op, rng)
    if call_epi is not None:
        fails += pin_epilogue(call_epi, rng)
    if call_batched is not None:
        fails += pin_batched(call_batched, rng)
    if call_mixed is not None:
        fails += pin_mixed(call_mixed, rng)
    return fails


def _square_brute(call, rng) -> list[str]:
    fails = []
    for n in range(2, 6):
        A = rng.uniform(-2, 2, (n, n)).astype(F32)
        B = rng.uniform(-2, 2, (n, n)).astype(F32)
        st, C = run(call, A, B, None, 1.0, 0.0)
        for i in range(n):
            for j in range(n):
                ex, mag = exact_cell(A, B, None, i, j, 1.0, 0.0)
                if st or not within_fp64_rounding(float(C[i, j]), ex, mag, n):
                    fails.append(f"square brute {n} {(i, j)}")
    return fails


# ------------------------------------------------------------- epilogue --
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3, 4


def act_exact(act: int, x: Fraction) -> float:
    """The activation of an exact rational, at 40 digits, rounded to fp32."""
    if act == ACT_NONE:
        return rn32(x)
    if act == ACT_RELU:
        return rn32(max(x, Fraction(0)))
    with mpmath.workdps(40):
        v = mpmath.mpf(x.numerator) / x.denominator
        if act == ACT_SILU:
            y = v / (1 + mpmath.exp(-v))
        elif act == ACT_GELU_ERF:
            y = v * mpmath.ncdf(v)
        elif act == ACT_GELU_TANH:
            u = mpmath.sqrt(2 / mpmath.pi) * (v + mpmath.mpf("0.044715") * v ** 3)
            # 1 + tanh(u) loses about 2|u| / ln 10 digits to cancellation for
            # u < 0: evaluate the printed form with that many digits more
            with mpmath.workdps(40 + int(2 * abs(u) / mpmath.log(10)) + 10):
                v = mpmath.mpf(x.numerator) / x.denominator
                u = mpmath.sqrt(2 / mpmath.pi) * (v + mpmath.mpf("0.044715") * v ** 3)
                y = v / 2 * (1 + mpmath.tanh(u))
        else:
            raise ValueError(act)
        m, e = mpmath.frexp(y)
        return rn32(Fraction(int(mpmath.nint(m * 2 ** 80))) * Fraction(2) ** (int(e) - 80))


def ulp32(x: float) -> float:
    x = abs(np.float32(x))
    return float(np.nextafter(x, F32(np.inf)) - x)


def run_epi(call_epi, ta, tb, A, B, C0, alpha, beta, bias, act):
    """The epilogue entry point on logical A (M x K), B (K x N); bias is passed
    inside a longer buffer (so that a reading past N stays in memory)."""
    M, K = A.shape
    N = B.shape[1]
    As = np.ascontiguousarray(A.T if ta else A, dtype=F32)
    Bs = np.ascontiguousarray(B.T if tb else B, dtype=F32)
    C = (np.ascontiguousarray(C0, dtype=F32).copy() if C0 is not None
         else np.full((M, N), np.nan, dtype=F32))
    buf = None
    if bias is not None:
        buf = np.concatenate([bias.astype(F32), np.full(M + 8, 1000.0, F32)])
    st = call_epi(int(ta), int(tb), M, N, K, alpha, As.reshape(-1), max(As.shape[1], 1),
                  Bs.reshape(-1), max(Bs.shape[1], 1), beta, C.reshape(-1), max(N, 1), buf, act)
    return st, C


def pin_epilogue(call_epi, rng, dims=range(1, 4)) -> list[str]:
    fails = []
    for M in dims:
        for N in dims:
            for K in dims:
                A = rng.uniform(-2, 2, (M, K)).astype(F32)
                B = rng.uniform(-2, 2, (K, N)).astype(F32)
                C0 = rng.uniform(-2, 2, (M, N)).astype(F32)
                bias = rng.uniform(-2, 2, N).astype(F32)
                alpha, beta = float(F32(rng.uniform(-3, 3))), float(F32(rng.uniform(-3, 3)))
                ta, tb = int(rng.integers(2)), int(rng.integers(2))
                for act in range(5):
                    for bz in (bias, None):
                        st, C = run_epi(call_epi, ta, tb, A, B, C0, alpha, beta, bz, act)
                        if st != 0:
                            fails.append(f"epilogue status {st} at {(M, N, K, act)}")
                            continue
                        bad = False
                        for i in range(M):
                            for j in range(N):
                                x, _ = exact_cell(A, B, C0, i, j, alpha, beta)
                                if bz is not None:
                                    x += Fraction(float(bz[j]))
                                ref = act_exact(act, x)
                                if abs(float(C[i, j]) - ref) > ulp32(ref) or \
                                        (ref == 0.0) != (float(C[i, j]) == 0.0):
                                    fails.append(f"epilogue act={act} bias={bz is not None} "
                                                 f"{(M, N, K)} cell {(i, j)}: {C[i, j]!r} vs "
                                                 f"{ref!r}")
                                    bad = True
                                    break
                            if bad:
                                break
    # integers: ReLU and bias are exact, bias goes along columns
    M, N, K = 5, 7, 6
    A = rng.integers(-4, 5, (M, K)).astype(F32)
    B = rng.integers(-4, 5, (K, N)).astype(F32)
    C0 = rng.integers(-4, 5, (M, N)).astype(F32)
    bias = rng.integers(-20, 21, N).astype(F32)
    exact = (A.astype(np.int64) @ B.astype(np.int64)) * 2 - C0.astype(np.int64) + \
        bias.astype(np.int64)[None, :]
    st, C = run_epi(call_epi, 0, 0, A, B, C0, 2.0, -1.0, bias, ACT_RELU)
    if st or not np.array_equal(C, np.maximum(exact, 0).astype(F32)):
        fails.append("epilogue integer relu+bias")
    st, C = run_epi(call_epi, 1, 1, A, B, C0, 2.0, -1.0, bias, ACT_NONE)
    if st or not np.array_equal(C, exact.astype(F32)):
        fails.append("epilogue integer bias (transposed storage)")
    # alpha == 0: act(beta * C + bias) without reading A or B
    An = np.full((M, K), np.nan, F32)
    st, C = run_epi(call_epi, 0, 0, An, B, C0, 0.0, 0.5, bias, ACT_RELU)
    if st or not np.array_equal(C, np.maximum(0.5 * C0 + bias[None, :], 0).astype(F32)):
        fails.append("epilogue alpha0")
    st, C = run_epi(call_epi, 0, 0, A, B, None, 0.0, 0.0, bias, ACT_NONE)
    if st or not np.array_equal(C, np.broadcast_to(bias, (M, N))):
        fails.append("epilogue alpha0 beta0")
    # beta == 0 never reads C (NaN-filled C)
    st, C = run_epi(call_epi, 0, 0, A, B, None, 1.0, 0.0, bias, ACT_SILU)
    if st or not np.all(np.isfinite(C)):
        fails.append("epilogue beta0 read C")
    # act codes
    if run_epi(call_epi, 0, 0, A, B, C0, 1.0, 0.0, bias, 5)[0] != -15 or \
            run_epi(call_epi, 0, 0, A, B, C0, 1.0, 0.0, bias, -1)[0] != -15:
        fails.append("epilogue act code check")
    return fails


# -------------------------------------------------------------- batched --
def pin_batched(call_batched, rng) -> list[str]:
    """call_batched(ta, tb, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C,
    ldc, sc, batch) on flat buffers."""
    fails = []
    for trial in range(12):
        M, N, K = (int(v) for v in rng.integers(1, 4, 3))
        batch = int(rng.integers(1, 4))
        ta, tb = int(rng.integers(2)), int(rng.integers(2))
        share_a, share_b = trial % 4 == 1, trial % 4 == 2
        As = [rng.uniform(-2, 2, (M, K)).astype(F32) for _ in range(batch)]
        Bs = [rng.uniform(-2, 2, (K, N)).astype(F32) for _ in range(batch)]
        if share_a:
            As = [As[0]] * batch
        if share_b:
            Bs = [Bs[0]] * batch
        C0 = [rng.uniform(-2, 2, (M, N)).astype(F32) for _ in range(batch)]
        alpha, beta = float(F32(rng.uniform(-3, 3))), float(F32(rng.uniform(-3, 3)))

        def pack(mats, trans, pad_rows, pad_gap, share):
            # stored matrices with padded rows, gap floats between batch entries
            st = [np.ascontiguousarray(m.T if trans else m) for m in mats]
            r, c = st[0].shape
            ld = c + pad_rows
            stride = 0 if share else r * ld + pad_gap
            buf = np.full(max(stride * (len(st) - 1), 0) + r * ld + 1, np.nan, F32)
            for b, m in enumerate(st[:1] if share else st):
                for i in range(r):
                    buf[b * stride + i * ld: b * stride + i * ld + c] = m[i]
            return buf, max(ld, 1), stride

        a, lda, sa = pack(As, ta, int(rng.integers(0, 3)), int(rng.integers(0, 4)), share_a)
        b, ldb, sb = pack(Bs, tb, int(rng.integers(0, 3)), int(rng.integers(0, 4)), share_b)
        ldc = N + int(rng.integers(0, 3))
        sc = M * ldc + int(rng.integers(0, 4))
        c = np.full(sc * batch + 4, 777.0, F32)
        for bi in range(batch):
            for i in range(M):
                c[bi * sc + i * ldc: bi * sc + i * ldc + N] = C0[bi][i]
        st = call_batched(ta, tb, M, N, K, alpha, a, lda, sa, b, ldb, sb, beta, c, ldc, sc, batch)
        if st != 0:
            fails.append(f"batched status {st}")
            continue
        bad = False
        for bi in range(batch):
            for i in range(M):
                row = c[bi * sc + i * ldc: bi * sc + i * ldc + ldc]
                if np.any(row[N:] != 777.0):
                    fails.append("batched C padding written")
                    bad = True
                for j in range(N):
                    ex, mag = exact_cell(As[bi], Bs[bi], C0[bi], i, j, alpha, beta)
                    if not within_fp64_rounding(float(row[j]), ex, mag, K):
                        fails.append(f"batched {(ta, tb, M, N, K)} batch {bi} cell {(i, j)}")
                        bad = True
                        break
                if bad:
                    break
            if bad:
                break
        if not bad and np.any(c[sc * batch:] != 777.0):
            fails.append("batched wrote past the last C")
    # batch = 0 touches nothing; argument checks (1-based positions)
    buf = np.full(64, 5.0, F32)
    if call_batched(0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, 4, 0.0, buf, 2, 4, 0) != 0 or \
            np.any(buf != 5.0):
        fails.append("batched batch 0")
    checks = (((0, 0, 2, 2, 2, 1.0, buf, 2, -1, buf, 2, 4, 0.0, buf, 2, 4, 2), -9),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, -4, 0.0, buf, 2, 4, 2), -12),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, 4, 0.0, buf, 2, 3, 2), -16),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, 4, 0.0, buf, 2, 4, -1), -17),
              ((0, 0, 2, 2, 2, 1.0, buf, 1, 4, buf, 2, 4, 0.0, buf, 2, 4, 2), -8),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 1, 4, 0.0, buf, 2, 4, 2), -11),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, 4, 0.0, buf, 1, 4, 2), -15),
              ((0, 0, 2, 2, 2, 1.0, buf, 2, 4, buf, 2, 4, 0.0, None, 2, 4, 2), -14))
    for args, code in checks:
        if call_batched(*args) != code:
            fails.append(f"batched check {code}")
    return fails


# ---------------------------------------------------------- 16-bit inputs --
BF16, F16 = 1, 2

# bit patterns with the values their formats define (closed forms)
DECODE_CASES = {
    BF16: [(0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7), (0x0001, 2.0 ** -133),
           (0x0080, 2.0 ** -126), (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0x0000, 0.0),
           (0x8000, -0.0), (0x7F80, np.inf), (0xFF80, -np.inf), (0x7FC0, np.nan),
           (0x4049, 3.140625)],
    F16: [(0x3C00, 1.0), (0xC000, -2.0), (0x3C01, 1.0 + 2.0 ** -10), (0x0001, 2.0 ** -24),
          (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14), (0x7BFF, 65504.0), (0x0000, 0.0),
          (0x8000, -0.0), (0x7C00, np.inf), (0xFC00, -np.inf), (0x7E00, np.nan),
          (0x4248, 3.140625)],
}


def decode_ref(dtype, bits: np.ndarray) -> np.ndarray:
    """Test-side decoding: numpy's binary16 for F16; for BF16 the binary32
    whose high half the pattern is."""
    with np.errstate(invalid="ignore"):
        if dtype == F16:
            return bits.astype(np.uint16).view(np.float16).astype(np.float64)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_mixed(call_mixed, rng) -> list[str]:
    """call_mixed(dtype, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    on flat buffers (A, B uint16 bit patterns, C float32)."""
    fails = []
    for dtype in (BF16, F16):
        # decoding: every listed pattern times 1.0 (K = 1) gives its value
        pats = np.array([b for b, _ in DECODE_CASES[dtype]], np.uint16)
        vals = np.array([v for _, v in DECODE_CASES[dtype]], np.float64)
        one = np.array([DECODE_CASES[dtype][0][0]], np.uint16)
        C = np.full(len(pats), 7.0, np.float32)
        st = call_mixed(dtype, 0, 0, len(pats), 1, 1, 1.0, pats, 1, one, 1, 0.0, C, 1)
        # (a lone -0 product sums to +0 from the zero accumulator: compare values)
        ok = st == 0 and np.array_equal(np.isnan(C), np.isnan(vals)) and \
            np.all((C == vals) | np.isnan(vals))
        if not ok:
            fails.append(f"mixed decode dtype {dtype}")
        # every finite pattern through the same route, against the test-side decode
        allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        ref = decode_ref(dtype, allp)
        fin = np.isfinite(ref) & (np.abs(ref) < 3e38)
        allp = allp[fin]
        C = np.empty(len(allp), np.float32)
        st = call_mixed(dtype, 0, 0, len(allp), 1, 1, 1.0, allp, 1, one, 1, 0.0, C, 1)
        if st or not np.array_equal(C.astype(np.float64), ref[fin]):
            fails.append(f"mixed decode all patterns dtype {dtype}")
        # exact rational brute force over small shapes and every transposition
        for trial in range(24):
            M, N, K = (int(v) for v in rng.integers(1, 4, 3))
            ta, tb = int(rng.integers(2)), int(rng.integers(2))
            # finite values of moderate size: random sign, exponent, fraction
            def draw(shape):
                x = rng.uniform(-4, 4, shape)
                if dtype == F16:
                    return x.astype(np.float16).view(np.uint16)
                return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            Ab, Bb = draw((M, K)), draw((K, N))
            Av, Bv = decode_ref(dtype, Ab), decode_ref(dtype, Bb)
            C0 = rng.uniform(-2, 2, (M, N)).astype(F32)
            alpha, beta = float(F32(rng.uniform(-3, 3))), float(F32(rng.uniform(-3, 3)))
            As = np.ascontiguousarray(Ab.T if ta else Ab)
            Bs = np.ascontiguousarray(Bb.T if tb else Bb)
            C = C0.copy()
            st = call_mixed(dtype, ta, tb, M, N, K, alpha, As.reshape(-1), As.shape[1],
                            Bs.reshape(-1), Bs.shape[1], beta, C.reshape(-1), N)
            if st:
                fails.append(f"mixed status {st}")
                continue
            for i in range(M):
                for j in range(N):
                    ex, mag = exact_cell(Av.astype(F32), Bv.astype(F32), C0, i, j, alpha, beta)
                    if not within_fp64_rounding(float(C[i, j]), ex, mag, K):
                        fails.append(f"mixed dtype {dtype} {(ta, tb, M, N, K)} cell {(i, j)}")
                        break
    buf = np.zeros(16, np.uint16)
    cb = np.zeros(16, np.float32)
    if call_mixed(3, 0, 0, 2, 2, 2, 1.0, buf, 2, buf, 2, 0.0, cb, 2) != -1:
        fails.append("mixed dtype check")
    if call_mixed(BF16, 0, 0, 2, 2, 4, 1.0, buf, 2, buf, 2, 0.0, cb, 2) != -9:   # lda < K
        fails.append("mixed lda check")
    return fails
