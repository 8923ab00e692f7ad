"""The CPU oracle against what the mathematics fixes (runs without a GPU).

Beyond the pins in oracle_pins.py this file checks the oracle against test-only
library routines (numpy int64 and float64 matrix products), checks thread-count
invariance and argument validation, and compiles deliberately broken copies of
the oracle to show that each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

from oracle_pins import all_pins, run

F32 = np.float32
HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "sgemm_oracle.c")


def _caller(lib, nthreads=1):
    fn = lib.oracle_sgemm
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]

    def call(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
        p = lambda x: x.ctypes.data if (x is not None and x.size) else None
        return fn(M, N, K, alpha, p(A), lda, p(B), ldb, beta, p(C), ldc, nthreads)
    return call


def _op_caller(lib, nthreads=1):
    fn = lib.oracle_sgemm_op
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]

    def call_op(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
        p = lambda x: x.ctypes.data if (x is not None and x.size) else None
        return fn(ta, tb, M, N, K, alpha, p(A), lda, p(B), ldb, beta, p(C), ldc, nthreads)
    return call_op


def _epi_caller(lib, nthreads=1):
    fn = lib.oracle_sgemm_epilogue
    fn.restype = ctypes.c_int
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    fn.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p, i, i]

    def call_epi(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act):
        q = lambda x: x.ctypes.data if (x is not None and x.size) else None
        return fn(ta, tb, M, N, K, alpha, q(A), lda, q(B), ldb, beta, q(C), ldc, q(bias), act,
                  nthreads)
    return call_epi


def _batched_caller(lib, nthreads=1):
    fn = lib.oracle_sgemm_strided_batched
    fn.restype = ctypes.c_int
    i, f, p, ll = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_longlong
    fn.argtypes = [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p, i, ll, i, i]

    def call_batched(ta, tb, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta, C, ldc, sc, batch):
        q = lambda x: x.ctypes.data if (x is not None and x.size) else None
        return fn(ta, tb, M, N, K, alpha, q(A), lda, sa, q(B), ldb, sb, beta, q(C), ldc, sc,
                  batch, nthreads)
    return call_batched


def _mixed_caller(lib, nthreads=1):
    fn = lib.oracle_gemm_mixed
    fn.restype = ctypes.c_int
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    fn.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i, i]

    def call_mixed(dtype, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
        q = lambda x: x.ctypes.data if (x is not None and x.size) else None
        return fn(dtype, ta, tb, M, N, K, alpha, q(A), lda, q(B), ldb, beta, q(C), ldc, nthreads)
    return call_mixed


def _callers(lib, nthreads=1):
    return dict(call_op=_op_caller(lib, nthreads), call_epi=_epi_caller(lib, nthreads),
                call_batched=_batched_caller(lib, nthreads),
                call_mixed=_mixed_caller(lib, nthreads))


@pytest.fixture(scope="module")
def call(oracle_mod):
    return _caller(ctypes.CDLL(oracle_mod._LIB), nthreads=3)


@pytest.fixture(scope="module")
def call_op(oracle_mod):
    return _op_caller(ctypes.CDLL(oracle_mod._LIB), nthreads=2)


def test_all_pins_pass(call, oracle_mod):
    assert all_pins(call, **_callers(ctypes.CDLL(oracle_mod._LIB), nthreads=2)) == []


def test_transposed_storage_matches_explicit_transpose(oracle_mod):
    """op(A), op(B) read from transposed storage give the bits of the
    untransposed product of explicit transposes (same arithmetic order)."""
    rng = np.random.default_rng(12)
    M, N, K = 37, 29, 301
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    C0 = rng.uniform(-1, 1, (M, N)).astype(F32)
    ref = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    for ta, tb in ((1, 0), (0, 1), (1, 1)):
        got = oracle_mod.sgemm(At if ta else A, Bt if tb else B, C0.copy(), 0.5, -1.25,
                               trans_a=bool(ta), trans_b=bool(tb))
        assert np.array_equal(got, ref), (ta, tb)


def test_integer_exact_matches_int64_library(oracle_mod):
    rng = np.random.default_rng(7)
    M, N, K = 67, 45, 301
    A = rng.integers(-4, 5, (M, K))
    B = rng.integers(-4, 5, (K, N))
    C = oracle_mod.sgemm(A.astype(F32), B.astype(F32))
    assert np.array_equal(C, (A @ B).astype(F32))


def test_matches_float64_library_within_one_ulp(oracle_mod):
    rng = np.random.default_rng(8)
    n = 256
    A = rng.uniform(-1, 1, (n, n)).astype(F32)
    B = rng.uniform(-1, 1, (n, n)).astype(F32)
    C = oracle_mod.sgemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(F32))
    assert np.all(np.abs(C.astype(np.float64) - ref) <= ulp)


def test_large_k_sampled_rows_float64(oracle_mod):
    """Rows sampled from a 4096-deep product agree with the float64 library."""
    rng = np.random.default_rng(9)
    M, N, K = 8, 512, 4096
    A = rng.uniform(-1, 1, (M, K)).astype(F32)
    B = rng.uniform(-1, 1, (K, N)).astype(F32)
    C = oracle_mod.sgemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(C - ref) <= np.spacing(np.abs(ref).astype(F32)))


def test_thread_count_does_not_change_bits(oracle_mod):
    rng = np.random.default_rng(10)
    A = rng.uniform(-1, 1, (97, 130)).astype(F32)
    B = rng.uniform(-1, 1, (130, 61)).astype(F32)
    C1 = oracle_mod.sgemm(A, B, nthreads=1)
    C7 = oracle_mod.sgemm(A, B, nthreads=7)
    assert np.array_equal(C1, C7)


def test_scaling_by_two_is_exact(oracle_mod):
    rng = np.random.default_rng(11)
    A = rng.uniform(-1, 1, (40, 50)).astype(F32)
    B = rng.uniform(-1, 1, (50, 30)).astype(F32)
    assert np.array_equal(oracle_mod.sgemm(A * F32(2), B), oracle_mod.sgemm(A, B) * F32(2))


def test_fp32_probe_is_exact(oracle_mod):
    """17-significant-bit A times {-1,0,1} B over K=256: every partial sum is a
    multiple of 2^-16 below 2^8 in magnitude, hence exact in fp32 and fp64."""
    import workloads
    A, B, _ = workloads.inputs("probe256")
    C = oracle_mod.sgemm(A, B)
    exact = (np.rint(A.astype(np.float64) * 2 ** 16).astype(np.int64)
             @ B.astype(np.int64)).astype(np.float64) * 2.0 ** -16
    assert np.array_equal(C.astype(np.float64), exact)


def test_quick_returns(call):
    # M == 0 / N == 0 touch nothing, even with null pointers
    assert call(0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5) == 0
    assert call(5, 0, 5, 1.0, None, 5, None, 1, 0.0, None, 1) == 0
    # K == 0: C = beta * C
    C = np.arange(6, dtype=F32)
    assert call(2, 3, 0, 1.0, None, 1, None, 3, 2.0, C, 3) == 0
    assert np.array_equal(C, np.arange(6, dtype=F32) * 2)
    # alpha == 0, beta == 1: unchanged, NaN included
    C = np.array([1.0, np.nan, 3.0, 4.0], F32)
    A = np.full(4, np.nan, F32)
    assert call(2, 2, 2, 0.0, A, 2, A, 2, 1.0, C, 2) == 0
    assert np.isnan(C[1]) and C[0] == 1 and C[3] == 4


@pytest.mark.parametrize("args,code", [
    ((-1, 1, 1, 1, 1, 1), -1),
    ((1, -1, 1, 1, 1, 1), -2),
    ((1, 1, -1, 1, 1, 1), -3),
    ((2, 3, 4, 3, 3, 3), -6),   # lda < K
    ((2, 3, 4, 4, 2, 3), -8),   # ldb < N
    ((2, 3, 4, 4, 3, 2), -11),  # ldc < N
])
def test_argument_validation(call, args, code):
    M, N, K, lda, ldb, ldc = args
    buf = np.zeros(64, F32)
    assert call(M, N, K, 1.0, buf, lda, buf, ldb, 0.0, buf, ldc) == code


def test_null_operands_rejected(call):
    buf = np.zeros(16, F32)
    assert call(2, 2, 2, 1.0, None, 2, buf, 2, 0.0, buf, 2) == -5
    assert call(2, 2, 2, 1.0, buf, 2, None, 2, 0.0, buf, 2) == -7
    assert call(2, 2, 2, 1.0, buf, 2, buf, 2, 0.0, None, 2) == -10


# --- deliberately broken copies of the oracle must fail the pins -----------
MUTANTS = {
    # a dropped term: the first k is skipped
    "dropped_term": ("for (int k = 0; k < K; ++k)", "for (int k = 1; k < K; ++k)", False),
    # a wrong sign in the accumulation
    "wrong_sign": ("acc[j] += a * (double)brow[(long long)j * b->b_col];",
                   "acc[j] -= a * (double)brow[(long long)j * b->b_col];", False),
    # a wrong index: A walked backwards along k
    "wrong_index": ("const double a = (double)arow[(long long)k * b->a_col];",
                    "const double a = (double)arow[(long long)(K - 1 - k) * b->a_col];", False),
    # a transposed operand: A(k, i) instead of A(i, k) (memory-safe on squares)
    "transposed_a": ("const double a = (double)arow[(long long)k * b->a_col];",
                     "const double a = (double)b->A[(long long)k * b->a_row + "
                     "(long long)i * b->a_col];", True),
    # transposed storage of A ignored (memory-safe on squares)
    "trans_a_ignored": ("b->a_row = trans_a ? 1 : lda; b->a_col = trans_a ? lda : 1;",
                        "b->a_row = lda; b->a_col = 1;", True),
    # transposed storage of B ignored (memory-safe on squares)
    "trans_b_ignored": ("b->B = B; b->b_row = trans_b ? 1 : ldb; b->b_col = trans_b ? ldb : 1;",
                        "b->B = B; b->b_row = ldb; b->b_col = 1;", True),
    # alpha dropped
    "no_alpha": ("double out = b->alpha * acc[j];", "double out = acc[j];", False),
    # beta == 0 still reads C
    "beta0_reads_c": ("if (b->beta != 0.0)\n", "if (1)\n", False),
    # alpha == 0 path ignores beta
    "alpha0_ignores_beta": ("(b->beta == 0.0) ? 0.0 : b->beta * (double)crow[j]);",
                            "(b->beta == 0.0) ? 0.0 : (double)crow[j]);", False),
    # epilogue sign error on beta
    "beta_sign": ("out += b->beta * (double)crow[j];", "out -= b->beta * (double)crow[j];",
                  False),
    # bias dropped
    "bias_dropped": ("if (b->bias) out += (double)b->bias[j];", "if (0) out += 0.0;", False),
    # bias taken per row instead of per column (the pins pad the bias buffer)
    "bias_per_row": ("out += (double)b->bias[j];", "out += (double)b->bias[b->i0];", False),
    # the activation applied before the bias
    "act_before_bias": ("    if (b->bias) out += (double)b->bias[j];\n"
                        "    return (float)activate(b->act, out);",
                        "    out = activate(b->act, out);\n"
                        "    if (b->bias) out += (double)b->bias[j];\n    return (float)out;",
                        False),
    # alpha == 0 path skips bias and activation
    "alpha0_no_epilogue": ("crow[j] = finish(b, j, (b->beta == 0.0) ? 0.0 : "
                           "b->beta * (double)crow[j]);",
                           "crow[j] = (float)((b->beta == 0.0) ? 0.0 : "
                           "b->beta * (double)crow[j]);", False),
    # leaky instead of plain ReLU
    "relu_leaky": ("return x < 0.0 ? 0.0 : x;", "return x < 0.0 ? 0.01 * x : x;", False),
    # SiLU with the wrong sign in the exponent
    "silu_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));", False),
    # GELU without the 1/sqrt(2) scaling of the erf argument
    "gelu_no_sqrt2": ("erfc(-x / sqrt(2.0))", "erfc(-x)", False),
    # GELU tanh form with a perturbed cubic coefficient
    "gelu_tanh_coeff": ("(x + 0.044715 * x * x * x)", "(x + 0.0447 * x * x * x)", False),
    # GELU tanh form with the factor 2 of the exponent dropped
    "gelu_tanh_half": ("return x / (1.0 + exp(-2.0 * u));", "return x / (1.0 + exp(-u));",
                       False),
    # the batch stride of A ignored
    "batch_stride_a_ignored": ("A ? A + b * stride_a : A", "A", False),
    # the batch stride of C ignored
    "batch_stride_c_ignored": ("C + b * stride_c, ldc", "C, ldc", False),
    # bfloat16 decoded from the wrong bits
    "bf16_shift": ("const uint32_t bits = (uint32_t)h << 16;",
                   "const uint32_t bits = (uint32_t)h << 15;", False),
    # float16 exponent bias off by one
    "f16_bias": ("v = ldexp((double)(1024 + frac), e - 25);",
                 "v = ldexp((double)(1024 + frac), e - 24);", False),
    # float16 subnormals scaled wrongly
    "f16_subnormal": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -23);", False),
    # float16 sign dropped
    "f16_sign": ("return (float)(sign ? -v : v);", "return (float)v;", False),
    # the last matrix of the batch skipped
    "batch_last_skipped": ("for (int b = 0; b < batch; ++b)", "for (int b = 0; b + 1 < batch; ++b)",
                           False),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, square_only = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-pthread",
                    str(c), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    if square_only:
        fails = all_pins(_caller(lib), square_only=True, call_op=_op_caller(lib))
    else:
        fails = all_pins(_caller(lib), **_callers(lib))
    if square_only:
        # the square subset must catch it; the full suite is not memory-safe here
        assert fails, f"mutant {name} passed every square pin"
    else:
        assert fails, f"mutant {name} passed every pin"


def test_batched_wrapper_matches_float64_matmul(oracle_mod):
    """The batched entry point at a moderate size against numpy's float64
    batched matmul (a library routine): within one fp32 ulp per cell, with a
    stacked A and a B shared by the batch."""
    rng = np.random.default_rng(21)
    A = rng.uniform(-1, 1, (5, 33, 40)).astype(F32)
    B = rng.uniform(-1, 1, (40, 29)).astype(F32)
    C0 = rng.uniform(-1, 1, (5, 33, 29)).astype(F32)
    got = oracle_mod.sgemm_batched(A, B, C0.copy(), 0.75, -0.5)
    ref = 0.75 * np.matmul(A.astype(np.float64), B.astype(np.float64)) - 0.5 * C0
    ulp = np.spacing(np.abs(ref.astype(F32)))
    assert np.all(np.abs(got - ref) <= ulp)
    # transposed storage of both operands, per-batch B
    Bt = rng.uniform(-1, 1, (5, 29, 40)).astype(F32)
    At = np.ascontiguousarray(np.transpose(A, (0, 2, 1)))
    got = oracle_mod.sgemm_batched(At, Bt, trans_a=True, trans_b=True)
    ref = np.matmul(A.astype(np.float64), np.transpose(Bt, (0, 2, 1)).astype(np.float64))
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref.astype(F32))))


def test_epilogue_wrapper(oracle_mod):
    """bias broadcast along rows and the activation codes, through the numpy
    wrapper, against float64 numpy/scipy evaluations (within a few ulp)."""
    from scipy.special import expit, ndtr
    rng = np.random.default_rng(22)
    A = rng.uniform(-1, 1, (17, 50)).astype(F32)
    B = rng.uniform(-1, 1, (50, 23)).astype(F32)
    bias = rng.uniform(-1, 1, 23).astype(F32)
    x = A.astype(np.float64) @ B.astype(np.float64) + bias
    refs = {0: x, 1: np.maximum(x, 0), 2: x * expit(x), 3: x * ndtr(x)}
    for act, ref in refs.items():
        got = oracle_mod.sgemm(A, B, bias=bias, act=act)
        assert np.all(np.abs(got - ref) <= 2 * np.spacing(np.abs(ref.astype(F32))) + 1e-30), act
