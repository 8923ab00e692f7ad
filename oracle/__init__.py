"""CPU oracle for single-precision GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``sgemm_oracle.c`` (plain C, fp64 accumulation, one
rounding to float).  This module builds that file with gcc and marshals numpy
arrays into it.  The operation is C = alpha * (A * B) + beta * C on row-major
matrices, as defined in "a CUDA matmul" (plasmient.com labs) section 00 and
"The GEMM Scrapbook" introduction; see the C file's header for the readings
taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile sgemm_oracle.c into liboracle.so next to it (gcc, no GPU code).

    -ffp-contract=off keeps the epilogue as separate multiply and add; the
    k-loop products are exact in double, so contraction there would not change
    any result either.
    """
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_sgemm.restype = ctypes.c_int
        lib.oracle_sgemm.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.oracle_sgemm_op.restype = ctypes.c_int
        lib.oracle_sgemm_op.argtypes = [ctypes.c_int, ctypes.c_int] + lib.oracle_sgemm.argtypes
        i, f, p, ll = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_longlong
        lib.oracle_sgemm_epilogue.restype = i
        lib.oracle_sgemm_epilogue.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p, i, i]
        lib.oracle_gemm_mixed.restype = i
        lib.oracle_gemm_mixed.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i, i]
        lib.oracle_sgemm_strided_batched.restype = i
        lib.oracle_sgemm_strided_batched.argtypes = [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p,
                                                     i, ll, i, i]
        lib.oracle_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def sgemm_raw(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nthreads=None) -> int:
    """Direct call on flat float32 numpy buffers (C is updated in place)."""
    lib = _load()

    def ptr(x):
        if x is None:
            return None
        assert x.dtype == np.float32 and x.flags.c_contiguous
        return x.ctypes.data

    return lib.oracle_sgemm(int(M), int(N), int(K), float(alpha), ptr(A), int(lda),
                            ptr(B), int(ldb), float(beta), ptr(C), int(ldc),
                            int(nthreads or default_threads()))


def _ld(x: np.ndarray) -> int:
    """Leading dimension (in elements) of a row-major 2-D float32 view."""
    assert x.dtype == np.float32 and x.ndim == 2
    if x.size == 0:
        return max(x.shape[1], 1)
    assert x.shape[1] <= 1 or x.strides[1] == 4, "rows must be contiguous"
    ld = x.strides[0] // 4
    if x.shape[0] <= 1 or x.shape[1] == 0:
        ld = max(ld, x.shape[1], 1)
    return ld


def _base(x: np.ndarray):
    return x.ctypes.data if x.size else None


ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3, 4


def sgemm(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None,
          alpha: float = 1.0, beta: float = 0.0, nthreads: int | None = None,
          trans_a: bool = False, trans_b: bool = False, bias: np.ndarray | None = None,
          act: int = ACT_NONE) -> np.ndarray:
    """C = act(alpha * op(A) @ op(B) + beta * C + bias) on 2-D float32 arrays
    (row-major views with unit column stride; padded rows are allowed).  op(X)
    is X, or X transposed when trans_x (X is then stored transposed: A as
    K x M, B as N x K).  bias (N floats, one per column) and act (ACT_*) are
    optional.  C is updated in place when given; otherwise a new (M, N) array
    is returned (beta must then be 0)."""
    lib = _load()
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    assert K == K2, "inner dimensions differ"
    if C is None:
        assert beta == 0.0
        C = np.empty((M, N), dtype=np.float32)
    assert C.shape == (M, N)
    threads = int(nthreads or default_threads())
    if bias is None and act == ACT_NONE:
        st = lib.oracle_sgemm_op(int(trans_a), int(trans_b), M, N, K, float(alpha), _base(A),
                                 _ld(A), _base(B), _ld(B), float(beta), _base(C), _ld(C), threads)
    else:
        if bias is not None:
            assert bias.dtype == np.float32 and bias.shape == (N,) and bias.flags.c_contiguous
        st = lib.oracle_sgemm_epilogue(int(trans_a), int(trans_b), M, N, K, float(alpha),
                                       _base(A), _ld(A), _base(B), _ld(B), float(beta), _base(C),
                                       _ld(C), None if bias is None else _base(bias), int(act),
                                       threads)
    if st != 0:
        raise RuntimeError(f"oracle returned {st}")
    return C


BF16, F16 = 1, 2


def _ld16(x: np.ndarray) -> int:
    assert x.dtype == np.uint16 and x.ndim == 2
    if x.size == 0:
        return max(x.shape[1], 1)
    assert x.shape[1] <= 1 or x.strides[1] == 2, "rows must be contiguous"
    ld = x.strides[0] // 2
    if x.shape[0] <= 1:
        ld = max(ld, x.shape[1], 1)
    return ld


def gemm_mixed(dtype: int, A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None,
               alpha: float = 1.0, beta: float = 0.0, nthreads: int | None = None,
               trans_a: bool = False, trans_b: bool = False) -> np.ndarray:
    """C = alpha * op(A) @ op(B) + beta * C with A and B given as 16-bit float
    bit patterns (uint16 arrays; dtype BF16 or F16) and C float32, through
    oracle_gemm_mixed."""
    lib = _load()
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    assert K == K2, "inner dimensions differ"
    if C is None:
        assert beta == 0.0
        C = np.empty((M, N), dtype=np.float32)
    assert C.shape == (M, N)
    st = lib.oracle_gemm_mixed(int(dtype), int(trans_a), int(trans_b), M, N, K, float(alpha),
                               _base(A), _ld16(A), _base(B), _ld16(B), float(beta), _base(C),
                               _ld(C), int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError(f"oracle_gemm_mixed returned {st}")
    return C


def _batched_view(x: np.ndarray):
    """(base, leading dimension, batch stride in floats, rows, cols) of a 3-D
    float32 stack of row-major matrices, or of a 2-D matrix shared by every
    batch (stride 0)."""
    assert x.dtype == np.float32
    if x.ndim == 2:
        return _base(x), _ld(x), 0, x.shape[0], x.shape[1]
    assert x.ndim == 3 and x.strides[0] % 4 == 0 and x.strides[0] >= 0
    return _base(x), _ld(x[0]) if x.shape[0] else max(x.shape[2], 1), x.strides[0] // 4, \
        x.shape[1], x.shape[2]


def sgemm_batched(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None,
                  alpha: float = 1.0, beta: float = 0.0, nthreads: int | None = None,
                  trans_a: bool = False, trans_b: bool = False) -> np.ndarray:
    """C[b] = alpha * op(A[b]) @ op(B[b]) + beta * C[b] for every b, through
    oracle_sgemm_strided_batched.  A and B are 3-D stacks (batch, rows, cols)
    or 2-D matrices shared by the whole batch; C is a 3-D stack, updated in
    place when given (otherwise a new one, beta must then be 0)."""
    lib = _load()
    a, lda, sa, ar, ac = _batched_view(A)
    b, ldb, sb, br, bc = _batched_view(B)
    M, K = (ac, ar) if trans_a else (ar, ac)
    K2, N = (bc, br) if trans_b else (br, bc)
    assert K == K2, "inner dimensions differ"
    batch = max(A.shape[0] if A.ndim == 3 else 1, B.shape[0] if B.ndim == 3 else 1)
    if C is None:
        assert beta == 0.0
        C = np.empty((batch, M, N), dtype=np.float32)
    assert C.ndim == 3 and C.shape == (batch, M, N)
    c, ldc, sc, _, _ = _batched_view(C)
    st = lib.oracle_sgemm_strided_batched(int(trans_a), int(trans_b), M, N, K, float(alpha), a,
                                          lda, sa, b, ldb, sb, float(beta), c, ldc, sc, batch,
                                          int(nthreads or default_threads()))
    if st != 0:
        raise RuntimeError(f"oracle_sgemm_strided_batched returned {st}")
    return C


def version() -> int:
    return _load().oracle_version()
