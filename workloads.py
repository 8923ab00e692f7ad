"""Seeded synthetic workloads for the SGEMM path.

This module holds only the named problem shapes and the seeded input draws.
It performs none of the GEMM arithmetic, and both the CPU oracle's tests and
the GPU path's tests and benchmark take their inputs from here.

The pages measure one workload: square 4096 fp32 C = A * B ("The GEMM
Scrapbook", roofline paragraph and ladder table; "The 1% kernel", section 1)
and state no value distribution.  The shapes below extend that with BLAS-form,
ragged, sweep and transformer-MLP shapes; the value distributions are fixed
here so that every run draws the same matrices.

Recipe (one fresh generator per shape):
  rng = numpy.random.default_rng(seed)       # PCG64
  draw order: A (M x K), then B (K x N), then C (M x N, only when beta != 0)
  "uniform":   rng.uniform(-1, 1, shape) cast to float32
  "int4":      rng.integers(-4, 5, shape) cast to float32 (values -4..4)
  "mlp":       A = rng.standard_normal(dtype=float32);
               B = rng.standard_normal(dtype=float32) * float32(1/sqrt(K))
               (variance 1/K, so each cell of A*B has unit variance)
  "probe":     A = rng.integers(-2**16, 2**16 + 1) * 2**-16 (17 significant
               bits), B = rng.integers(-1, 2) (values -1, 0, 1)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = np.float32


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str          # "uniform" | "int4" | "mlp" | "probe"
    seed: int
    note: str = ""
    # scoring roofline: "mfma" (compute) or "hbm" (memory)
    bound: str = field(default="mfma")

    @property
    def flops(self) -> int:
        """2*M*N*K: one multiply and one add per (i, j, k) term; the epilogue is
        not counted (as in the pages' GFLOP/s figures)."""
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """Algorithmic bytes: A, B and the C write once, plus the C read when
        beta != 0."""
        c_traffic = 2 if self.beta != 0.0 else 1
        return 4 * (self.M * self.K + self.K * self.N + c_traffic * self.M * self.N)


def _ragged(name, M, N, K, note="", bound="mfma"):
    return Workload(name, M, N, K, 1.0, 1.0, "uniform", 3, note, bound)


WORKLOADS: dict[str, Workload] = {}


def _add(w: Workload):
    WORKLOADS[w.name] = w


_add(Workload("square256", 256, 256, 256, 1.0, 0.0, "uniform", 0,
              "small square; the oracle finishes in well under a second"))
_add(Workload("square4096", 4096, 4096, 4096, 1.0, 0.0, "uniform", 1,
              "the pages' headline shape: 137 GFLOP"))
_add(Workload("blas4096", 4096, 4096, 4096, 0.5, -1.25, "uniform", 2,
              "full BLAS form with alpha and beta"))
_add(Workload("int4096", 4096, 4096, 4096, 1.0, 0.0, "int4", 2,
              "integer-valued A, B in [-4, 4]: every partial sum is exact"))
_add(Workload("int4096_blas", 4096, 4096, 4096, 0.5, -1.25, "int4", 2,
              "integer-valued A, B, C: alpha*acc and beta*C exact multiples of 1/4"))
_add(_ragged("ragged_4097x1000x3001", 4097, 1000, 3001))
_add(_ragged("row_1x4096x4096", 1, 4096, 4096, "one row of C: streams B", "hbm"))
_add(_ragged("col_4096x1x4096", 4096, 1, 4096, "one column of C: streams A", "hbm"))
_add(_ragged("ragged_777x777x33", 777, 777, 33, "K tail and lda = 33", "hbm"))
for _n in (128, 256, 512, 1024, 2048, 4096, 8192):
    _add(_ragged(f"sweep{_n}", _n, _n, _n, "square sweep", "hbm" if _n <= 128 else "mfma"))
_add(Workload("mlp_up", 8192, 14336, 4096, 1.0, 0.0, "mlp", 4,
              "transformer MLP up-projection: (M,K,N) = (8192,4096,14336)"))
_add(Workload("mlp_down", 8192, 4096, 14336, 1.0, 0.0, "mlp", 4,
              "transformer MLP down-projection: (M,K,N) = (8192,14336,4096)"))
_add(Workload("mlp_decode16", 16, 14336, 4096, 1.0, 0.0, "mlp", 4,
              "decode-like skinny: 16 rows against the up-projection weight", "hbm"))
_add(Workload("probe256", 256, 256, 256, 1.0, 0.0, "probe", 5,
              "fp32-ness probe: exact in fp32, not in any 10- or 7-bit-mantissa format"))


def draw(M: int, N: int, K: int, dist: str, seed: int, with_c: bool):
    """(A, B, C or None) as C-contiguous float32 arrays, drawn in the order
    A, B, C from one fresh generator."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        A = rng.uniform(-1.0, 1.0, (M, K)).astype(F32)
        B = rng.uniform(-1.0, 1.0, (K, N)).astype(F32)
        C = rng.uniform(-1.0, 1.0, (M, N)).astype(F32) if with_c else None
    elif dist == "int4":
        A = rng.integers(-4, 5, (M, K)).astype(F32)
        B = rng.integers(-4, 5, (K, N)).astype(F32)
        C = rng.integers(-4, 5, (M, N)).astype(F32) if with_c else None
    elif dist == "mlp":
        A = rng.standard_normal((M, K), dtype=F32)
        B = rng.standard_normal((K, N), dtype=F32)
        B *= F32(1.0 / np.sqrt(K))
        C = rng.standard_normal((M, N), dtype=F32) if with_c else None
    elif dist == "probe":
        A = (rng.integers(-(1 << 16), (1 << 16) + 1, (M, K)).astype(np.float64)
             * 2.0 ** -16).astype(F32)
        B = rng.integers(-1, 2, (K, N)).astype(F32)
        C = rng.uniform(-1.0, 1.0, (M, N)).astype(F32) if with_c else None
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return A, B, C


def inputs(w: Workload | str):
    """Inputs of a named workload: (A, B, C0) with C0 None when beta == 0."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return draw(w.M, w.N, w.K, w.dist, w.seed, w.beta != 0.0)


def padded(x: np.ndarray, extra_cols: int, fill: float) -> np.ndarray:
    """A copy of x stored with `extra_cols` padding floats after every row
    (filled with `fill`); returns the (rows, cols) view into that storage."""
    rows, cols = x.shape
    store = np.full((rows, cols + extra_cols), fill, dtype=F32)
    store[:, :cols] = x
    return store[:, :cols]
