"""fp32_sgemm_02_amd -- single-precision GEMM for AMD Instinct MI355X (gfx950).

C = alpha * (A * B) + beta * C on row-major fp32 matrices, computed by the
hand-written HIP kernels of ``libfp32sgemm.so`` (C ABI: include/fp32_sgemm.h).
This module only marshals arguments: every step of the product runs in the
library's GPU kernels.  PyTorch supplies device memory and streams.

The operation is the SGEMM of "a CUDA matmul" (plasmient.com labs) section 00
and "The GEMM Scrapbook" introduction: A is M x K, B is K x N, C is M x N, and
every cell of C is the dot product of a row of A and a column of B.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "sgemm", "sgemm_ex", "sgemm_op", "sgemm_op_noalloc", "sgemm_cblas", "sgemm_epilogue", "sgemm_strided_batched",
    "sgemm_mixed", "gemm", "gemm_batched", "gemm_mixed", "select", "tile_count", "tile_info", "status_string",
    "version", "workspace_release", "plan", "SgemmConfig", "TileDesc", "SgemmError", "LIB_PATH",
    "VARIANT_AUTO", "VARIANT_MFMA", "VARIANT_VALU", "VARIANT_SKINNY", "VARIANT_MFMA16",
    "VARIANT_GENERIC16", "VARIANT_SMALL", "DTYPE_BF16", "DTYPE_F16", "FLAG_SCALAR_IO", "FLAG_UNTUNED", "FLAG_STREAMK",
    "TILE_WHOLE", "TILE_DIRECT", "TILE_TRANS_B", "TILE_TRANS_A", "TILE_STREAMK",
    "ACT_NONE", "ACT_RELU", "ACT_SILU", "ACT_GELU_ERF", "ACT_GELU_TANH",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp32sgemm.so")

VARIANT_AUTO, VARIANT_MFMA, VARIANT_VALU, VARIANT_SKINNY = 0, 1, 2, 3
VARIANT_MFMA16, VARIANT_GENERIC16, VARIANT_SMALL = 4, 5, 6
DTYPE_BF16, DTYPE_F16 = 1, 2
FLAG_SCALAR_IO = 0x1
FLAG_UNTUNED = 0x2
FLAG_STREAMK = 0x4
TILE_WHOLE = 0x1
TILE_DIRECT = 0x2
TILE_TRANS_B = 0x4
TILE_TRANS_A = 0x8
TILE_STREAMK = 0x10
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3, 4


class SgemmConfig(ctypes.Structure):
    """Mirror of ``sgemm_config``."""
    _fields_ = [("variant", ctypes.c_int), ("tile", ctypes.c_int),
                ("flags", ctypes.c_int), ("group_m", ctypes.c_int)]


class TileDesc(ctypes.Structure):
    """Mirror of ``sgemm_tile_desc``."""
    _fields_ = [(n, ctypes.c_int) for n in
                ("bm", "bn", "bk", "wm", "wn", "tm", "tn", "threads", "lds_bytes", "stages", "flags")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class SgemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"sgemm status {status}: {status_string(status)}")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m fp32_sgemm_02_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.sgemm.restype = i
    lib.sgemm.argtypes = [i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_ex.restype = i
    lib.sgemm_ex.argtypes = [i, i, i, f, p, i, p, i, f, p, i, p, ctypes.POINTER(SgemmConfig)]
    lib.sgemm_op.restype = i
    lib.sgemm_op.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_op_ex.restype = i
    lib.sgemm_op_ex.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p,
                                ctypes.POINTER(SgemmConfig)]
    lib.sgemm_op_ex_noalloc.restype = i
    lib.sgemm_op_ex_noalloc.argtypes = lib.sgemm_op_ex.argtypes
    lib.sgemm_select.restype = i
    lib.sgemm_select.argtypes = [i, i, i, p, i, p, i, p, i, ctypes.POINTER(SgemmConfig)]
    ll = ctypes.c_longlong
    lib.sgemm_epilogue.restype = i
    lib.sgemm_epilogue.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p, i, p]
    lib.sgemm_epilogue_ex.restype = i
    lib.sgemm_epilogue_ex.argtypes = lib.sgemm_epilogue.argtypes + [ctypes.POINTER(SgemmConfig)]
    lib.sgemm_strided_batched.restype = i
    lib.sgemm_strided_batched.argtypes = [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p, i, ll, i, p]
    lib.sgemm_strided_batched_ex.restype = i
    lib.sgemm_strided_batched_ex.argtypes = (lib.sgemm_strided_batched.argtypes +
                                             [ctypes.POINTER(SgemmConfig)])
    lib.sgemm_mixed.restype = i
    lib.sgemm_mixed.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_mixed_ex.restype = i
    lib.sgemm_mixed_ex.argtypes = lib.sgemm_mixed.argtypes + [ctypes.POINTER(SgemmConfig)]
    lib.sgemm_cblas.restype = i
    lib.sgemm_cblas.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_op_plan.restype = i
    lib.sgemm_op_plan.argtypes = [i, i, i, i, i, p, i, p, i, p, i, ctypes.POINTER(SgemmConfig),
                                  ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.sgemm_plan.restype = i
    lib.sgemm_plan.argtypes = [i, i, i, p, i, p, i, p, i, ctypes.POINTER(SgemmConfig),
                               ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.sgemm_tile_count.restype = i
    lib.sgemm_tile_count.argtypes = [i]
    lib.sgemm_tile_info.restype = i
    lib.sgemm_tile_info.argtypes = [i, i, ctypes.POINTER(TileDesc)]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_status_string.argtypes = [i]
    lib.sgemm_version.restype = i
    lib.sgemm_version.argtypes = []
    lib.sgemm_workspace_release.restype = i
    lib.sgemm_workspace_release.argtypes = []
    _lib = lib
    return lib


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """Raw C-ABI call: A, B, C are device addresses (int) or None; returns the status."""
    return _load().sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None,
             cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call with an explicit configuration (None = automatic)."""
    return _load().sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                            ctypes.byref(cfg) if cfg is not None else None)


def sgemm_op(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None,
             cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call of sgemm_op (cfg given: sgemm_op_ex)."""
    if cfg is None:
        return _load().sgemm_op(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                stream)
    return _load().sgemm_op_ex(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               stream, ctypes.byref(cfg))


def sgemm_op_noalloc(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     stream=None, cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call of sgemm_op_ex_noalloc (partial sums in the library's
    static scratch array; no device allocation)."""
    return _load().sgemm_op_ex_noalloc(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                       ldc, stream,
                                       ctypes.byref(cfg) if cfg is not None else None)


def sgemm_epilogue(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                   stream=None, cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call of sgemm_epilogue (cfg given: sgemm_epilogue_ex)."""
    args = (trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, stream)
    if cfg is None:
        return _load().sgemm_epilogue(*args)
    return _load().sgemm_epilogue_ex(*args, ctypes.byref(cfg))


def sgemm_strided_batched(trans_a, trans_b, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b,
                          beta, C, ldc, stride_c, batch, stream=None,
                          cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call of sgemm_strided_batched (cfg given: the _ex form)."""
    args = (trans_a, trans_b, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta, C, ldc,
            stride_c, batch, stream)
    if cfg is None:
        return _load().sgemm_strided_batched(*args)
    return _load().sgemm_strided_batched_ex(*args, ctypes.byref(cfg))


def sgemm_mixed(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                stream=None, cfg: SgemmConfig | None = None) -> int:
    """Raw C-ABI call of sgemm_mixed (cfg given: sgemm_mixed_ex)."""
    args = (dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    if cfg is None:
        return _load().sgemm_mixed(*args)
    return _load().sgemm_mixed_ex(*args, ctypes.byref(cfg))


def sgemm_cblas(order, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                stream=None) -> int:
    """Raw C-ABI call with cblas_sgemm's conventions (order 101 row-major /
    102 column-major; trans 111 / 112 / 113)."""
    return _load().sgemm_cblas(order, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                               ldc, stream)


def select(M, N, K, A=None, lda=None, B=None, ldb=None, C=None, ldc=None, *,
           trans_a=False, trans_b=False) -> SgemmConfig:
    """The configuration sgemm() (sgemm_op() with transposition flags) picks
    for this shape (and these addresses); with edge strips, the main part's."""
    return plan(M, N, K, A, lda, B, ldb, C, ldc, trans_a=trans_a, trans_b=trans_b)[0]


def plan(M, N, K, A=None, lda=None, B=None, ldb=None, C=None, ldc=None, *,
         trans_a=False, trans_b=False):
    """(main-part configuration, edge rows, edge columns) of the automatic
    plan for this shape (and these addresses).  Leading dimensions default to
    the tight ones of the stored operands."""
    out = SgemmConfig()
    rows, cols = ctypes.c_int(0), ctypes.c_int(0)
    lda = lda or max(M if trans_a else K, 1)
    ldb = ldb or max(K if trans_b else N, 1)
    st = _load().sgemm_op_plan(int(trans_a), int(trans_b), M, N, K, A, lda, B, ldb, C,
                               ldc or max(N, 1), ctypes.byref(out), ctypes.byref(rows),
                               ctypes.byref(cols))
    if st != 0:
        raise SgemmError(st)
    return out, rows.value, cols.value


def tile_count(variant: int) -> int:
    return _load().sgemm_tile_count(variant)


def tile_info(variant: int, tile: int) -> dict:
    d = TileDesc()
    st = _load().sgemm_tile_info(variant, tile, ctypes.byref(d))
    if st != 0:
        raise SgemmError(st)
    return d.as_dict()


def status_string(status: int) -> str:
    return _load().sgemm_status_string(status).decode()


def version() -> int:
    return _load().sgemm_version()


def workspace_release() -> None:
    """Synchronise the current device and free the workspaces the library
    keeps for it (stream-K and split-K partial sums, one per stream)."""
    st = _load().sgemm_workspace_release()
    if st != 0:
        raise SgemmError(st)


def _ld(t) -> int:
    """Leading dimension of a 2-D row-major tensor view, in elements."""
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    ld = t.stride(0)
    if rows <= 1 or cols == 0:
        ld = max(ld, cols, 1)
    return ld


def _check_tensor(name, t, torch, device=None):
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _on_device(device, torch):
    """A context that makes `device` current: a no-op when it already is
    (the common case, and the switch costs host time on every call)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _stream_handle(stream, device, torch):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, *, trans_a: bool = False,
         trans_b: bool = False, bias=None, act: int = ACT_NONE, variant: int = VARIANT_AUTO,
         tile: int = -1, flags: int = 0, group_m: int = 0, stream=None, noalloc: bool = False):
    """C = act(alpha * op(A) @ op(B) + beta * C + bias) for 2-D float32 CUDA
    tensors (row-major views with unit column stride; padded rows are used
    through their leading dimension).  op(X) is X, or X transposed when
    trans_x: A is then stored K x M and B N x K (e.g. a linear layer's weight,
    C = X W^T with B = W, trans_b=True).  bias (N floats, one per column) and
    act (ACT_*) are optional (sgemm_epilogue).  C is updated in place when
    given; otherwise a new tensor is returned (beta must then be 0).  Runs
    asynchronously on ``stream`` (default: the current stream of A's
    device).  noalloc: run through sgemm_op_ex_noalloc (no bias or act)."""
    import torch

    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    _check_tensor("A", A, torch)
    _check_tensor("B", B, torch, A.device)
    if bias is not None:
        _check_tensor("bias", bias, torch, A.device)
        if bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1):
            raise ValueError(f"bias must be a contiguous vector of {N} floats")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        if C.dtype != torch.float32 or C.device != A.device or tuple(C.shape) != (M, N):
            raise ValueError(f"C must be float32 ({M}, {N}) on {A.device}")
    with _on_device(A.device, torch):
        s = _stream_handle(stream, A.device, torch)
        ptr = lambda t: t.data_ptr() if t.numel() else None
        args = (M, N, K, float(alpha), ptr(A), _ld(A), ptr(B), _ld(B), float(beta), ptr(C),
                _ld(C))
        explicit = not (variant == VARIANT_AUTO and tile < 0 and flags == 0 and group_m == 0)
        cfg = SgemmConfig(variant, tile, flags, group_m) if explicit else None
        if noalloc:
            if bias is not None or act != ACT_NONE:
                raise ValueError("noalloc: no bias or activation")
            st = sgemm_op_noalloc(int(trans_a), int(trans_b), *args, s, cfg=cfg)
        elif bias is not None or act != ACT_NONE:
            st = sgemm_epilogue(int(trans_a), int(trans_b), *args,
                                None if bias is None else ptr(bias), int(act), s, cfg=cfg)
        elif trans_a or trans_b:
            st = sgemm_op(int(trans_a), int(trans_b), *args, s, cfg=cfg)
        elif explicit:
            st = sgemm_ex(*args, s, cfg=cfg)
        else:
            st = sgemm(*args, s)
    if st != 0:
        raise SgemmError(st)
    return C


def gemm_mixed(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, *, trans_a: bool = False,
               trans_b: bool = False, variant: int = VARIANT_AUTO, tile: int = -1, group_m: int = 0,
               stream=None):
    """C = alpha * op(A) @ op(B) + beta * C for 2-D bfloat16 or float16 CUDA
    tensors A and B (the same dtype) and a float32 C (sgemm_mixed: fp32
    accumulation).  Layout and stream handling as gemm()."""
    import torch

    codes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if A.dtype not in codes or B.dtype != A.dtype:
        raise ValueError("A and B must both be bfloat16 or both float16")
    if not A.is_cuda or B.device != A.device:
        raise ValueError("A and B must be GPU tensors on one device")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape[::-1] if trans_a else A.shape
    K2, N = B.shape[::-1] if trans_b else B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _check_tensor("C", C, torch, A.device)
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be ({M}, {N})")
    with _on_device(A.device, torch):
        s = _stream_handle(stream, A.device, torch)
        ptr = lambda t: t.data_ptr() if t.numel() else None
        explicit = not (variant == VARIANT_AUTO and tile < 0 and group_m == 0)
        cfg = SgemmConfig(variant, tile, 0, group_m) if explicit else None
        st = sgemm_mixed(codes[A.dtype], int(trans_a), int(trans_b), M, N, K, float(alpha),
                         ptr(A), _ld(A), ptr(B), _ld(B), float(beta), ptr(C), _ld(C), s, cfg=cfg)
    if st != 0:
        raise SgemmError(st)
    return C


def _batch_view(name, t, torch):
    """(batch, rows, cols, leading dimension, batch stride) of a 3-D stack of
    row-major matrices, or of a 2-D matrix shared by the batch (stride 0)."""
    if t.dim() == 2:
        rows, cols = t.shape
        return None, rows, cols, _ld(t), 0
    if t.dim() != 3:
        raise ValueError(f"{name} must be 2-D or 3-D")
    nb, rows, cols = t.shape
    if cols > 1 and t.stride(2) != 1:
        raise ValueError(f"{name}: rows must be contiguous (stride(2) == 1)")
    ld = t.stride(1) if rows > 1 else max(t.stride(1), cols, 1)
    return nb, rows, cols, max(ld, cols, 1), t.stride(0) if nb > 1 else 0


def gemm_batched(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, *, trans_a: bool = False,
                 trans_b: bool = False, variant: int = VARIANT_AUTO, tile: int = -1,
                 flags: int = 0, group_m: int = 0, stream=None):
    """C[b] = alpha * op(A[b]) @ op(B[b]) + beta * C[b] for every b
    (sgemm_strided_batched).  A and B are 3-D float32 CUDA tensors (batch,
    rows, cols) with unit column stride, or 2-D matrices shared by the whole
    batch (batch stride 0); C is a 3-D tensor (batch, M, N), updated in place
    when given (otherwise a new one; beta must then be 0)."""
    import torch

    _check_tensor("A", A, torch)
    _check_tensor("B", B, torch, A.device)
    na, ar, ac, lda, sa = _batch_view("A", A, torch)
    nb, br, bc, ldb, sb = _batch_view("B", B, torch)
    M, K = (ac, ar) if trans_a else (ar, ac)
    K2, N = (bc, br) if trans_b else (br, bc)
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    sizes = {n for n in (na, nb) if n is not None}
    if len(sizes) > 1:
        raise ValueError(f"batch sizes differ: {sorted(sizes)}")
    batch = sizes.pop() if sizes else (C.shape[0] if C is not None and C.dim() == 3 else 1)
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((batch, M, N), dtype=torch.float32, device=A.device)
    _check_tensor("C", C, torch, A.device)
    if C.dim() != 3 or tuple(C.shape) != (batch, M, N):
        raise ValueError(f"C must be ({batch}, {M}, {N})")
    _, _, _, ldc, sc = _batch_view("C", C, torch)
    with _on_device(A.device, torch):
        s = _stream_handle(stream, A.device, torch)
        ptr = lambda t: t.data_ptr() if t.numel() else None
        explicit = not (variant == VARIANT_AUTO and tile < 0 and flags == 0 and group_m == 0)
        cfg = SgemmConfig(variant, tile, flags, group_m) if explicit else None
        st = sgemm_strided_batched(int(trans_a), int(trans_b), M, N, K, float(alpha), ptr(A), lda,
                                   sa, ptr(B), ldb, sb, float(beta), ptr(C), ldc, sc, batch, s,
                                   cfg=cfg)
    if st != 0:
        raise SgemmError(st)
    return C
