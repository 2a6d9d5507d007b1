"""MI355X (gfx950) software-pipelined fp16/bf16 GEMM.

Thin Python binding of the C ABI declared in ``include/bpt_gemm.h``: the
functions here only marshal torch tensors (device pointers, leading
dimensions, batch strides, the current HIP stream) into the library calls of
the same names.  Every step of the product runs in the HIP kernels of
``libbpt_gemm.so``; there is no fallback path -- if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "GemmError", "lib", "gemm_f16", "gemm_bf16", "gemm_batched_f16", "gemm_ex", "gemm_ex_bt", "gemm_ex_noalloc",
    "attention_fwd",
    "variants", "select_variant", "library", "LIB_PATH", "POISON_LIB_PATH",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbpt_gemm.so")
# the same library built with every LDS-DMA destination filled with NaN just
# before its copy (race detection; build.build_poison)
POISON_LIB_PATH = os.path.join(_PKG, "libbpt_gemm_poison.so")

BPT_OK, BPT_ERR_INVALID_ARG, BPT_ERR_UNSUPPORTED, BPT_ERR_HIP = 0, 1, 2, 3


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {0: "BPT_OK", 1: "BPT_ERR_INVALID_ARG", 2: "BPT_ERR_UNSUPPORTED", 3: "BPT_ERR_HIP"}
_lib = None


def lib() -> ctypes.CDLL:
    """Load libbpt_gemm.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route this module's calls through another build of the library at
    `path` (such as POISON_LIB_PATH) while the block runs; yields it.  The
    switch is process-wide: calls from other threads during the block use
    that build too."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"GEMM library not built: {path} is missing "
                           "(run __graft_entry__.build() or barrier_pipelined_tiled_amd/build.py)")
    L = ctypes.CDLL(path)
    i64, p, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.gemm_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ci, p]
    L.gemm_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ci, p]
    L.gemm_batched_f16.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, ci, p]
    L.gemm_ex.argtypes = [ci, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, ci, ci, p]
    L.gemm_ex_bt.argtypes = [ci, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, ci, ci, p]
    L.gemm_ex_noalloc.argtypes = [ci, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, ci, ci, p]
    L.bpt_noalloc_scratch_bytes.argtypes = []
    L.bpt_noalloc_scratch_bytes.restype = i64
    L.attention_fwd.argtypes = [ci, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64,
                                p, i64, i64, ctypes.c_float, ci, p]
    for fn in (L.gemm_f16, L.gemm_bf16, L.gemm_batched_f16, L.gemm_ex, L.gemm_ex_bt, L.gemm_ex_noalloc,
               L.attention_fwd):
        fn.restype = ci
    L.bpt_select_variant.argtypes = [ci, i64, i64, i64, i64, p, i64, p, i64, ci]
    L.bpt_select_variant.restype = ci
    L.bpt_select_variant_bt.argtypes = [ci, i64, i64, i64, i64, p, i64, p, i64, ci]
    L.bpt_select_variant_bt.restype = ci
    L.bpt_variant_count.argtypes = []
    L.bpt_variant_count.restype = ci
    L.bpt_variant_name.argtypes = [ci]
    L.bpt_variant_name.restype = ctypes.c_char_p
    L.bpt_status_string.argtypes = [ci]
    L.bpt_status_string.restype = ctypes.c_char_p
    L.bpt_last_error.argtypes = []
    L.bpt_last_error.restype = ctypes.c_char_p
    return L


def _check(status: int) -> None:
    if status != BPT_OK:
        raise GemmError(status, lib().bpt_last_error().decode())


def variants() -> dict:
    """Variant name -> id (ids are what gemm_ex(variant=...) takes)."""
    L = lib()
    return {L.bpt_variant_name(v).decode(): v for v in range(1, L.bpt_variant_count() + 1)}


def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    # the current stream's raw handle without building a Stream object (which
    # costs about 3 us, as much as the library call); the public route when
    # this torch build lacks the direct query
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return ctypes.c_void_p(raw(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _mat(t, name):
    """(rows, cols, ld, batch_stride, batch) of a 2-D or 3-D row-major tensor
    (read from shape and strides directly: this runs three times per call)."""
    shape = t.shape
    st = t.stride()
    if len(shape) == 2:
        rows, cols = shape
        srow, scol = st
        batch, sb = 1, 0
    elif len(shape) == 3:
        batch, rows, cols = shape
        sb, srow, scol = st
        if batch <= 1:
            sb = 0
    else:
        raise ValueError(f"{name} must be 2-D or 3-D, got {tuple(shape)}")
    if cols > 1 and scol != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")
    return rows, cols, (srow if rows > 1 else max(cols, 1)), sb, batch


_DT = {"f16": 0, "bf16": 1}


def gemm_ex(A, B, C=None, *, dtype: str = "f16", out_fp32: bool = False, variant: int = 0,
            stream=None, _entry: str = "ex"):
    """C = A @ B through gemm_ex.  A (M,K) or (b,M,K), B (K,N) or (b,K,N);
    C is allocated when None.  Returns C."""
    torch = _torch()
    want = torch.float16 if dtype == "f16" else torch.bfloat16
    if A.dtype != want or B.dtype != want:
        raise TypeError(f"A and B must be {want}, got {A.dtype} and {B.dtype}")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    M, K, lda, sA, bA = _mat(A, "A")
    K2, N, ldb, sB, bB = _mat(B, "B")
    if K2 != K or bA != bB:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)}")
    out_t = torch.float32 if out_fp32 else want
    if C is None:
        shape = (M, N) if A.dim() == 2 else (bA, M, N)
        C = torch.empty(shape, dtype=out_t, device=A.device)
    if C.dtype != out_t:
        raise TypeError(f"C must be {out_t}, got {C.dtype}")
    Mc, Nc, ldc, sC, bC = _mat(C, "C")
    if (Mc, Nc, bC) != (M, N, bA):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(bA, M, N)}")
    L = lib()
    fn = L.gemm_ex_noalloc if _entry == "noalloc" else L.gemm_ex
    _check(fn(_DT[dtype], bA, M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB,
              C.data_ptr(), ldc, sC, int(out_fp32), int(variant), _stream_handle(stream)))
    return C


def gemm_ex_noalloc(A, B, C, *, dtype: str = "f16", out_fp32: bool = False, variant: int = 0,
                    stream=None):
    """C = A @ B through gemm_ex_noalloc (no device allocation in the call;
    scratch in the library's fixed device array).  C must be given."""
    return gemm_ex(A, B, C, dtype=dtype, out_fp32=out_fp32, variant=variant, stream=stream, _entry="noalloc")


def gemm_ex_bt(A, Bt, C=None, *, dtype: str = "f16", out_fp32: bool = False, variant: int = 0,
               stream=None):
    """C = A @ Bt^T through gemm_ex_bt.  A (M,K) or (b,M,K), Bt (N,K) or
    (b,N,K) -- B given transposed; C is allocated when None.  Returns C."""
    torch = _torch()
    want = torch.float16 if dtype == "f16" else torch.bfloat16
    if A.dtype != want or Bt.dtype != want:
        raise TypeError(f"A and Bt must be {want}, got {A.dtype} and {Bt.dtype}")
    if not (A.is_cuda and Bt.is_cuda):
        raise ValueError("A and Bt must be device tensors")
    M, K, lda, sA, bA = _mat(A, "A")
    N, K2, ldbt, sB, bB = _mat(Bt, "Bt")
    if K2 != K or bA != bB:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} Bt {tuple(Bt.shape)}")
    out_t = torch.float32 if out_fp32 else want
    if C is None:
        shape = (M, N) if A.dim() == 2 else (bA, M, N)
        C = torch.empty(shape, dtype=out_t, device=A.device)
    if C.dtype != out_t:
        raise TypeError(f"C must be {out_t}, got {C.dtype}")
    Mc, Nc, ldc, sC, bC = _mat(C, "C")
    if (Mc, Nc, bC) != (M, N, bA):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(bA, M, N)}")
    _check(lib().gemm_ex_bt(_DT[dtype], bA, M, N, K, A.data_ptr(), lda, sA, Bt.data_ptr(), ldbt, sB,
                            C.data_ptr(), ldc, sC, int(out_fp32), int(variant), _stream_handle(stream)))
    return C


def attention_fwd(Q, K, V, O=None, *, scale: float | None = None, dtype: str = "f16",
                  out_fp32: bool = False, stream=None):
    """O = softmax(scale * Q K^T) V through attention_fwd.  Q (Sq, D) or
    (BH, Sq, D); K, V (Skv, D) or (BH, Skv, D); scale defaults to
    1/sqrt(D).  O is allocated when None.  Returns O."""
    torch = _torch()
    want = torch.float16 if dtype == "f16" else torch.bfloat16
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        if t.dtype != want:
            raise TypeError(f"{n} must be {want}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{n} must be a device tensor")
    Sq, D, ldq, sQ, BH = _mat(Q, "Q")
    Skv, Dk, ldk, sK, bK = _mat(K, "K")
    Skv2, Dv, ldv, sV, bV = _mat(V, "V")
    if Dk != D or Dv != D or Skv2 != Skv or bK != BH or bV != BH:
        raise ValueError(f"shape mismatch: Q {tuple(Q.shape)} K {tuple(K.shape)} V {tuple(V.shape)}")
    out_t = torch.float32 if out_fp32 else want
    if O is None:
        O = torch.empty(Q.shape, dtype=out_t, device=Q.device)
    if O.dtype != out_t:
        raise TypeError(f"O must be {out_t}, got {O.dtype}")
    So, Do, ldo, sO, bO = _mat(O, "O")
    if (So, Do, bO) != (Sq, D, BH):
        raise ValueError(f"O has shape {tuple(O.shape)}, expected {tuple(Q.shape)}")
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    _check(lib().attention_fwd(_DT[dtype], BH, Sq, Skv, D, Q.data_ptr(), ldq, sQ, K.data_ptr(), ldk, sK,
                               V.data_ptr(), ldv, sV, O.data_ptr(), ldo, sO, float(scale), int(out_fp32),
                               _stream_handle(stream)))
    return O


def gemm_f16(A, B, C=None, *, out_fp32: bool = False, stream=None):
    """fp16 C = A @ B through gemm_f16 (2-D tensors)."""
    torch = _torch()
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("gemm_f16 takes 2-D tensors; use gemm_batched_f16 for batches")
    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("gemm_f16 takes float16 tensors")
    M, K, lda, _, _ = _mat(A, "A")
    _, N, ldb, _, _ = _mat(B, "B")
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32 if out_fp32 else torch.float16, device=A.device)
    _, _, ldc, _, _ = _mat(C, "C")
    _check(lib().gemm_f16(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                          int(out_fp32), _stream_handle(stream)))
    return C


def gemm_bf16(A, B, C=None, *, out_fp32: bool = False, stream=None):
    """bf16 C = A @ B through gemm_bf16 (2-D tensors)."""
    torch = _torch()
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("gemm_bf16 takes 2-D tensors")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16 takes bfloat16 tensors")
    M, K, lda, _, _ = _mat(A, "A")
    _, N, ldb, _, _ = _mat(B, "B")
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32 if out_fp32 else torch.bfloat16, device=A.device)
    _, _, ldc, _, _ = _mat(C, "C")
    _check(lib().gemm_bf16(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                           int(out_fp32), _stream_handle(stream)))
    return C


def gemm_batched_f16(A, B, C=None, *, out_fp32: bool = False, stream=None):
    """Batched fp16 C[b] = A[b] @ B[b] through gemm_batched_f16 (3-D tensors)."""
    torch = _torch()
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("gemm_batched_f16 takes 3-D tensors")
    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("gemm_batched_f16 takes float16 tensors")
    M, K, lda, sA, batch = _mat(A, "A")
    _, N, ldb, sB, bB = _mat(B, "B")
    if B.shape[1] != K or bB != batch:
        raise ValueError("shape mismatch")
    if C is None:
        C = torch.empty((batch, M, N), dtype=torch.float32 if out_fp32 else torch.float16, device=A.device)
    _, _, ldc, sC, _ = _mat(C, "C")
    _check(lib().gemm_batched_f16(batch, M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB,
                                  C.data_ptr(), ldc, sC, int(out_fp32), _stream_handle(stream)))
    return C


def select_variant(dtype: str, batch: int, M: int, N: int, K: int, lda: int, ldb: int,
                   out_fp32: bool = False, A_ptr: int = 0, B_ptr: int = 0, bt: bool = False) -> int:
    """Variant id the automatic choice would run (0: rejected / nothing to do).
    bt: for gemm_ex_bt (B given transposed, ldb is then Bt's leading dimension)."""
    fn = lib().bpt_select_variant_bt if bt else lib().bpt_select_variant
    return int(fn(_DT[dtype], batch, M, N, K, A_ptr or 256, lda, B_ptr or 256, ldb, int(out_fp32)))
