"""CPU oracle for the dense half-precision GEMM C = A * B, and for the
second workload, scaled dot-product attention O = softmax(scale Q K^T) V.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports or calls anything here, and nothing here imports the GPU package.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation in
ascending k, one rounding to fp32).  This module loads it with ctypes and
adds the comparison metrics of the "Xe2 ESIMD GEMM" page, section
"Correctness testing": look for non-finite values first, then judge the
relative RMS error (read as the Frobenius norm of the difference over the
Frobenius norm of the reference).

Attention (``attention``) is the plain definition in fp64, row by row
(oracle.c, oracle_attention), judged by ``compare_attention``.

Inputs are numpy ``uint16`` arrays of 16-bit bit patterns (fp16 or bf16),
2-D ``(rows, cols)`` or 3-D ``(batch, rows, cols)``, contiguous in the last
dimension; leading dimensions and batch strides are taken from the array
strides, so sub-block views work.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# No -ffast-math: the ascending-k fp64 summation must run as written.
GCC_CMD = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH, _SRC, "-lm"]


def build() -> str:
    """Compile oracle.c into liboracle.so next to it; return the path."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    for name in ("oracle_decode_f16", "oracle_decode_bf16", "oracle_encode_f16", "oracle_encode_bf16"):
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [p, p, i64]
    lib.oracle_gemm.restype = None
    lib.oracle_gemm.argtypes = [ctypes.c_int, i64, i64, i64, i64,
                                p, i64, i64, p, i64, i64, p, p, i64, i64]
    lib.oracle_gemm_at.restype = None
    lib.oracle_gemm_at.argtypes = [ctypes.c_int, i64, p, i64, i64, p, i64, i64,
                                   i64, p, p, p, p, p]
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [ctypes.c_int, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64,
                                     ctypes.c_double, i64, p, p, p, p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


_DTYPES = {"f16": 0, "bf16": 1}


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Run the oracle's parallel loops on n threads (results do not depend
    on n: each output element is summed by one thread, in ascending k)."""
    _load().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------------------
# decoders / encoders
# ----------------------------------------------------------------------------

def decode(bits: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """Exact value of each 16-bit pattern as float64."""
    src = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(src.shape, dtype=np.float64)
    fn = _load().oracle_decode_f16 if dtype == "f16" else _load().oracle_decode_bf16
    fn(src.ctypes.data, out.ctypes.data, src.size)
    return out


def encode(values: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """fp32 values -> 16-bit patterns, round to nearest even."""
    src = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint16)
    fn = _load().oracle_encode_f16 if dtype == "f16" else _load().oracle_encode_bf16
    fn(src.ctypes.data, out.ctypes.data, src.size)
    return out


# ----------------------------------------------------------------------------
# the product
# ----------------------------------------------------------------------------

def _as3d(x: np.ndarray, name: str):
    if x.dtype != np.uint16:
        raise TypeError(f"{name} must hold uint16 bit patterns, got {x.dtype}")
    if x.ndim == 2:
        x = x[None]
    if x.ndim != 3:
        raise ValueError(f"{name} must be 2-D or 3-D")
    if x.size == 0:
        return x, max(x.shape[2], 1), 0
    if x.shape[2] > 1 and x.strides[2] != 2:
        raise ValueError(f"{name} must be contiguous in its last dimension")
    ld = x.strides[1] // 2 if x.shape[1] > 1 else max(x.shape[2], 1)
    sb = x.strides[0] // 2 if x.shape[0] > 1 else 0
    return x, ld, sb


def gemm(a: np.ndarray, b: np.ndarray, dtype: str = "f16", want64: bool = False):
    """C = A * B for 16-bit pattern inputs.

    ``a``: (M, K) or (batch, M, K); ``b``: (K, N) or (batch, K, N).
    Returns the fp32 result (same rank as ``a``), and the unrounded fp64
    sums as well when ``want64``.
    """
    two_d = a.ndim == 2
    a3, lda, sa = _as3d(a, "A")
    b3, ldb, sb = _as3d(b, "B")
    batch, M, K = a3.shape
    if b3.shape[0] != batch or b3.shape[1] != K:
        raise ValueError(f"shape mismatch: A {a.shape}, B {b.shape}")
    N = b3.shape[2]
    c32 = np.empty((batch, M, N), dtype=np.float32)
    c64 = np.empty((batch, M, N), dtype=np.float64) if want64 else None
    if batch and M and N:
        _load().oracle_gemm(_DTYPES[dtype], batch, M, N, K,
                            a3.ctypes.data, lda, sa, b3.ctypes.data, ldb, sb,
                            c32.ctypes.data, c64.ctypes.data if want64 else None,
                            N, M * N)
    if two_d:
        c32 = c32[0]
        c64 = c64[0] if want64 else None
    return (c32, c64) if want64 else c32


def gemm_at(a: np.ndarray, b: np.ndarray, bidx, rows, cols, dtype: str = "f16",
            want64: bool = False):
    """C at chosen positions (bidx[t], rows[t], cols[t]), each a plain
    ascending-k dot product.  For products too large to form whole."""
    a3, lda, sa = _as3d(a, "A")
    b3, ldb, sb = _as3d(b, "B")
    K = a3.shape[2]
    bi = np.ascontiguousarray(bidx, dtype=np.int64)
    ri = np.ascontiguousarray(rows, dtype=np.int64)
    ci = np.ascontiguousarray(cols, dtype=np.int64)
    n = ri.size
    if not (bi.size == n == ci.size):
        raise ValueError("position arrays differ in length")
    if n and (bi.min() < 0 or bi.max() >= a3.shape[0] or ri.min() < 0 or ri.max() >= a3.shape[1]
              or ci.min() < 0 or ci.max() >= b3.shape[2]):
        raise ValueError("position out of range")
    out32 = np.empty(n, dtype=np.float32)
    out64 = np.empty(n, dtype=np.float64)
    if n:
        _load().oracle_gemm_at(_DTYPES[dtype], K, a3.ctypes.data, lda, sa, b3.ctypes.data, ldb, sb,
                               n, bi.ctypes.data, ri.ctypes.data, ci.ctypes.data,
                               out32.ctypes.data, out64.ctypes.data)
    return (out32, out64) if want64 else out32


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, dtype: str = "f16",
              rows=None, want64: bool = False):
    """O = softmax(scale * Q K^T) V for 16-bit pattern inputs (oracle.c,
    oracle_attention).

    ``q``: (Sq, D) or (BH, Sq, D); ``k``, ``v``: (Skv, D) or (BH, Skv, D).
    With ``rows`` None every output row is formed and the result has q's
    shape; with ``rows = (bh_idx, row_idx)`` only those rows are, returned as
    (n, D).  fp32 results, plus the fp64 values when ``want64``.
    ``scale`` is taken as the fp32 value the GPU receives."""
    two_d = q.ndim == 2
    q3, ldq, sq = _as3d(q, "Q")
    k3, ldk, sk = _as3d(k, "K")
    v3, ldv, sv = _as3d(v, "V")
    BH, Sq, D = q3.shape
    if k3.shape[0] != BH or v3.shape[0] != BH or k3.shape[2] != D or v3.shape[2] != D \
            or k3.shape[1] != v3.shape[1]:
        raise ValueError(f"shape mismatch: Q {q.shape}, K {k.shape}, V {v.shape}")
    Skv = k3.shape[1]
    if rows is None:
        bi = np.repeat(np.arange(BH, dtype=np.int64), Sq)
        ri = np.tile(np.arange(Sq, dtype=np.int64), BH)
    else:
        bi = np.ascontiguousarray(rows[0], dtype=np.int64)
        ri = np.ascontiguousarray(rows[1], dtype=np.int64)
        if bi.size != ri.size:
            raise ValueError("row index arrays differ in length")
        if bi.size and (bi.min() < 0 or bi.max() >= BH or ri.min() < 0 or ri.max() >= Sq):
            raise ValueError("row out of range")
    n = bi.size
    out32 = np.zeros((n, D), dtype=np.float32)
    out64 = np.zeros((n, D), dtype=np.float64)
    if n and D:
        _load().oracle_attention(_DTYPES[dtype], Skv, D, q3.ctypes.data, ldq, sq,
                                 k3.ctypes.data, ldk, sk, v3.ctypes.data, ldv, sv,
                                 float(np.float32(scale)), n, bi.ctypes.data, ri.ctypes.data,
                                 out32.ctypes.data, out64.ctypes.data)
    if rows is None:
        out32 = out32.reshape(BH, Sq, D)
        out64 = out64.reshape(BH, Sq, D)
        if two_d:
            out32, out64 = out32[0], out64[0]
    return (out32, out64) if want64 else out32


# ----------------------------------------------------------------------------
# comparison metrics
# ----------------------------------------------------------------------------

REL_RMS_TOL = 5e-3


def max_abs_tol(K: int, ref_absmax: float) -> float:
    """Element-wise bound 2e-2 * sqrt(max(K, 256)/256) * max|C_ref|.

    The sqrt(K/256) growth is measured from the 256-wide correctness shape;
    for K < 256 the K = 256 bound applies, since a shorter sum accumulates
    no more error and the bound must still admit the output rounding of a
    16-bit result (half an ulp of bf16 is 2^-9 of the value)."""
    return 2e-2 * np.sqrt(max(K, 256) / 256.0) * ref_absmax


def compare(gpu: np.ndarray, ref: np.ndarray, K: int) -> dict:
    """Judge a GPU result against the oracle's fp32 reference.

    Non-finite values are counted first (a NaN would otherwise slip through
    a ratio test).  rel_rms = ||G - R||_F / ||R||_F and max_abs = max|G - R|
    are computed in fp64.  When the reference is identically zero, the
    relative metrics are undefined and only G == 0 passes.
    """
    return _judge(gpu, ref, lambda absmax: max_abs_tol(K, absmax))


# Attention outputs are convex combinations of value rows, so every error is
# relative to the values' scale, not to a length of sum: the weights enter
# the second product rounded to 16 bits (relative error <= 2^-11 each for
# fp16) and the output is rounded once more, which bounds the element-wise
# error by a few 2^-11 of max|O|.  1e-2 * max|O_ref| leaves a wide margin
# for that and still fails a dropped term, a wrong scale or a missed
# rescale of the running sums (each moves outputs by far more).
ATTN_MAX_ABS_REL = 1e-2


def compare_attention(gpu: np.ndarray, ref: np.ndarray) -> dict:
    """Judge a GPU attention output against the oracle's: non-finite count
    first, then rel_rms <= 5e-3 (the pages' criterion) and max|G - R| <=
    1e-2 * max|R|."""
    return _judge(gpu, ref, lambda absmax: ATTN_MAX_ABS_REL * absmax)


def _judge(gpu, ref, tol_of_absmax) -> dict:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    nonfinite = int(g.size - np.count_nonzero(np.isfinite(g)))
    ref_nonfinite = int(r.size - np.count_nonzero(np.isfinite(r)))
    out = {"nonfinite": nonfinite, "ref_nonfinite": ref_nonfinite, "n": int(g.size)}
    if nonfinite or ref_nonfinite:
        out.update(rel_rms=float("nan"), max_abs=float("nan"), ok=False)
        return out
    diff = g - r
    rnorm = float(np.sqrt(np.sum(r * r)))
    ref_absmax = float(np.max(np.abs(r))) if r.size else 0.0
    max_abs = float(np.max(np.abs(diff))) if r.size else 0.0
    if rnorm == 0.0:
        out.update(rel_rms=0.0 if max_abs == 0.0 else float("inf"), max_abs=max_abs,
                   max_abs_tol=0.0, ok=(max_abs == 0.0))
        return out
    rel_rms = float(np.sqrt(np.sum(diff * diff)) / rnorm)
    tol = float(tol_of_absmax(ref_absmax))
    out.update(rel_rms=rel_rms, max_abs=max_abs, max_abs_tol=tol,
               ok=bool(rel_rms <= REL_RMS_TOL and max_abs <= tol))
    return out
