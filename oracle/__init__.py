"""CPU oracle for C = A·B  —  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path
(``tiled_gemm_tgemm_amd``) never imports it, and this package imports nothing
from there: the two share no code.  Inputs for both come from the seeded
generator module ``tiled_gemm_tgemm_amd.workloads``, which draws numbers only.

The arithmetic lives in plain C (``oracle.c``, loaded through ctypes); this
file only marshals numpy arrays.  Definitions followed, all on page 1
("[Multi-Core & GPU Programming] CUDA - Matrix Multiplication"):

* ``gemm``/``gemm_window``/``gemm_blocks``: section [Matrix Multiplication],
  P(i,j) = sum_k M(i,k)·N(k,j), in float64 with exact products;
* ``gemm_i64``: the same definition in exact integer arithmetic;
* ``gemm_fma_f32``: the register accumulator of the pages' kernels (sections
  [Matrix Multiplication] "sum" loop and [Shared Memory] Pvalue loop), one
  float32 fused multiply-add per k in ascending order;
* ``checksums``: row/column sums of the product, formed without the product;
* ``transpose``: page 2 ("Lec 29 · GPU Architecture (2)"), §1.4 — element
  (i, j) of the input moves to (j, i) of the output, as a 32-bit word.

Pins (what ties these to something other than themselves) are in
``tests/test_oracle_pins.py``.  The structural models of the pages' kernels
(index maps, phases, load counts, the bank model) are in ``oracle.models``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIBRARY):
        _build.build()
    lib = ctypes.CDLL(_build.LIBRARY)
    lib.oracle_gemm_f64_window.restype = ctypes.c_int
    lib.oracle_gemm_f64_window.argtypes = [_i64, _i64, _i64, _f32p, _i64, _f32p, _i64,
                                           _i64, _i64, _i64, _i64,
                                           _f64p, _i64, ctypes.c_void_p, _i64]
    lib.oracle_gemm_i64.restype = ctypes.c_int
    lib.oracle_gemm_i64.argtypes = [_i64, _i64, _i64, _f32p, _i64, _f32p, _i64, _i64p, _i64]
    lib.oracle_gemm_fma_f32.restype = ctypes.c_int
    lib.oracle_gemm_fma_f32.argtypes = [_i64, _i64, _i64, _f32p, _i64, _f32p, _i64, _f32p, _i64]
    lib.oracle_checksums.restype = ctypes.c_int
    lib.oracle_checksums.argtypes = [_i64, _i64, _i64, _f32p, _i64, _f32p, _i64,
                                     _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_transpose.restype = ctypes.c_int
    lib.oracle_transpose.argtypes = [_i64, _i64, _u32p, _i64, _u32p, _i64]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc == -2:
        raise OracleError(f"{what}: inputs are not integers below 2^24")
    if rc != 0:
        raise OracleError(f"{what}: invalid arguments (code {rc})")


def _operands(A, B):
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {A.shape} and {B.shape} do not chain")
    M, K = A.shape
    N = B.shape[1]
    # a zero-sized axis still needs a valid (non-null) buffer and ld >= 1
    if A.size == 0:
        A = np.zeros((max(M, 1), max(K, 1)), np.float32)
    if B.size == 0:
        B = np.zeros((max(K, 1), max(N, 1)), np.float32)
    return A, B, M, N, K


def gemm_window(A, B, i0, i1, j0, j1, with_abs=True, lib=None):
    """(P, S) for output rows [i0,i1) and columns [j0,j1); S is None if not asked."""
    lib = lib or _load()
    A, B, M, N, K = _operands(A, B)
    h, w = i1 - i0, j1 - j0
    P = np.empty((max(h, 1), max(w, 1)), np.float64)
    S = np.empty_like(P) if with_abs else None
    rc = lib.oracle_gemm_f64_window(M, N, K, A, A.shape[1], B, B.shape[1], i0, i1, j0, j1,
                                    P, P.shape[1],
                                    S.ctypes.data if S is not None else None,
                                    P.shape[1])
    _check(rc, "oracle_gemm_f64_window")
    P = P[:h, :w]
    S = S[:h, :w] if S is not None else None
    return P, S


def gemm(A, B, with_abs=True, lib=None):
    """Full product in float64: (P, S) with S_ij = sum_k |A_ik·B_kj|."""
    A_, B_ = np.asarray(A), np.asarray(B)
    return gemm_window(A_, B_, 0, A_.shape[0], 0, B_.shape[1], with_abs, lib)


def gemm_blocks(A, B, origins, size, lib=None):
    """[(P, S)] for the size×size output blocks whose top-left corners are `origins`."""
    return [gemm_window(A, B, r, r + size, c, c + size, True, lib) for r, c in origins]


def gemm_i64(A, B, lib=None):
    """Exact integer product of integer-valued float32 matrices (int64)."""
    lib = lib or _load()
    A, B, M, N, K = _operands(A, B)
    P = np.empty((max(M, 1), max(N, 1)), np.int64)
    _check(lib.oracle_gemm_i64(M, N, K, A, A.shape[1], B, B.shape[1], P, P.shape[1]),
           "oracle_gemm_i64")
    return P[:M, :N]


def gemm_fma_f32(A, B, lib=None):
    """float32 sequential fused-multiply-add model (k ascending, from +0)."""
    lib = lib or _load()
    A, B, M, N, K = _operands(A, B)
    C = np.empty((max(M, 1), max(N, 1)), np.float32)
    _check(lib.oracle_gemm_fma_f32(M, N, K, A, A.shape[1], B, B.shape[1], C, C.shape[1]),
           "oracle_gemm_fma_f32")
    return C[:M, :N]


def checksums(A, B, lib=None):
    """(row, rowabs, col, colabs): sums of P over j and over i, and of S likewise."""
    lib = lib or _load()
    A, B, M, N, K = _operands(A, B)
    row = np.empty(max(M, 1)); rowabs = np.empty(max(M, 1))
    col = np.empty(max(N, 1)); colabs = np.empty(max(N, 1))
    work = np.empty(4 * max(K, 1))
    _check(lib.oracle_checksums(M, N, K, A, A.shape[1], B, B.shape[1],
                                row, rowabs, col, colabs, work), "oracle_checksums")
    return row[:M], rowabs[:M], col[:N], colabs[:N]


def transpose(A, lib=None):
    """Aᵀ of a 2-D float32 array (N×M for M×N), every element's bits unchanged."""
    lib = lib or _load()
    A = np.ascontiguousarray(A, dtype=np.float32)
    if A.ndim != 2:
        raise ValueError(f"transpose needs a 2-D array, got shape {A.shape}")
    M, N = A.shape
    src = A.view(np.uint32) if A.size else np.zeros((max(M, 1), max(N, 1)), np.uint32)
    out = np.empty((max(N, 1), max(M, 1)), np.uint32)
    _check(lib.oracle_transpose(M, N, src, src.shape[1], out, out.shape[1]), "oracle_transpose")
    return out[:N, :M].view(np.float32)


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int((lib or _load()).oracle_num_threads())


def open_library(path: str):
    """ctypes handle for another build of oracle.c, with the same signatures.

    Used by the mutation tests, which plant a mistake in a copy of oracle.c
    and check that the pins catch it.
    """
    global _lib
    saved, _lib = _lib, None
    saved_path = _build.LIBRARY
    try:
        _build.LIBRARY = path
        lib = _load()
    finally:
        _build.LIBRARY = saved_path
        _lib = saved
    return lib
