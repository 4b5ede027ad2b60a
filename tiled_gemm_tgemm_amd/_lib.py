"""ctypes binding of libtgemm.so: the C entry points under the same names.

Argument marshalling only — every step of the product runs in the HIP
kernels of libtgemm.so.  If the library has not been built this module
raises; there is no other code path.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libtgemm.so")

# tgemm_status_t values (include/tgemm.h)
TGEMM_SUCCESS = 0
TGEMM_ERROR_INVALID_VALUE = 1
TGEMM_ERROR_NOT_SUPPORTED = 2
TGEMM_ERROR_HIP = 3
# size of the fixed device scratch behind tgemm_sgemm_splitk_noalloc (include/tgemm.h)
TGEMM_SPLITK_NOALLOC_BYTES = 32 << 20

# every function the header declares, with (restype, argtypes)
_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p
_GEMM = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64]
TGEMM_OP_N = 0
TGEMM_OP_T = 1
# tgemm_transpose_kernel_t values
TGEMM_TRANSPOSE_BLOCKED = 0
TGEMM_TRANSPOSE_NAIVE = 1
TGEMM_TRANSPOSE_TILED = 2
TGEMM_TRANSPOSE_TILED_PADDED = 3

SIGNATURES = {
    "tgemm_sgemm": (ctypes.c_int, _GEMM + [_ptr]),
    "tgemm_sgemm_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + _GEMM + [_ptr]),
    "tgemm_sgemm_mfma_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + _GEMM + [ctypes.c_int, _ptr]),
    "tgemm_sgemm_variant_for_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + _GEMM),
    "tgemm_sgemm_mfma": (ctypes.c_int, _GEMM + [ctypes.c_int, _ptr]),
    "tgemm_mfma_variant_count": (ctypes.c_int, []),
    "tgemm_mfma_variant_name": (ctypes.c_char_p, [ctypes.c_int]),
    "tgemm_sgemm_variant_for": (ctypes.c_int, _GEMM),
    "tgemm_sgemm_naive": (ctypes.c_int, _GEMM + [_ptr]),
    "tgemm_sgemm_lds": (ctypes.c_int, _GEMM + [ctypes.c_int, ctypes.c_int, _ptr]),
    "tgemm_sgemm_simt": (ctypes.c_int, _GEMM + [_ptr]),
    "tgemm_transpose": (ctypes.c_int, [_i64, _i64, _ptr, _i64, _ptr, _i64, ctypes.c_int, _ptr]),
    "tgemm_sgemm_host": (ctypes.c_int, _GEMM + [_ptr, _i64, _i64, _ptr, _ptr, _ptr]),
    "tgemm_sgemm_host_workspace_size": (_i64, [_i64, _i64, _i64, _i64]),
    "tgemm_sgemm_splitk": (ctypes.c_int, _GEMM + [ctypes.c_int, _ptr, ctypes.c_size_t, _ptr]),
    "tgemm_sgemm_splitk_ex": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + _GEMM
                              + [ctypes.c_int, _ptr, ctypes.c_size_t, _ptr]),
    "tgemm_sgemm_splitk_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_int] + _GEMM + [ctypes.c_int, _ptr]),
    "tgemm_sgemm_splitk_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, ctypes.c_int]),
    "tgemm_sgemm_splitk_choose": (ctypes.c_int, [_i64, _i64, _i64]),
    "tgemm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tgemm_version": (ctypes.c_int, []),
}

_lib = None


class TgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {tgemm_status_string(status)} (status {status})")


def library():
    """The loaded libtgemm.so (loads it on first use; raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is not built; run `python -m tiled_gemm_tgemm_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        for name, (restype, argtypes) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = restype
            fn.argtypes = argtypes
        _lib = lib
    return _lib


# ---- the C entry points, same names and argument order ---------------------

def tgemm_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return library().tgemm_sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream)


def tgemm_sgemm_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return library().tgemm_sgemm_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, stream)


def tgemm_sgemm_mfma_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, variant, stream=None) -> int:
    return library().tgemm_sgemm_mfma_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, variant, stream)


def tgemm_sgemm_variant_for_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return library().tgemm_sgemm_variant_for_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc)


def tgemm_sgemm_mfma(M, N, K, A, lda, B, ldb, C, ldc, variant, stream=None) -> int:
    return library().tgemm_sgemm_mfma(M, N, K, A, lda, B, ldb, C, ldc, variant, stream)


def tgemm_sgemm_naive(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return library().tgemm_sgemm_naive(M, N, K, A, lda, B, ldb, C, ldc, stream)


def tgemm_sgemm_lds(M, N, K, A, lda, B, ldb, C, ldc, tile, pad, stream=None) -> int:
    return library().tgemm_sgemm_lds(M, N, K, A, lda, B, ldb, C, ldc, tile, pad, stream)


def tgemm_sgemm_simt(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return library().tgemm_sgemm_simt(M, N, K, A, lda, B, ldb, C, ldc, stream)


def tgemm_transpose(M, N, A, lda, B, ldb, kernel=TGEMM_TRANSPOSE_BLOCKED, stream=None) -> int:
    return library().tgemm_transpose(M, N, A, lda, B, ldb, kernel, stream)


def tgemm_sgemm_host(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, panel_rows,
                     compute=None, copy_in=None, copy_out=None) -> int:
    return library().tgemm_sgemm_host(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes,
                                      panel_rows, compute, copy_in, copy_out)


def tgemm_sgemm_host_workspace_size(M, N, K, panel_rows=0) -> int:
    return library().tgemm_sgemm_host_workspace_size(M, N, K, panel_rows)


def tgemm_sgemm_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_bytes,
                       stream=None) -> int:
    return library().tgemm_sgemm_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace,
                                        workspace_bytes, stream)


def tgemm_sgemm_splitk_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_bytes,
                          stream=None) -> int:
    return library().tgemm_sgemm_splitk_ex(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, splits, workspace,
                                           workspace_bytes, stream)


def tgemm_sgemm_splitk_noalloc(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, splits, stream=None) -> int:
    return library().tgemm_sgemm_splitk_noalloc(op_a, op_b, M, N, K, A, lda, B, ldb, C, ldc, splits, stream)


def tgemm_sgemm_splitk_workspace_size(M, N, K, splits) -> int:
    return library().tgemm_sgemm_splitk_workspace_size(M, N, K, splits)


def tgemm_sgemm_splitk_choose(M, N, K) -> int:
    return library().tgemm_sgemm_splitk_choose(M, N, K)


def tgemm_mfma_variant_count() -> int:
    return library().tgemm_mfma_variant_count()


def tgemm_mfma_variant_name(variant: int):
    name = library().tgemm_mfma_variant_name(variant)
    return name.decode() if name is not None else None


def tgemm_sgemm_variant_for(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return library().tgemm_sgemm_variant_for(M, N, K, A, lda, B, ldb, C, ldc)


def tgemm_status_string(status: int) -> str:
    return library().tgemm_status_string(status).decode()


def tgemm_version() -> int:
    return library().tgemm_version()
