"""tiled_gemm_tgemm_amd: fp32 C = A·B for one MI355X (gfx950), hand-written HIP.

The compute lives in the C-ABI library libtgemm.so (sources in csrc/,
declarations in include/tgemm.h).  ``_lib`` exposes the C entry points under
their own names; ``sgemm`` and ``transpose`` below are the same calls for
torch tensors, with torch used for device memory and the current stream only.

Nothing here loads the library at import time; the first call does, and it
raises if libtgemm.so has not been built (``python -m
tiled_gemm_tgemm_amd.build``).
"""

from __future__ import annotations

from ._lib import (  # noqa: F401
    TGEMM_OP_N,
    TGEMM_OP_T,
    TGEMM_ERROR_HIP,
    TGEMM_ERROR_INVALID_VALUE,
    TGEMM_ERROR_NOT_SUPPORTED,
    TGEMM_SUCCESS,
    TGEMM_TRANSPOSE_BLOCKED,
    TGEMM_TRANSPOSE_NAIVE,
    TGEMM_TRANSPOSE_TILED,
    TGEMM_TRANSPOSE_TILED_PADDED,
    TgemmError,
    library,
    tgemm_mfma_variant_count,
    tgemm_mfma_variant_name,
    tgemm_sgemm,
    tgemm_sgemm_ex,
    tgemm_sgemm_lds,
    tgemm_sgemm_mfma,
    tgemm_sgemm_mfma_ex,
    tgemm_sgemm_variant_for_ex,
    tgemm_sgemm_naive,
    tgemm_sgemm_simt,
    tgemm_sgemm_host,
    tgemm_sgemm_host_workspace_size,
    tgemm_sgemm_splitk,
    tgemm_sgemm_splitk_ex,
    tgemm_sgemm_splitk_choose,
    tgemm_sgemm_splitk_noalloc,
    tgemm_sgemm_splitk_workspace_size,
    TGEMM_SPLITK_NOALLOC_BYTES,
    tgemm_sgemm_variant_for,
    tgemm_status_string,
    tgemm_transpose,
    tgemm_version,
)

KERNELS = ("auto", "mfma", "naive", "lds", "simt")


def _check(t, name):
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 torch tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must live on a GPU")
    return t


def _layout(t, name):
    """(op, ld) of a 2-D tensor: row-major (TGEMM_OP_N, row stride) or a
    transposed view of a row-major matrix (TGEMM_OP_T, column stride)."""
    rows, cols = t.shape
    if t.stride(1) == 1 or cols <= 1:
        return TGEMM_OP_N, max(t.stride(0), cols, 1)
    if t.stride(0) == 1 or rows <= 1:
        return TGEMM_OP_T, max(t.stride(1), rows, 1)
    raise ValueError(f"{name} must be row-major or a transposed row-major view")


def _hold_for_stream(stream, device, *tensors):
    """Tensors allocated here (on torch's current stream) but used by work
    queued on another `stream`.  Torch's caching allocator orders a block's
    reuse on the stream it was allocated on only, so: `stream` first waits for
    the work already queued on the current stream (a block just handed out
    may still be in use there by its previous owner), and the tensors record
    `stream`, so that their memory is not handed out again, once they are
    released, before the work queued on `stream` so far has finished."""
    import torch

    if stream is None or not tensors:
        return
    current = torch.cuda.current_stream(device)
    if int(stream) == int(current.cuda_stream):
        return
    other = torch.cuda.ExternalStream(stream, device=device)
    other.wait_stream(current)
    for t in tensors:
        t.record_stream(other)


def sgemm(A, B, out=None, *, kernel="auto", variant=None, tile=16, pad=1, stream=None):
    """C = A·B for float32 CUDA tensors.

    A and B may be row-major with any leading dimension, or transposed views
    of row-major matrices (e.g. X.t()); those are passed as TGEMM_OP_T, with
    no copy.  `out` must be row-major.
    kernel: "auto" (tgemm_sgemm_ex), "mfma" (tgemm_sgemm_mfma_ex with
    `variant`; without one it is "auto"), "naive" (tgemm_sgemm_naive) or
    "lds" (tgemm_sgemm_lds with tile/pad) or "simt" (tgemm_sgemm_simt) — the
    last three for row-major operands only.  The call is queued on `stream` (default: torch's current
    stream) and returns `out` without waiting.
    """
    import torch

    A = _check(A, "A")
    B = _check(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    op_a, lda = _layout(A, "A")
    op_b, ldb = _layout(B, "B")
    made = []
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        made.append(out)
    else:
        out = _check(out, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be {M}x{N}")
        if out.stride(1) != 1 and N > 1:
            raise ValueError("out must be row-major")
    ldc = max(out.stride(0), N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    _hold_for_stream(stream, A.device, *made)
    args = (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc)
    if kernel in ("naive", "lds", "simt") and (op_a, op_b) != (TGEMM_OP_N, TGEMM_OP_N):
        raise ValueError(f"the {kernel} kernel takes row-major operands only")
    if kernel == "auto" or (kernel == "mfma" and variant is None):
        st = tgemm_sgemm_ex(op_a, op_b, *args, stream)
    elif kernel == "mfma":
        st = tgemm_sgemm_mfma_ex(op_a, op_b, *args, variant, stream)
    elif kernel == "naive":
        st = tgemm_sgemm_naive(*args, stream)
    elif kernel == "lds":
        st = tgemm_sgemm_lds(*args, tile, pad, stream)
    elif kernel == "simt":
        st = tgemm_sgemm_simt(*args, stream)
    else:
        raise ValueError(f"kernel must be one of {KERNELS}")
    if st != TGEMM_SUCCESS:
        raise TgemmError(st, f"tgemm ({kernel})")
    return out


def sgemm_splitk(A, B, out=None, *, splits=None, workspace=None, stream=None):
    """C = A·B for float32 CUDA tensors with K split across work-groups
    (tgemm_sgemm_splitk_ex), for shapes with few output tiles and a long K.
    A and B may be row-major or transposed views of row-major matrices, as
    for sgemm.  splits: None for the library's choice (tgemm_sgemm_splitk_choose),
    else 1 ... 64.  workspace: a CUDA uint8 tensor of at least
    tgemm_sgemm_splitk_workspace_size bytes (allocated if omitted; two calls
    in flight at once need two).  Queued on `stream` (default: torch's current
    stream); returns `out` without waiting."""
    import torch

    A = _check(A, "A")
    B = _check(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    op_a, lda = _layout(A, "A")
    op_b, ldb = _layout(B, "B")
    made = []
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        made.append(out)
    else:
        out = _check(out, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be {M}x{N}")
        if out.stride(1) != 1 and N > 1:
            raise ValueError("out must be row-major")
    ldc = max(out.stride(0), N, 1)
    if splits is None:
        splits = tgemm_sgemm_splitk_choose(M, N, K)
    need = tgemm_sgemm_splitk_workspace_size(M, N, K, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=A.device)
        made.append(workspace)
    elif not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a CUDA uint8 tensor")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    # the workspace is released on return while the work on `stream` may still run
    _hold_for_stream(stream, A.device, *made)
    st = tgemm_sgemm_splitk_ex(op_a, op_b, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc,
                               splits, workspace.data_ptr(), workspace.numel(), stream)
    if st != TGEMM_SUCCESS:
        raise TgemmError(st, "tgemm_sgemm_splitk_ex")
    return out


def sgemm_splitk_noalloc(A, B, out, *, splits=None, stream=None):
    """sgemm_splitk for callers that cannot allocate (tgemm_sgemm_splitk_noalloc):
    the partial products live in the library's fixed per-GPU scratch of
    TGEMM_SPLITK_NOALLOC_BYTES, so `out` must be given and nothing is
    allocated; calls overlapping in time on one GPU race.  Queued on `stream`
    (default: torch's current stream); returns `out` without waiting."""
    import torch

    A = _check(A, "A")
    B = _check(B, "B")
    out = _check(out, "out")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be {M}x{N}")
    if out.stride(1) != 1 and N > 1:
        raise ValueError("out must be row-major")
    op_a, lda = _layout(A, "A")
    op_b, ldb = _layout(B, "B")
    if splits is None:
        splits = tgemm_sgemm_splitk_choose(M, N, K)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    st = tgemm_sgemm_splitk_noalloc(op_a, op_b, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(),
                                    max(out.stride(0), N, 1), splits, stream)
    if st != TGEMM_SUCCESS:
        raise TgemmError(st, "tgemm_sgemm_splitk_noalloc")
    return out


TRANSPOSE_KERNELS = {"blocked": TGEMM_TRANSPOSE_BLOCKED, "naive": TGEMM_TRANSPOSE_NAIVE,
                     "tiled": TGEMM_TRANSPOSE_TILED, "tiled_padded": TGEMM_TRANSPOSE_TILED_PADDED}


def transpose(A, out=None, *, kernel="blocked", stream=None):
    """B = Aᵀ (tgemm_transpose) for a row-major float32 CUDA tensor A (any row
    stride); `out`, if given, must be row-major N×M and not overlap A.
    kernel: "blocked" (default), "naive", "tiled" or "tiled_padded".  Queued
    on `stream` (default: torch's current stream); returns `out` without waiting."""
    import torch

    A = _check(A, "A")
    M, N = A.shape
    if A.stride(1) != 1 and N > 1:
        raise ValueError("A must be row-major")
    made = []
    if out is None:
        out = torch.empty((N, M), dtype=torch.float32, device=A.device)
        made.append(out)
    else:
        out = _check(out, "out")
        if tuple(out.shape) != (N, M):
            raise ValueError(f"out must be {N}x{M}")
        if out.stride(1) != 1 and M > 1:
            raise ValueError("out must be row-major")
    if kernel not in TRANSPOSE_KERNELS:
        raise ValueError(f"kernel must be one of {tuple(TRANSPOSE_KERNELS)}")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    _hold_for_stream(stream, A.device, *made)
    st = tgemm_transpose(M, N, A.data_ptr(), max(A.stride(0), N, 1), out.data_ptr(), max(out.stride(0), M, 1),
                         TRANSPOSE_KERNELS[kernel], stream)
    if st != TGEMM_SUCCESS:
        raise TgemmError(st, f"tgemm_transpose ({kernel})")
    return out


def sgemm_host(A, B, out=None, *, panel_rows=0, streams=None, workspace=None):
    """C = A·B for float32 CPU tensors (tgemm_sgemm_host): copies overlapped
    with the product, C returned in host memory.  A, B (and `out`) should be
    pinned (``pin_memory()``) for the copies to overlap; rows may have any
    stride.  streams: (compute, copy_in, copy_out) torch streams, default
    three new ones on the current device; workspace: a CUDA uint8 tensor of
    at least tgemm_sgemm_host_workspace_size bytes (allocated if omitted).
    Blocks until C is complete."""
    import torch

    for t, name in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2 or t.is_cuda:
            raise TypeError(f"{name} must be a 2-D float32 CPU tensor")
        if t.stride(1) != 1 and t.shape[1] > 1 and t.numel() > 0:
            raise ValueError(f"{name} must be row-major")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, pin_memory=A.is_pinned())
    elif out.is_cuda or tuple(out.shape) != (M, N) or (out.stride(1) != 1 and N > 1 and out.numel() > 0):
        raise ValueError(f"out must be a row-major {M}x{N} CPU tensor")
    need = tgemm_sgemm_host_workspace_size(M, N, K, panel_rows)
    if need < 0:
        raise ValueError("invalid sizes or panel_rows")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if streams is None:
        streams = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    # the streams start after work already queued on the current stream (e.g. the
    # workspace allocation)
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    st = tgemm_sgemm_host(M, N, K, A.data_ptr(), max(A.stride(0), K, 1), B.data_ptr(), max(B.stride(0), N, 1),
                          out.data_ptr(), max(out.stride(0), N, 1), workspace.data_ptr(), workspace.numel(),
                          panel_rows, *(s.cuda_stream for s in streams))
    if st != TGEMM_SUCCESS:
        raise TgemmError(st, "tgemm_sgemm_host")
    return out


def variant_names():
    """Names of the matrix-core tile configurations, by index."""
    return [tgemm_mfma_variant_name(i) for i in range(tgemm_mfma_variant_count())]
