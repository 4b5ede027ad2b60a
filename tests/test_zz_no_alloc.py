"""The allocation-free split-K entry point against the workspace one (GPU).

tgemm_sgemm_splitk_noalloc runs the same kernels and slices as
tgemm_sgemm_splitk_ex with the partial products in the library's fixed
per-GPU scratch, so on the same inputs the two must agree bit for bit; with
integer inputs both must also equal the oracle's exact int64 product.  Two
calls in a row, the second smaller, so that the second runs over what the
first left in the scratch.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_tgemm_amd as tg
from tiled_gemm_tgemm_amd import workloads as wl

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def stored(X, transposed):
    dev = torch.device("cuda:0")
    if transposed:
        return torch.from_numpy(np.ascontiguousarray(X.T)).to(dev)
    return torch.from_numpy(X).to(dev)


def run_pair(M, N, K, splits, ta, tb, seed, dist):
    A, B, _ = wl.random_matrices(M, N, K, dist, seed)
    dA, dB = stored(A, ta), stored(B, tb)
    lda = M if ta else K
    ldb = K if tb else N
    op_a = tg.TGEMM_OP_T if ta else tg.TGEMM_OP_N
    op_b = tg.TGEMM_OP_T if tb else tg.TGEMM_OP_N
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, splits)
    assert 0 < need <= tg.TGEMM_SPLITK_NOALLOC_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    C_ws = torch.full((M, N), float("nan"), device="cuda")
    C_na = torch.full((M, N), float("nan"), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    log(f"noalloc {M}x{N}x{K} splits={splits} ta={ta} tb={tb} {dist}")
    st = tg.tgemm_sgemm_splitk_ex(op_a, op_b, M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb, C_ws.data_ptr(), N,
                                  splits, ws.data_ptr(), need, stream)
    assert st == tg.TGEMM_SUCCESS
    st = tg.tgemm_sgemm_splitk_noalloc(op_a, op_b, M, N, K, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                                       C_na.data_ptr(), N, splits, stream)
    assert st == tg.TGEMM_SUCCESS
    torch.cuda.synchronize()
    a = C_ws.cpu().numpy()
    b = C_na.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "noalloc differs from the workspace entry point"
    return A, B, b


def test_noalloc_equals_workspace_entry_point_two_calls():
    # first call: 16 slices of 512×512 floats (16 MiB of the 32 MiB scratch)
    A, B, C = run_pair(512, 512, 16384, 16, False, False, 3, "int4")
    assert np.array_equal(C.astype(np.int64), oracle.gemm_i64(A, B))
    # second call, smaller and with A stored transposed, over the first call's leftovers
    A, B, C = run_pair(200, 136, 4100, 4, True, False, 4, "int4")
    assert np.array_equal(C.astype(np.int64), oracle.gemm_i64(A, B))


def test_noalloc_real_inputs_within_bound():
    M, N, K = 256, 320, 8192
    A, B, C = run_pair(M, N, K, 8, False, True, 5, "uniform")
    P, S = oracle.gemm(A, B)
    assert np.all(np.abs(C.astype(np.float64) - P) <= 4.0 * K * 2.0 ** -24 * S)


def test_noalloc_refuses_beyond_scratch_and_leaves_c():
    M, N, K = 2048, 2048, 1024
    dA = torch.zeros((M, K), device="cuda")
    dB = torch.zeros((K, N), device="cuda")
    C = torch.full((M, N), 7.0, device="cuda")
    st = tg.tgemm_sgemm_splitk_noalloc(tg.TGEMM_OP_N, tg.TGEMM_OP_N, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                                       C.data_ptr(), N, 4, torch.cuda.current_stream().cuda_stream)
    assert st == tg.TGEMM_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert bool(torch.all(C == 7.0))
