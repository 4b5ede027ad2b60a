"""GPU parity of tgemm_sgemm_host — the product of host-memory operands with
the transfers overlapped with the computation (page 1, section [CUDA
Performance Considerations], "Overlap I/O with Computation") — against the
oracle, through the C ABI.

Integer inputs must give the exact product; real inputs must lie within the
same bound as the device entry point, and, since each panel is an ordinary
tgemm_sgemm call, equal bit for bit what tgemm_sgemm gives for the same
rows when it runs the same configuration.
"""

import sys

import numpy as np
import pytest

import oracle
import tiled_gemm_tgemm_amd as tg
from tiled_gemm_tgemm_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TWO_M24 = 2.0 ** -24


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    tg.library()
    yield


def pinned(x):
    return torch.from_numpy(np.ascontiguousarray(x)).pin_memory()


def int_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    return (rng.integers(-4, 5, (M, K)).astype(np.float32), rng.integers(-4, 5, (K, N)).astype(np.float32))


@pytest.mark.parametrize("M,N,K,panel", [(1, 1, 1, 0), (300, 200, 100, 0), (300, 200, 100, 64),
                                         (1000, 513, 257, 256), (1031, 260, 64, 100), (513, 1, 9, 7),
                                         (2048, 2048, 512, 0)])
def test_integer_exact(M, N, K, panel):
    A, B = int_inputs(M, N, K, M + 3 * N + 7 * K + panel)
    Pi = oracle.gemm_i64(A, B)
    log(f"host {M}x{N}x{K} panel {panel}")
    C = tg.sgemm_host(pinned(A), pinned(B), panel_rows=panel).numpy()
    assert np.array_equal(C.astype(np.int64), Pi)


def test_real_workload_within_bound_and_equal_to_device_path():
    w = wl.WORKLOADS["rect3000x1000x5000_normal"]
    A, B = wl.make_inputs(w)
    P, S = oracle.gemm(A, B)
    log(f"host {w.name}")
    C = tg.sgemm_host(pinned(A), pinned(B), panel_rows=768).numpy()
    assert np.all(np.abs(C.astype(np.float64) - P) <= 4 * w.K * TWO_M24 * S)
    # each 768-row panel through the device entry point directly
    dB = torch.from_numpy(B).cuda()
    for r0 in range(0, w.M, 768):
        dA = torch.from_numpy(A[r0:r0 + 768]).cuda()
        Cd = tg.sgemm(dA, dB)
        torch.cuda.synchronize()
        assert np.array_equal(Cd.cpu().numpy(), C[r0:r0 + 768]), f"panel at row {r0}"


def test_strided_host_operands_and_output():
    """A and B with wider rows than K and N, C written into a wider buffer:
    the padding is never read into the product and never written."""
    M, N, K = 700, 333, 129
    A, B = int_inputs(M, N, K, 5)
    Pi = oracle.gemm_i64(A, B)
    Abig = np.full((M, K + 5), np.nan, np.float32)
    Abig[:, :K] = A
    Bbig = np.full((K, N + 3), np.nan, np.float32)
    Bbig[:, :N] = B
    Cbig = pinned(np.full((M, N + 6), 12345.0, np.float32))
    tA, tB = pinned(Abig), pinned(Bbig)
    tg.sgemm_host(tA[:, :K], tB[:, :N], out=Cbig[:, :N], panel_rows=128)
    c = Cbig.numpy()
    assert np.array_equal(c[:, :N].astype(np.int64), Pi)
    assert np.all(c[:, N:] == 12345.0)


def test_one_stream_and_pageable_memory():
    """All three streams the same (serial), and pageable host memory: same result."""
    M, N, K = 520, 300, 200
    A, B = int_inputs(M, N, K, 9)
    Pi = oracle.gemm_i64(A, B)
    s = torch.cuda.Stream()
    C = tg.sgemm_host(pinned(A), pinned(B), panel_rows=128, streams=(s, s, s)).numpy()
    assert np.array_equal(C.astype(np.int64), Pi)
    C2 = tg.sgemm_host(torch.from_numpy(A), torch.from_numpy(B), panel_rows=200).numpy()
    assert np.array_equal(C2.astype(np.int64), Pi)


def test_empty_and_errors():
    C = tg.sgemm_host(pinned(np.zeros((6, 0), np.float32)), pinned(np.zeros((0, 5), np.float32))).numpy()
    assert C.shape == (6, 5) and np.all(C == 0) and not np.any(np.signbit(C))
    A, B = int_inputs(64, 64, 64, 1)
    tA, tB = pinned(A), pinned(B)
    Cout = pinned(np.full((64, 64), 7.0, np.float32))
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    st = tg.tgemm_sgemm_host(64, 64, 64, tA.data_ptr(), 64, tB.data_ptr(), 64, Cout.data_ptr(), 64,
                             small.data_ptr(), small.numel(), 0, None, None, None)
    assert st == tg.TGEMM_ERROR_INVALID_VALUE
    assert np.all(Cout.numpy() == 7.0)
