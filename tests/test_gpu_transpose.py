"""GPU parity of tgemm_transpose against the oracle's transpose (page 2,
"Lec 29 · GPU Architecture (2)", §1.4).

A transpose moves words, so the bar is bit-exactness: outputs are compared
as uint32 words, on inputs that include NaNs with payloads, signed zeros,
infinities and subnormals.  Every kernel runs on every case; guard bands
(NaN around A, sentinels around B) catch reads and writes outside the
operands.  All calls go through the C ABI (ctypes, via tiled_gemm_tgemm_amd).
"""

import sys

import numpy as np
import pytest

import oracle
import tiled_gemm_tgemm_amd as tg
from tiled_gemm_tgemm_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KERNELS = ["blocked", "naive", "tiled", "tiled_padded"]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    tg.library()
    yield


def words(x):
    return np.ascontiguousarray(x).view(np.uint32)


def odd_words(M, N, seed):
    """M×N float32 with arbitrary bit patterns, specials first."""
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 2 ** 32, size=(M, N), dtype=np.uint64).astype(np.uint32)
    special = np.array([0x7FC01234, 0xFFA00001, 0x80000000, 0x00000000, 0x7F800000, 0xFF800000,
                        0x00000001, 0x807FFFFF, 0x7FBFFFFF], np.uint32)
    flat = w.reshape(-1)
    flat[: min(flat.size, special.size)] = special[: flat.size]
    return w.view(np.float32)


def gpu_transpose(A, kernel):
    B = tg.transpose(torch.from_numpy(np.ascontiguousarray(A)).cuda(), kernel=kernel)
    torch.cuda.synchronize()
    return B.cpu().numpy()


SHAPES = [(1, 1), (1, 2), (2, 1), (1, 100), (100, 1), (3, 5), (31, 33), (32, 32), (33, 31),
          (63, 65), (64, 64), (65, 64), (64, 65), (127, 129), (128, 128), (200, 3), (3, 200),
          (256, 260), (260, 256), (1000, 999),
          # at least 2^24 elements: the blocked kernel's 64×256 tiles, ragged and whole
          (4099, 4097), (4096, 4352)]


@pytest.mark.parametrize("M,N", SHAPES)
def test_shapes_bit_exact(M, N):
    A = odd_words(M, N, 7 * M + N)
    want = words(oracle.transpose(A))
    for kernel in KERNELS:
        log(f"transpose {M}x{N} {kernel}")
        got = gpu_transpose(A, kernel)
        assert got.shape == (N, M)
        assert np.array_equal(words(got), want), kernel


@pytest.mark.parametrize("name", ["transpose1024_uniform", "transpose3001x5003_uniform"])
def test_workloads_bit_exact(name):
    w = wl.TRANSPOSE_WORKLOADS[name]
    A = wl.make_transpose_input(w)
    want = words(oracle.transpose(A))
    for kernel in KERNELS:
        log(f"{name} {kernel}")
        assert np.array_equal(words(gpu_transpose(A, kernel)), want), kernel


def test_largest_workload_bit_exact():
    """The 16384×16384 workload (1 GiB each way), every kernel, whole output."""
    w = wl.TRANSPOSE_WORKLOADS["transpose16384_uniform"]
    A = wl.make_transpose_input(w)
    want = words(oracle.transpose(A))
    dA = torch.from_numpy(A).cuda()
    B = torch.empty((w.N, w.M), dtype=torch.float32, device="cuda")
    for kernel in KERNELS:
        log(f"{w.name} {kernel}")
        B.fill_(float("nan"))
        tg.transpose(dA, out=B, kernel=kernel)
        torch.cuda.synchronize()
        assert np.array_equal(words(B.cpu().numpy()), want), kernel
    del dA, B
    torch.cuda.empty_cache()


def guarded(x, rows_extra, cols_extra, fill):
    r, c = x.shape
    big = torch.full((r + rows_extra, c + cols_extra), fill, dtype=torch.float32, device="cuda")
    big[:r, :c] = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return big, big[:r, :c]


@pytest.mark.parametrize("M,N,pad_a,pad_b", [(65, 33, 3, 5), (64, 64, 4, 4), (130, 68, 8, 4),
                                             (1, 1, 1, 3), (257, 129, 0, 7), (100, 300, 4, 0),
                                             (4100, 4104, 4, 4), (4097, 4100, 3, 1)])
def test_guard_bands(M, N, pad_a, pad_b):
    """A inside NaN (wider rows, extra rows), B inside sentinels: a NaN in B
    means a read outside A, a changed sentinel a write outside B.  Covers the
    16-byte path (paddings that keep leading dimensions multiples of 4) and
    the single-word path (the others)."""
    A = (np.arange(M)[:, None] * N + np.arange(N)[None, :]).astype(np.float32)
    for kernel in KERNELS:
        log(f"guard {M}x{N} pads {pad_a},{pad_b} {kernel}")
        _, Av = guarded(A, 3, pad_a, float("nan"))
        Bbig, Bv = guarded(np.zeros((N, M), np.float32), 2, pad_b, 12345.0)
        tg.transpose(Av, out=Bv, kernel=kernel)
        torch.cuda.synchronize()
        big = Bbig.cpu().numpy()
        assert np.array_equal(big[:N, :M], A.T), kernel
        outside = np.ones(big.shape, bool)
        outside[:N, :M] = False
        assert np.all(big[outside] == 12345.0), f"{kernel} wrote outside B"


def test_unaligned_operands_take_the_word_path():
    """A and B one element past a 16-byte boundary: still exact."""
    M, N = 192, 256
    A = odd_words(M, N, 3)
    want = words(oracle.transpose(A))
    Abuf = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    Bbuf = torch.full((N * M + 1,), float("nan"), dtype=torch.float32, device="cuda")
    Av = Abuf[1:].view(M, N)
    Av.copy_(torch.from_numpy(A).cuda())
    Bv = Bbuf[1:].view(N, M)
    for kernel in KERNELS:
        st = tg.tgemm_transpose(M, N, Av.data_ptr(), N, Bv.data_ptr(), M, tg.TRANSPOSE_KERNELS[kernel], None)
        assert st == tg.TGEMM_SUCCESS
        torch.cuda.synchronize()
        assert np.array_equal(words(Bv.cpu().numpy()), want), kernel


def test_empty_is_noop_and_errors_leave_b_untouched():
    B = torch.full((4, 3), 7.0, device="cuda")
    for kernel in KERNELS:
        tg.transpose(torch.empty((0, 4), device="cuda"), out=torch.empty((4, 0), device="cuda"), kernel=kernel)
        A = torch.ones((3, 4), device="cuda")
        # B overlapping A is refused before anything runs
        st = tg.tgemm_transpose(3, 4, A.data_ptr(), 4, A.data_ptr() + 8, 3, tg.TRANSPOSE_KERNELS[kernel], None)
        assert st == tg.TGEMM_ERROR_INVALID_VALUE
        st = tg.tgemm_transpose(3, 4, A.data_ptr(), 3, B.data_ptr(), 3, tg.TRANSPOSE_KERNELS[kernel], None)
        assert st == tg.TGEMM_ERROR_INVALID_VALUE  # lda < N
    torch.cuda.synchronize()
    assert torch.all(B == 7.0)


def test_non_default_stream_and_graph_replay():
    M, N = 300, 500
    A = odd_words(M, N, 11)
    want = words(oracle.transpose(A))
    dA = torch.from_numpy(A).cuda()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B = tg.transpose(dA)
    s.synchronize()
    assert np.array_equal(words(B.cpu().numpy()), want)
    B.fill_(0.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tg.transpose(dA, out=B)
    for rep in range(3):
        B.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(words(B.cpu().numpy()), want), f"replay {rep}"
