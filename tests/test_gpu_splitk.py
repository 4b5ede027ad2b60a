"""GPU parity of tgemm_sgemm_splitk (K split across work-groups, partial
products summed in slice order by a second pass) against the CPU oracle.

Acceptance as for the other products: integer-valued inputs whose partial
sums stay below 2^24 give the exact integer product element for element
(every float32 partial sum, the slices' and their total, is exact); real
inputs stay within |C_ij − P_ij| <= 4·K·2^-24·S_ij.  Also: results do not
depend on timing (repeated calls are bitwise equal), C's padding columns and
the rest of a larger workspace are never touched where they must not be, and
a rejected call leaves C as it was.
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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def splitk(A, B, splits=None, **kw):
    C = tg.sgemm_splitk(dev(A), dev(B), splits=splits, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def assert_exact(C, P_int, what):
    got, want = C.astype(np.float64), P_int.astype(np.float64)
    if not np.array_equal(got, want):
        i, j = np.argwhere(got != want)[0]
        pytest.fail(f"{what}: first difference at ({i},{j}): {got[i, j]} vs {want[i, j]}")


def assert_within_bound(C, P, S, K, what):
    C = C.astype(np.float64)
    assert np.all(np.isfinite(C)), what
    bad = np.abs(C - P) > 4.0 * K * TWO_M24 * S
    if bad.any():
        i, j = np.argwhere(bad)[0]
        pytest.fail(f"{what}: {bad.sum()} outside the bound; first ({i},{j}) C={C[i, j]!r} P={P[i, j]!r}")


# shapes: few tiles with long K, ragged edges, K shorter than the slices
# asked for (fewer slices run), one element, and K not a multiple of 4
# (4-byte loads)
INT_CASES = [(64, 64, 4096, 4), (100, 60, 1000, 8), (33, 65, 17, 4), (1, 1, 1, 2), (300, 7, 513, 3),
             (512, 512, 4096, 16), (96, 96, 2048, 64), (130, 68, 36, 5), (257, 129, 1001, 2)]


@pytest.mark.parametrize("M,N,K,splits", INT_CASES)
def test_splitk_integer_exact(M, N, K, splits):
    log(f"splitk int {M}x{N}x{K} splits={splits}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 11)
    C = splitk(A, B, splits)
    assert_exact(C, oracle.gemm_i64(A, B), f"{M}x{N}x{K}/{splits}")


def test_splitk_chosen_split_integer_exact():
    for (M, N, K) in [(256, 256, 16384), (2048, 256, 8192), (384, 640, 4096)]:
        s = tg.tgemm_sgemm_splitk_choose(M, N, K)
        log(f"splitk int {M}x{N}x{K} chosen splits={s}")
        assert s > 1, (M, N, K, s)
        A, B, _ = wl.random_matrices(M, N, K, "int4", 12)
        C = splitk(A, B)
        assert_exact(C, oracle.gemm_i64(A, B), f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,splits", [(384, 640, 4096, None), (200, 300, 1000, 8), (64, 64, 8192, 64)])
def test_splitk_real_within_bound_and_deterministic(M, N, K, splits):
    log(f"splitk real {M}x{N}x{K} splits={splits}")
    A, B, _ = wl.random_matrices(M, N, K, "uniform", 13)
    C1 = splitk(A, B, splits)
    C2 = splitk(A, B, splits)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "repeated calls differ"
    P, S = oracle.gemm(A, B)
    assert_within_bound(C1, P, S, K, f"{M}x{N}x{K}")


def test_splitk_padding_and_workspace_tail_untouched():
    M, N, K, splits, pad = 65, 33, 3000, 8, 7
    log(f"splitk guard bands {M}x{N}x{K}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 14)
    C_full = torch.full((M, N + pad), float("nan"), device="cuda")
    out = C_full[:, :N]
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, splits)
    ws = torch.full((need + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    tg.sgemm_splitk(dev(A), dev(B), out=out, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    got = C_full.cpu().numpy()
    assert_exact(got[:, :N], oracle.gemm_i64(A, B), "inside")
    assert np.isnan(got[:, N:]).all(), "padding columns of C were written"
    assert (ws[need:].cpu().numpy() == 0xAB).all(), "bytes past the workspace size were written"


def test_splitk_misaligned_operand_takes_4_byte_loads():
    M, N, K = 96, 80, 2048
    log(f"splitk misaligned {M}x{N}x{K}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 15)
    A_big = torch.zeros(M * K + 1, device="cuda")
    A_big[1:] = dev(A).reshape(-1)
    A_view = A_big[1:].view(M, K)  # 4 bytes past a 16-byte boundary
    C = tg.sgemm_splitk(A_view, dev(B), splits=8)
    torch.cuda.synchronize()
    assert_exact(C.cpu().numpy(), oracle.gemm_i64(A, B), "misaligned A")


def test_splitk_zero_k_and_empty():
    A = torch.empty(5, 0, device="cuda")
    B = torch.empty(0, 7, device="cuda")
    C = torch.full((5, 7), float("nan"), device="cuda")
    tg.sgemm_splitk(A, B, out=C, splits=4)
    torch.cuda.synchronize()
    z = C.cpu().numpy()
    assert (z == 0).all() and not np.signbit(z).any()
    tg.sgemm_splitk(torch.empty(0, 3, device="cuda"), torch.empty(3, 4, device="cuda"), splits=4)


def test_splitk_errors_leave_c_untouched():
    M, N, K = 64, 64, 4096
    A = torch.ones(M, K, device="cuda")
    B = torch.ones(K, N, device="cuda")
    C = torch.full((M, N), 7.0, device="cuda")
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, 4)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    for bad in [dict(splits=4, workspace=small), dict(splits=0), dict(splits=65)]:
        with pytest.raises(tg.TgemmError):
            tg.sgemm_splitk(A, B, out=C, **bad)
    torch.cuda.synchronize()
    assert (C.cpu().numpy() == 7.0).all()


def test_splitk_sampled_at_size():
    """512×512×16384, in the configuration the library chooses, checked on
    sampled 64×64 blocks and full row/column checksums."""
    M, N, K = 512, 512, 16384
    log(f"splitk sampled {M}x{N}x{K}")
    A, B, _ = wl.random_matrices(M, N, K, "uniform", 16)
    C = splitk(A, B).astype(np.float64)
    rng = np.random.default_rng(16)
    origins = [(int(r) * 64, int(c) * 64) for r, c in rng.integers(0, 8, size=(6, 2))]
    for (r, c), (P, S) in zip(origins, oracle.gemm_blocks(A, B, origins, 64)):
        assert_within_bound(C[r:r + 64, c:c + 64], P, S, K, f"block ({r},{c})")
    row, rowabs, col, colabs = oracle.checksums(A, B)
    assert np.all(np.abs(C.sum(axis=1) - row) <= 4.0 * K * TWO_M24 * rowabs + 1e-9 * rowabs + N * 1e-12)
    assert np.all(np.abs(C.sum(axis=0) - col) <= 4.0 * K * TWO_M24 * colabs + 1e-9 * colabs + M * 1e-12)


def test_splitk_graph_capture_replays():
    """Both launches of a split-K call (slices, then the sum) captured into a
    HIP graph replay correctly, many times, with the workspace and C dirtied
    and eager work between replays."""
    cases = [(96, 96, 2048, 8), (256, 256, 8192, 16)]
    ins = []
    for i, (M, N, K, s) in enumerate(cases):
        A, B, _ = wl.random_matrices(M, N, K, "int4", 20 + i)
        ws = torch.empty(tg.tgemm_sgemm_splitk_workspace_size(M, N, K, s), dtype=torch.uint8, device="cuda")
        ins.append((dev(A), dev(B), torch.empty((M, N), device="cuda"), ws, s, oracle.gemm_i64(A, B)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the capture
        for dA, dB, dC, ws, s, _ in ins:
            tg.sgemm_splitk(dA, dB, out=dC, splits=s, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dA, dB, dC, ws, s, _ in ins:
            tg.sgemm_splitk(dA, dB, out=dC, splits=s, workspace=ws)
    for rep in range(5):
        for _, _, dC, ws, _, _ in ins:
            dC.fill_(float("nan"))
            ws.fill_(0xFF)  # NaN patterns in every partial block
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, dC, _, s, Pi) in ins:
            C = dC.cpu().numpy()
            if not np.array_equal(C.astype(np.float64), Pi.astype(np.float64)):
                pytest.fail(f"replay {rep}, splits {s}: result differs from the exact product")
        x = torch.randn(1024, 1024, device="cuda")
        _ = (x @ x).sum().item()


def test_splitk_two_streams_two_workspaces():
    """Two split-K products in flight at once on two streams, each with its
    own workspace, give the same results as alone."""
    M, N, K = 256, 256, 16384
    (A1, B1, _), (A2, B2, _) = (wl.random_matrices(M, N, K, "int4", 30 + i) for i in range(2))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    d = [(dev(A1), dev(B1)), (dev(A2), dev(B2))]
    outs = [torch.empty((M, N), device="cuda") for _ in range(2)]
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, 16)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for (dA, dB), out, ws, st in zip(d, outs, wss, (s1, s2)):
            tg.sgemm_splitk(dA, dB, out=out, splits=16, workspace=ws, stream=st.cuda_stream)
        torch.cuda.synchronize()
        assert_exact(outs[0].cpu().numpy(), oracle.gemm_i64(A1, B1), f"stream 1, rep {rep}")
        assert_exact(outs[1].cpu().numpy(), oracle.gemm_i64(A2, B2), f"stream 2, rep {rep}")


def test_splitk_side_stream_internal_workspace_not_reused_early():
    """sgemm_splitk on a side stream with no workspace given: the workspace
    it allocates is released when it returns, while the side stream may
    still be using it.  Allocations of the same size on the current stream
    right after, each written at once, must not be handed that memory before
    the side stream's work ends (the binding records the side stream on the
    tensors it allocates); otherwise they overwrite partial products."""
    M, N, K = 512, 512, 16384
    A, B, _ = wl.random_matrices(M, N, K, "int4", 50)
    dA, dB = dev(A), dev(B)
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, 16)
    side = torch.cuda.Stream()
    X = torch.rand(4096, 4096, device="cuda")
    Y = torch.empty_like(X)
    torch.cuda.synchronize()
    for rep in range(3):
        log(f"splitk side stream, internal workspace, rep {rep}")
        # queue a few milliseconds of other work first, so that the split-K
        # kernels are still pending when this thread returns and reallocates
        for _ in range(3):
            tg.sgemm(X, X, out=Y, stream=side.cuda_stream)
        C = tg.sgemm_splitk(dA, dB, splits=16, stream=side.cuda_stream)
        junk = []
        for _ in range(24):
            t = torch.empty(need, dtype=torch.uint8, device="cuda")
            t.fill_(0xFF)  # NaN bit patterns, on the current stream
            junk.append(t)
            del junk[0:len(junk) - 2]
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), oracle.gemm_i64(A, B), f"side stream rep {rep}")
        del C, junk


@pytest.mark.parametrize("ta,tb", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("M,N,K,splits", [(96, 80, 2048, 8), (65, 33, 3000, 4), (256, 256, 16384, None)])
def test_splitk_transposed_operands_integer_exact(ta, tb, M, N, K, splits):
    log(f"splitk transposed ta={ta} tb={tb} {M}x{N}x{K} splits={splits}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 40)
    dA = dev(A.T).t() if ta else dev(A)
    dB = dev(B.T).t() if tb else dev(B)
    C = tg.sgemm_splitk(dA, dB, splits=splits)
    torch.cuda.synchronize()
    assert_exact(C.cpu().numpy(), oracle.gemm_i64(A, B), f"ta={ta} tb={tb} {M}x{N}x{K}")
