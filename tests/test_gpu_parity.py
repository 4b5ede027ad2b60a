"""GPU parity: every kernel through the C ABI against the CPU oracle.

Acceptance (the product's definition gives no tolerance, so it is derived
from the arithmetic):
* integer-valued inputs whose partial sums stay below 2^24: every float32
  partial sum is exact in any order, so the result must equal the exact
  integer product element for element;
* real inputs: |C_ij − P_ij| <= 4·K·2^-24·S_ij with S_ij = sum_k |A_ik·B_kj|,
  compared in float64 (4× the classical bound for recursive float32
  summation, leaving room for any order and the matrix cores' internal
  rounding);
* the two one-product-per-step ablation kernels must also equal, bit for
  bit, the oracle's float32 sequential fused-multiply-add model.

Workloads are the seeded synthetic ones of tiled_gemm_tgemm_amd.workloads;
the two largest are checked on sampled 64×64 blocks plus full row and column
checksums (4096² also in full), in the launch configuration the benchmark
times (tgemm_sgemm on contiguous operands).
"""

import itertools
import json
import os
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
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    tg.library()  # raises if libtgemm.so is missing
    yield


VARIANTS = None


def variants():
    global VARIANTS
    if VARIANTS is None:
        VARIANTS = tg.variant_names()
    return VARIANTS


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(A, B, kernel="auto", **kw):
    C = tg.sgemm(dev(A), dev(B), kernel=kernel, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


# How much of the acceptance bound real-valued results use: a drift in the
# kernels' accumulation order or rounding shows here long before it could
# break the bound itself.  Above CANARY (a quarter of the worst case of
# recursive float32 summation, K·2^-24·S) a test fails: the kernels measure
# below 0.01 on every workload.
CANARY = 0.25


def error_stats(C, P, S, K):
    """max and RMS over the elements of |C - P| / (K·2^-24·S); where S is
    zero the element must be exactly zero (checked by the caller's bound)."""
    err = np.abs(C.astype(np.float64) - P)
    scale = K * TWO_M24 * S
    pos = scale > 0
    r = err[pos] / scale[pos]
    if not r.size:
        return 0.0, 0.0
    return float(r.max()), float(np.sqrt(np.mean(r * r)))


def record_error(what, K, mx, rms):
    line = f"error ratio {what} (K={K}): max {mx:.5f} rms {rms:.6f} of K·2^-24·S"
    log(line)
    path = os.environ.get("TGEMM_ERROR_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"what": what, "K": K, "max_ratio": mx, "rms_ratio": rms}) + "\n")


def assert_within_bound(C, P, S, K, what="", record=True):
    C = C.astype(np.float64)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    err = np.abs(C - P)
    bound = 4.0 * K * TWO_M24 * S
    bad = err > bound
    if bad.any():
        i, j = np.argwhere(bad)[0]
        pytest.fail(f"{what}: {bad.sum()} elements outside the bound; first ({i},{j}): "
                    f"C={C[i, j]!r} P={P[i, j]!r} bound={bound[i, j]!r}")
    mx, rms = error_stats(C, P, S, K)
    if record:
        record_error(what, K, mx, rms)
    assert mx <= CANARY, f"{what}: max error ratio {mx} above the canary {CANARY}"
    return mx


def assert_exact(C, P_int, what=""):
    got = C.astype(np.float64)
    want = P_int.astype(np.float64)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i, j = bad[0]
        pytest.fail(f"{what}: {len(bad)} elements differ; first ({i},{j}) {got[i, j]} vs {want[i, j]}")


def int_inputs(M, N, K, seed):
    A, B, _ = wl.random_matrices(M, N, K, "int4", seed)
    return A, B


def vec4_shape(M, N, K):
    return K % 4 == 0 and N % 4 == 0


def runnable(name, M, N, K, ta=False, tb=False):
    """Whether variant `name` takes contiguous aligned operands of these
    shapes and orders (ta: A stored K×M, tb: B stored N×K)."""
    if (ta or tb) and (name.endswith("_flat") or name.endswith("_nn")):
        return False
    if "vec4" not in name:
        return True
    return (M if ta else K) % 4 == 0 and (K if tb else N) % 4 == 0


def auto_variant(M, N, K):
    """Name of the variant tgemm_sgemm picks for contiguous, aligned operands."""
    v = tg.tgemm_sgemm_variant_for(M, N, K, 1 << 20, K, 1 << 36, N, 1 << 44, N)
    return variants()[v] if v >= 0 else None


# ------------------------------------------------------------ the workloads

def test_square512_uniform_all_kernels():
    w = wl.WORKLOADS["square512_uniform"]
    A, B = wl.make_inputs(w)
    P, S = oracle.gemm(A, B)
    fma = oracle.gemm_fma_f32(A, B)
    log(f"{w.name}: auto")
    assert_within_bound(run(A, B), P, S, w.K, f"{w.name} auto")
    for v, name in enumerate(variants()):
        log(f"{w.name}: {name}")
        assert_within_bound(run(A, B, "mfma", variant=v), P, S, w.K, f"{w.name} {name}")
    log(f"{w.name}: naive")
    C = run(A, B, "naive")
    assert np.array_equal(C, fma), "naive differs from the sequential fma model"
    for tile, pad in itertools.product((8, 16, 32), (0, 1)):
        log(f"{w.name}: lds tile={tile} pad={pad}")
        C = run(A, B, "lds", tile=tile, pad=pad)
        assert np.array_equal(C, fma), f"lds{tile} pad{pad} differs from the fma model"
    log(f"{w.name}: simt")
    assert np.array_equal(run(A, B, "simt"), fma), "simt differs from the sequential fma model"


def test_square1024_int4_bit_exact():
    w = wl.WORKLOADS["square1024_int4"]
    A, B = wl.make_inputs(w)
    Pi = oracle.gemm_i64(A, B)
    P, _ = oracle.gemm(A, B, with_abs=False)
    assert np.array_equal(P, Pi.astype(np.float64))  # the two oracle paths agree
    log(f"{w.name}: auto")
    assert_exact(run(A, B), Pi, "auto")
    for v, name in enumerate(variants()):
        log(f"{w.name}: {name}")
        assert_exact(run(A, B, "mfma", variant=v), Pi, name)
    log(f"{w.name}: naive / lds")
    assert_exact(run(A, B, "naive"), Pi, "naive")
    assert_exact(run(A, B, "lds", tile=16, pad=1), Pi, "lds16")
    assert_exact(run(A, B, "lds", tile=32, pad=0), Pi, "lds32")
    assert_exact(run(A, B, "simt"), Pi, "simt")


# the pages' kernels and the vector-ALU one: (kernel, sgemm arguments)
ABLATIONS = [("naive", {}), ("lds", dict(tile=16, pad=1)), ("lds", dict(tile=32, pad=0)), ("simt", {})]


def test_rect3000x1000x5000_normal_masked_edges():
    w = wl.WORKLOADS["rect3000x1000x5000_normal"]
    A, B = wl.make_inputs(w)
    log(f"{w.name}: oracle")
    P, S = oracle.gemm(A, B)
    log(f"{w.name}: auto ({auto_variant(w.M, w.N, w.K)})")
    assert_within_bound(run(A, B), P, S, w.K, f"{w.name} auto")
    for v, name in enumerate(variants()):
        log(f"{w.name}: {name}")
        assert_within_bound(run(A, B, "mfma", variant=v), P, S, w.K, f"{w.name} {name}")
    # C's rows one word off 16-byte alignment: the automatic choice leaves the
    # 160×128 tile (whose epilogue writes 16-byte row pieces), and that tile
    # run explicitly stores element by element, with the same bits as its
    # aligned run
    row_store = "m160n128k32_w1x4_vec4_nn"
    big = torch.full((w.M, w.N + 1), float("nan"), dtype=torch.float32, device="cuda")
    Cv = big[:, 1:]
    Ad, Bd = dev(A), dev(B)
    chosen = tg.tgemm_sgemm_variant_for(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N,
                                        Cv.data_ptr(), w.N + 1)
    log(f"{w.name}: auto into unaligned C ({variants()[chosen]})")
    assert variants()[chosen] != row_store
    tg.sgemm(Ad, Bd, out=Cv)
    torch.cuda.synchronize()
    assert_within_bound(Cv.cpu().numpy(), P, S, w.K, f"{w.name} auto, unaligned C", record=False)
    log(f"{w.name}: {row_store} into unaligned C")
    tg.sgemm(Ad, Bd, out=Cv, kernel="mfma", variant=variants().index(row_store))
    torch.cuda.synchronize()
    assert np.array_equal(Cv.cpu().numpy(), run(A, B, "mfma", variant=variants().index(row_store))), \
        f"{row_store}: unaligned C differs from aligned C"
    del big, Cv, Ad, Bd
    # the ablation kernels through the full ragged shape (no dimension a
    # multiple of any of their tiles): within the bound everywhere, and bit
    # for bit the oracle's sequential float32 FMA model on the first rows and
    # on the rows of the last, partial tile row
    rows = np.r_[0:32, w.M - 40:w.M]
    fma_rows = oracle.gemm_fma_f32(np.ascontiguousarray(A[rows]), B)
    for kernel, kw in ABLATIONS:
        name = kernel + "".join(f"{k}{v}" for k, v in kw.items())
        log(f"{w.name}: {name}")
        C = run(A, B, kernel, **kw)
        assert_within_bound(C, P, S, w.K, f"{w.name} {name}")
        assert np.array_equal(C[rows], fma_rows), f"{name} differs from the fma model on the sampled rows"


def check_sampled(C, A, B, blocks, K, what, oracle_blocks=None):
    oracle_blocks = oracle_blocks or oracle.gemm_blocks(A, B, blocks, 64)
    for (r, c), (P, S) in zip(blocks, oracle_blocks):
        assert_within_bound(C[r:r + 64, c:c + 64], P, S, K, f"{what} block ({r},{c})", record=False)
    # the blocks' error ratios together
    Cb = np.concatenate([C[r:r + 64, c:c + 64] for r, c in blocks])
    Pb = np.concatenate([P for P, _ in oracle_blocks])
    Sb = np.concatenate([S for _, S in oracle_blocks])
    mx, rms = error_stats(Cb, Pb, Sb, K)
    record_error(f"{what} ({len(blocks)} blocks of 64x64)", K, mx, rms)
    row, rowabs, col, colabs = oracle.checksums(A, B)
    C64 = C.astype(np.float64)
    M, N = C.shape
    rs, cs = C64.sum(axis=1), C64.sum(axis=0)
    # each sum of C inherits the per-element bound; float64 rounding of the
    # sums themselves adds at most (N+K)·2^-53 of the magnitudes involved
    slack_r = 4 * K * TWO_M24 * rowabs + 2 * (N + K) * 2.0 ** -53 * (rowabs + np.abs(C64).sum(1))
    slack_c = 4 * K * TWO_M24 * colabs + 2 * (M + K) * 2.0 ** -53 * (colabs + np.abs(C64).sum(0))
    assert np.all(np.abs(rs - row) <= slack_r), f"{what}: row checksums"
    assert np.all(np.abs(cs - col) <= slack_c), f"{what}: column checksums"


def test_square4096_uniform_full():
    w = wl.WORKLOADS["square4096_uniform"]
    A, B, blocks = wl.make_inputs_and_blocks(w)
    log(f"{w.name}: auto ({auto_variant(w.M, w.N, w.K)})")
    C = run(A, B)
    check_sampled(C, A, B, blocks, w.K, f"{w.name} auto")
    log(f"{w.name}: full oracle")
    P, S = oracle.gemm(A, B)
    assert_within_bound(C, P, S, w.K, f"{w.name} auto")
    # every configuration against the whole product
    for v, name in enumerate(variants()):
        log(f"{w.name}: {name}")
        assert_within_bound(run(A, B, "mfma", variant=v), P, S, w.K, f"{w.name} {name}")


def test_square8192_uniform_sampled():
    w = wl.WORKLOADS["square8192_uniform"]
    A, B, blocks = wl.make_inputs_and_blocks(w)
    log(f"{w.name}: auto ({auto_variant(w.M, w.N, w.K)})")
    C = run(A, B)
    ob = oracle.gemm_blocks(A, B, blocks, 64)
    check_sampled(C, A, B, blocks, w.K, f"{w.name} auto", ob)
    # every configuration on the same blocks (the checksums once, above)
    for v, name in enumerate(variants()):
        log(f"{w.name}: {name}")
        C = run(A, B, "mfma", variant=v)
        for (r, c), (P, S) in zip(blocks, ob):
            assert_within_bound(C[r:r + 64, c:c + 64], P, S, w.K, f"{w.name} {name} block ({r},{c})",
                                record=False)
        Cb = np.concatenate([C[r:r + 64, c:c + 64] for r, c in blocks])
        mx, rms = error_stats(Cb, np.concatenate([P for P, _ in ob]), np.concatenate([S for _, S in ob]), w.K)
        record_error(f"{w.name} {name} ({len(blocks)} blocks of 64x64)", w.K, mx, rms)


# ------------------------------------------------------------ edges, in integers

EDGE = [1, 2, 3, 7, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def edge_triples(count, seed, mult4=False):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M, N, K = (int(x) for x in rng.choice(EDGE, 3))
        if mult4:
            N, K = (N + 3) // 4 * 4, (K + 3) // 4 * 4
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", edge_triples(24, 11) + [(1, 1, 1), (257, 257, 257), (300, 7, 513)])
def test_edge_shapes_integer_exact(M, N, K):
    A, B = int_inputs(M, N, K, M * 1000003 + N * 1009 + K)
    Pi = oracle.gemm_i64(A, B)
    log(f"edge {M}x{N}x{K}")
    assert_exact(run(A, B), Pi, "auto")
    for v, name in enumerate(variants()):
        if not runnable(name, M, N, K):
            continue
        assert_exact(run(A, B, "mfma", variant=v), Pi, name)
    assert_exact(run(A, B, "naive"), Pi, "naive")
    assert_exact(run(A, B, "simt"), Pi, "simt")
    for tile in (2, 16, 32) if max(M, N) <= 64 else (16, 32):
        assert_exact(run(A, B, "lds", tile=tile, pad=1), Pi, f"lds{tile}")


@pytest.mark.parametrize("M,N,K", edge_triples(16, 12, mult4=True) + [(256, 256, 36), (255, 260, 4)])
def test_edge_shapes_vector_loads_exact(M, N, K):
    A, B = int_inputs(M, N, K, M * 7 + N * 11 + K * 13)
    Pi = oracle.gemm_i64(A, B)
    log(f"edge vec4 {M}x{N}x{K}")
    for v, name in enumerate(variants()):
        assert_exact(run(A, B, "mfma", variant=v), Pi, name)


def guarded(x, rows_extra, cols_extra, fill):
    """x embedded top-left in a larger buffer filled with `fill`; returns (big, view)."""
    r, c = x.shape
    big = torch.full((r + rows_extra, c + cols_extra), fill, dtype=torch.float32, device="cuda")
    big[:r, :c] = dev(x)
    return big, big[:r, :c]


@pytest.mark.parametrize("M,N,K,pad", [(65, 33, 31, 5), (130, 68, 36, 4), (257, 129, 40, 8),
                                       (1, 1, 1, 3), (64, 256, 100, 4)])
def test_guard_bands(M, N, K, pad):
    """NaN around A and B (wider leading dimensions, extra rows) and sentinels
    around C: a NaN in C means something outside A or B was used, a changed
    sentinel means a write outside C."""
    A, B = int_inputs(M, N, K, 5 + M + N + K)
    Pi = oracle.gemm_i64(A, B)
    kernels = [("auto", {})] + [("mfma", {"variant": v}) for v, n in enumerate(variants())
                                if runnable(n, M, N, K) and ("vec1" in n or pad % 4 == 0)]
    kernels += [("naive", {}), ("lds", {"tile": 16, "pad": 1}), ("simt", {})]
    for kernel, kw in kernels:
        log(f"guard {M}x{N}x{K} pad {pad}: {kernel} {kw}")
        _, Av = guarded(A, 3, pad, float("nan"))
        _, Bv = guarded(B, 3, pad, float("nan"))
        Cbig, Cv = guarded(np.zeros((M, N), np.float32), 2, pad, 12345.0)
        tg.sgemm(Av, Bv, out=Cv, kernel=kernel, **kw)
        torch.cuda.synchronize()
        big = Cbig.cpu().numpy()
        assert_exact(big[:M, :N], Pi, f"{kernel} {kw}")
        outside = np.ones(big.shape, bool)
        outside[:M, :N] = False
        assert np.all(big[outside] == 12345.0), f"{kernel} {kw} wrote outside C"


@pytest.mark.parametrize("shift,extra", [(0, 0), (0, 1), (1, 3), (2, 4)])
def test_row_store_epilogue_any_c_alignment(shift, extra):
    """The 160×128 tile forms its blocks transposed and stores C four columns
    at a time when C's rows are 16-byte aligned, one element at a time
    otherwise.  C placed `shift` words into a sentinel buffer whose rows are
    N + extra words apart: every placement gives the exact product and
    writes nothing outside C (page 1, section [Matrix Multiplication]: each
    output written once, where it belongs)."""
    M, N, K = 333, 260, 100
    A, B = int_inputs(M, N, K, 77 + shift + extra)
    Pi = oracle.gemm_i64(A, B)
    name = "m160n128k32_w1x4_vec4_nn"
    v = variants().index(name)
    rows, cols = M + 2, N + extra + shift
    big = torch.full((rows, cols), 12345.0, dtype=torch.float32, device="cuda")
    Cv = big[:M, shift:shift + N]
    log(f"row-store epilogue {M}x{N}x{K} shift {shift} extra {extra}: {name}")
    tg.sgemm(dev(A), dev(B), out=Cv, kernel="mfma", variant=v)
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    assert_exact(got[:M, shift:shift + N], Pi, f"{name} shift {shift} extra {extra}")
    outside = np.ones(got.shape, bool)
    outside[:M, shift:shift + N] = False
    assert np.all(got[outside] == 12345.0), f"{name} wrote outside C"


@pytest.mark.parametrize("K", [1, 4, 15, 16, 17, 20, 31, 32, 33, 36, 48, 64, 100])
def test_partial_phases_integer_exact(K):
    """K below, at and just past the phase depths (16 and 32) of every
    configuration, with ragged M and N, in integers (exact)."""
    M, N = 259, 131 if K % 4 else 132
    A, B = int_inputs(M, N, K, 1000 + K)
    Pi = oracle.gemm_i64(A, B)
    log(f"partial phases K={K}")
    for v, name in enumerate(variants()):
        if runnable(name, M, N, K):
            assert_exact(run(A, B, "mfma", variant=v), Pi, f"{name} K={K}")
    assert_exact(run(A, B), Pi, "auto")


RING_KS = sorted({16 * f + r for f in range(4, 13) for r in (0, 5)} |
                 {32 * f + r for f in range(4, 10) for r in (0, 9)})


@pytest.mark.parametrize("K", RING_KS)
def test_phase_ring_tail_integer_exact(K):
    """The tiled kernels run their main loop two phases at a time and finish
    in a tail loop; K sweeps the number of full phases (4 to 12 at depth 16,
    4 to 9 at depth 32), with and without a shorter last phase, so the main
    loop hands over to the tail at every offset.  Integers, exact."""
    M, N = 259, 131 if K % 4 else 132
    A, B = int_inputs(M, N, K, 2000 + K)
    Pi = oracle.gemm_i64(A, B)
    log(f"phase ring K={K}")
    for v, name in enumerate(variants()):
        if runnable(name, M, N, K):
            assert_exact(run(A, B, "mfma", variant=v), Pi, f"{name} K={K}")


def test_persistent_grid_integer_exact_with_guard_bands():
    """More tiles than the chip holds at once for every configuration
    (4100² is 561 tiles of 256×128, 1089 of 128², 4225 of 64², so each
    work-group of the persistent grid runs several), ragged in M and N, with
    enough whole phases at either depth (16 and 32) for the main loop's
    whole-phase loads and a shorter last phase.  A and B sit in NaN-filled
    wider buffers and C inside sentinels: a NaN in C means a load outside
    the operands, a changed sentinel a store outside C.  Integers, exact."""
    M, N, K = 4100, 4100, 196
    A, B = int_inputs(M, N, K, 4100)
    Pi = oracle.gemm_i64(A, B)
    for v, name in [(None, "auto")] + list(enumerate(variants())):
        if v is not None and not runnable(name, M, N, K):
            continue
        log(f"persistent grid {M}x{N}x{K}: {name}")
        _, Av = guarded(A, 3, 8, float("nan"))
        _, Bv = guarded(B, 5, 4, float("nan"))
        Cbig, Cv = guarded(np.zeros((M, N), np.float32), 2, 4, 12345.0)
        if v is None:
            tg.sgemm(Av, Bv, out=Cv)
        else:
            tg.sgemm(Av, Bv, out=Cv, kernel="mfma", variant=v)
        torch.cuda.synchronize()
        big = Cbig.cpu().numpy()
        assert_exact(big[:M, :N], Pi, name)
        outside = np.ones(big.shape, bool)
        outside[:M, :N] = False
        assert np.all(big[outside] == 12345.0), f"{name} wrote outside C"


def test_persistent_grid_transposed_integer_exact():
    """The persistent grid with operands stored transposed (the main
    configuration in all four orders), ragged and with a shorter last
    phase.  Integers, exact."""
    M, N, K = 4100, 4100, 100
    A, B = int_inputs(M, N, K, 4101)
    Pi = oracle.gemm_i64(A, B)
    for ta, tb in OPS:
        dA, dB = stored(A, ta), stored(B, tb)
        log(f"persistent grid transposed ta={ta} tb={tb}")
        C = tg.sgemm(dA, dB)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), Pi, f"auto ta={ta} tb={tb}")


def test_leading_dimension_beyond_buffer_offsets():
    """lda past what 32-bit buffer offsets cover: tgemm_sgemm runs the 64-bit
    pointer configuration, buffer configurations refuse it."""
    M, N, K = 130, 68, 40
    lda = (1 << 24) + 8  # past every buffer configuration's limit (32+ rows × lda × 4 B >= 2^31)
    A, B = int_inputs(M, N, K, 4242)
    Pi = oracle.gemm_i64(A, B)
    big = torch.empty((M, lda), dtype=torch.float32, device="cuda")
    big[:, :K] = dev(A)
    Av = big[:, :K]
    dB = dev(B)
    C = tg.sgemm(Av, dB)
    torch.cuda.synchronize()
    assert_exact(C.cpu().numpy(), Pi, "auto, huge lda")
    v = tg.tgemm_sgemm_variant_for(M, N, K, Av.data_ptr(), lda, dB.data_ptr(), N, C.data_ptr(), N)
    assert variants()[v].endswith("_flat")
    for v, name in enumerate(variants()):
        st = tg.tgemm_sgemm_mfma(M, N, K, Av.data_ptr(), lda, dB.data_ptr(), N, C.data_ptr(), N, v, None)
        assert (st == tg.TGEMM_SUCCESS) == name.endswith("_flat"), name
    torch.cuda.synchronize()
    del big


def test_largest_k():
    """K at the largest size the interface takes (2^31 - 2^16), M = N = 1, A
    stored transposed (K×1): one dot product of random ±1 values through the
    split-K configuration tgemm_sgemm picks.  Every partial sum any kernel can
    form is a sum of at most K independent ±1 terms, far below 2^24 in
    magnitude (Hoeffding), so float32 sums are exact.  With the values drawn
    as bits (1 -> +1, 0 -> -1) the exact dot product is K - 2·popcount(a xor b)."""
    K = 2 ** 31 - 2 ** 16
    rng = np.random.default_rng(20)
    pa = np.frombuffer(bytearray(rng.bytes(K // 8)), np.uint8)
    pb = np.frombuffer(bytearray(rng.bytes(K // 8)), np.uint8)
    want = K - 2 * int(np.bitwise_count(np.bitwise_xor(pa, pb)).sum(dtype=np.int64))

    def unpack(packed):  # bit b of byte i -> element 8i + b, as ±1 in float32
        bits = (torch.from_numpy(packed).to("cuda").unsqueeze(1) >>
                torch.arange(8, dtype=torch.uint8, device="cuda")) & 1
        x = bits.reshape(K, 1).float()
        del bits
        return x.mul_(2).sub_(1)

    log(f"largest K = {K}")
    dA, dB = unpack(pa), unpack(pb)  # both stored K×1
    C = torch.full((1, 1), float("nan"), device="cuda")
    v = tg.tgemm_sgemm_variant_for_ex(tg.TGEMM_OP_T, tg.TGEMM_OP_N, 1, 1, K, dA.data_ptr(), 1,
                                      dB.data_ptr(), 1, C.data_ptr(), 1)
    log(f"largest K: {variants()[v]}")
    st = tg.tgemm_sgemm_ex(tg.TGEMM_OP_T, tg.TGEMM_OP_N, 1, 1, K, dA.data_ptr(), 1, dB.data_ptr(), 1,
                           C.data_ptr(), 1, None)
    assert st == tg.TGEMM_SUCCESS
    torch.cuda.synchronize()
    assert C.item() == want
    st = tg.tgemm_sgemm_ex(tg.TGEMM_OP_T, tg.TGEMM_OP_N, 1, 1, K + 1, dA.data_ptr(), 1, dB.data_ptr(), 1,
                           C.data_ptr(), 1, None)
    assert st == tg.TGEMM_ERROR_NOT_SUPPORTED
    del dA, dB
    torch.cuda.empty_cache()


OPS = [(True, False), (False, True), (True, True)]


def stored(X, trans):
    """Device tensor with logical value X, stored as is or transposed."""
    if trans:
        return dev(np.ascontiguousarray(X.T)).t()
    return dev(X)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 5, 3), (33, 65, 17), (64, 64, 64), (129, 100, 36),
                                   (260, 131, 200), (300, 268, 513), (512, 512, 40)])
def test_transposed_operands_integer_exact(M, N, K):
    A, B = int_inputs(M, N, K, 31 * M + 7 * N + K)
    Pi = oracle.gemm_i64(A, B)
    for ta, tb in OPS:
        dA, dB = stored(A, ta), stored(B, tb)
        log(f"transposed {M}x{N}x{K} ta={ta} tb={tb}")
        C = tg.sgemm(dA, dB)
        torch.cuda.synchronize()
        assert_exact(C.cpu().numpy(), Pi, f"auto ta={ta} tb={tb}")
        for v, name in enumerate(variants()):
            if not runnable(name, M, N, K, ta, tb):
                continue
            C = tg.sgemm(dA, dB, kernel="mfma", variant=v)
            torch.cuda.synchronize()
            assert_exact(C.cpu().numpy(), Pi, f"{name} ta={ta} tb={tb}")


def test_transposed_operands_real_bound_and_guard_bands():
    """Real inputs within the bound; transposed storage inside NaN-filled,
    wider buffers, C inside sentinels."""
    M, N, K = 1000, 1300, 700
    A, B, _ = wl.random_matrices(M, N, K, "uniform", 17)
    P, S = oracle.gemm(A, B)
    for ta, tb in OPS:
        log(f"transposed real ta={ta} tb={tb}")
        sa = A.T if ta else A
        sb = B.T if tb else B
        _, va = guarded(np.ascontiguousarray(sa), 3, 8, float("nan"))
        _, vb = guarded(np.ascontiguousarray(sb), 5, 4, float("nan"))
        Cbig, Cv = guarded(np.zeros((M, N), np.float32), 2, 4, 12345.0)
        tg.sgemm(va.t() if ta else va, vb.t() if tb else vb, out=Cv)
        torch.cuda.synchronize()
        big = Cbig.cpu().numpy()
        assert_within_bound(big[:M, :N], P, S, K, f"ta={ta} tb={tb}")
        outside = np.ones(big.shape, bool)
        outside[:M, :N] = False
        assert np.all(big[outside] == 12345.0)


def test_transposed_identities_bit_exact():
    """Aᵀ-stored identity times Bᵀ-stored B, and Aᵀ-stored A times a
    Bᵀ-stored identity, are exact on real inputs for every configuration
    that takes transposed operands."""
    K, N, M = 136, 72, 100
    B = wl.random_matrices(K, 1, N, "normal", 5)[0]   # K×N
    A = wl.random_matrices(M, 1, K, "normal", 6)[0]   # M×K
    I_k = np.eye(K, dtype=np.float32)
    for v, name in enumerate(variants()):
        if runnable(name, K, N, K, True, True):
            C = tg.sgemm(stored(I_k, True), stored(B, True), kernel="mfma", variant=v)
            torch.cuda.synchronize()
            assert np.array_equal(C.cpu().numpy(), B), name
        if runnable(name, M, K, K, True, True):
            C = tg.sgemm(stored(A, True), stored(I_k, True), kernel="mfma", variant=v)
            torch.cuda.synchronize()
            assert np.array_equal(C.cpu().numpy(), A), name


# ------------------------------------------------------------ identities and invariants

def test_identities_bit_exact_real_inputs():
    """I·B = B, A·I = A and permutations are exact for any finite input: each
    output is one product by 1 plus exact zeros, in any summation order."""
    rng = np.random.default_rng(21)
    for (M, N, K) in [(200, 136, 72), (64, 64, 64), (33, 65, 129)]:
        A, B, _ = wl.random_matrices(M, N, K, "normal", 31)
        for kernel, kw in [("auto", {})] + [("mfma", {"variant": v}) for v, n in enumerate(variants())
                                             if runnable(n, M, N, K)]:
            log(f"identities {M}x{N}x{K} {kernel} {kw}")
            assert np.array_equal(run(np.eye(M, dtype=np.float32), A, kernel, **kw), A)
            assert np.array_equal(run(B, np.eye(N, dtype=np.float32), kernel, **kw), B)
            perm = rng.permutation(K)
            Pm = np.eye(K, dtype=np.float32)[perm]
            assert np.array_equal(run(Pm, B, kernel, **kw), B[perm])
            assert np.array_equal(run(A, np.ascontiguousarray(Pm.T), kernel, **kw), A[:, perm])


def test_one_hot_locates_every_position():
    M, N, K = 130, 100, 70
    rng = np.random.default_rng(3)
    for _ in range(6):
        i0, k0, j0 = int(rng.integers(M)), int(rng.integers(K)), int(rng.integers(N))
        A = np.zeros((M, K), np.float32)
        B = np.zeros((K, N), np.float32)
        A[i0, k0] = 3.0
        B[k0, j0] = -5.0
        want = np.zeros((M, N), np.float32)
        want[i0, j0] = -15.0
        for v, name in enumerate(variants()):
            if not runnable(name, M, N, K):
                continue
            assert np.array_equal(run(A, B, "mfma", variant=v), want), (name, i0, k0, j0)


def test_transpose_symmetry():
    """(A·B)ᵀ == Bᵀ·Aᵀ: exact on integers, within twice the bound on reals."""
    A, B = int_inputs(96, 160, 200, 77)
    C = run(A, B)
    Ct = run(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct)
    A, B, _ = wl.random_matrices(96, 160, 200, "uniform", 78)
    _, S = oracle.gemm(A, B)
    C = run(A, B).astype(np.float64)
    Ct = run(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T)).astype(np.float64)
    assert np.all(np.abs(C.T - Ct) <= 8 * 200 * TWO_M24 * S.T)


def test_invariants_scaling_sign_determinism():
    A, B, _ = wl.random_matrices(320, 288, 264, "uniform", 91)
    for kernel, kw in [("auto", {}), ("naive", {}), ("lds", {"tile": 16, "pad": 1}), ("simt", {})] + \
            [("mfma", {"variant": v}) for v in range(len(variants()))]:
        log(f"invariants {kernel} {kw}")
        C = run(A, B, kernel, **kw)
        assert np.array_equal(C, run(A, B, kernel, **kw)), "not deterministic"
        assert np.array_equal(run(A * np.float32(8), B * np.float32(0.25), kernel, **kw), C * 2)
        assert np.array_equal(run(-A, B, kernel, **kw), -C)


def test_worked_example_tile2():
    """Page 1's 4x4 example through the TILE_WIDTH = 2 tiled kernel: values
    M_ik = 4i+k+1, N_kj = 4k+j+1; closed form (4i+1)(4j+28) + 6j + 62."""
    Mx = np.array([[4 * i + k + 1 for k in range(4)] for i in range(4)], np.float32)
    Nx = np.array([[4 * k + j + 1 for j in range(4)] for k in range(4)], np.float32)
    want = np.array([[(4 * i + 1) * (4 * j + 28) + 6 * j + 62 for j in range(4)] for i in range(4)],
                    np.float32)
    for pad in (0, 1):
        assert np.array_equal(run(Mx, Nx, "lds", tile=2, pad=pad), want)
    assert np.array_equal(run(Mx, Nx, "naive"), want)
    assert np.array_equal(run(Mx, Nx, "simt"), want)
    for v, name in enumerate(variants()):
        assert np.array_equal(run(Mx, Nx, "mfma", variant=v), want), name


def test_graph_capture_replays():
    """Calls captured into a HIP graph (torch.cuda.graph) replay correctly, many
    times, with eager work and synchronisations between the replays; K = 0
    (the fill kernel) is captured too."""
    shapes = [(300, 260, 180), (512, 512, 512), (1030, 900, 700)]
    ins = []
    for s_, (M, N, K) in enumerate(shapes):
        A, B = int_inputs(M, N, K, 70 + s_)
        ins.append((dev(A), dev(B), torch.empty((M, N), device="cuda"), oracle.gemm_i64(A, B)))
    Cz = torch.full((7, 9), float("nan"), device="cuda")
    Az, Bz = torch.empty((7, 0), device="cuda"), torch.empty((0, 9), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the capture
        for dA, dB, dC, _ in ins:
            tg.sgemm(dA, dB, out=dC)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dA, dB, dC, _ in ins:
            tg.sgemm(dA, dB, out=dC)
        tg.sgemm(Az, Bz, out=Cz)
    for rep in range(5):
        for _, _, dC, _ in ins:
            dC.fill_(float("nan"))
        Cz.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, _, dC, Pi) in ins:
            assert_exact(dC.cpu().numpy(), Pi, f"replay {rep}")
        cz = Cz.cpu().numpy()
        assert np.all(cz == 0) and not np.any(np.signbit(cz)), f"replay {rep}: K = 0 fill"
        # eager work between replays
        x = torch.randn(1024, 1024, device="cuda")
        _ = (x @ x).sum().item()


# ------------------------------------------------------------ ABI on the device

def test_zero_k_fills_positive_zero_and_empty_is_noop():
    for kernel, kw in [("auto", {}), ("naive", {}), ("lds", {"tile": 16, "pad": 0}), ("simt", {}),
                       ("mfma", {"variant": 0})]:
        C = torch.full((5, 12), float("nan"), device="cuda")
        tg.sgemm(torch.empty((5, 0), device="cuda"), torch.empty((0, 12), device="cuda"), out=C,
                 kernel=kernel, **kw)
        torch.cuda.synchronize()
        c = C.cpu().numpy()
        assert np.all(c == 0) and not np.any(np.signbit(c)), kernel
        C = torch.full((0, 12), 7.0, device="cuda")
        tg.sgemm(torch.ones((0, 3), device="cuda"), torch.ones((3, 12), device="cuda"), out=C,
                 kernel=kernel, **kw)
    sentinel = torch.full((4, 4), 7.0, device="cuda")
    st = tg.tgemm_sgemm(4, 4, 4, sentinel.data_ptr(), 4, sentinel.data_ptr(), 4, 0, 4, None)
    assert st == tg.TGEMM_ERROR_INVALID_VALUE


def test_errors_leave_c_untouched():
    A = dev(np.ones((8, 8), np.float32))
    C = torch.full((8, 8), 3.0, device="cuda")
    st = tg.tgemm_sgemm(8, 8, 8, A.data_ptr(), 7, A.data_ptr(), 8, C.data_ptr(), 8, None)
    assert st == tg.TGEMM_ERROR_INVALID_VALUE
    st = tg.tgemm_sgemm(8, 8, 8, A.data_ptr(), 8, A.data_ptr(), 8, A.data_ptr(), 8, None)
    assert st == tg.TGEMM_ERROR_INVALID_VALUE  # C overlaps A
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


def test_non_default_stream():
    A, B = int_inputs(300, 260, 180, 5)
    Pi = oracle.gemm_i64(A, B)
    s = torch.cuda.Stream()
    dA, dB = dev(A), dev(B)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = tg.sgemm(dA, dB)
    s.synchronize()
    assert_exact(C.cpu().numpy(), Pi, "side stream")
    C2 = torch.empty_like(C)
    tg.sgemm(dA, dB, out=C2, stream=s.cuda_stream)
    s.synchronize()
    assert torch.equal(C, C2)


def test_concurrent_products_on_two_streams():
    """Two products queued at once on two streams, each with more tiles than
    the chip holds (so each launches the persistent grid that can fill every
    compute unit), interleaved several times: every result exact."""
    shapes = [(4100, 2052, 100), (2100, 4100, 68)]
    ins = [int_inputs(M, N, K, 77 + i) for i, (M, N, K) in enumerate(shapes)]
    want = [oracle.gemm_i64(A, B) for A, B in ins]
    dins = [(dev(A), dev(B)) for A, B in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(3)] for M, N, _ in shapes]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, s in enumerate(streams):
            tg.sgemm(*dins[i], out=outs[i][rep], stream=s.cuda_stream)
    for s in streams:
        s.synchronize()
    for i in range(2):
        for rep in range(3):
            log(f"concurrent stream {i} call {rep}")
            assert_exact(outs[i][rep].cpu().numpy(), want[i], f"stream {i} call {rep}")


def test_side_stream_output_allocation_waits_for_current_stream():
    """sgemm and transpose with `out` omitted and a side stream given: the
    output is allocated on the current stream, whose pending work may still
    read the block's previous owner.  Here a tensor X is freed while a copy
    of it, queued behind several milliseconds of other work, is still
    pending on the current stream; the output allocated next (same size) may
    be handed X's block.  The binding makes the side stream wait for the
    current one first, so the copy still sees X and the product is exact."""
    M, N, K = 1024, 1024, 512
    A, B = int_inputs(M, N, K, 91)
    Pi = oracle.gemm_i64(A, B)
    dA, dB = dev(A), dev(B)
    T = np.arange(M * N, dtype=np.float32).reshape(M, N)  # exact in float32
    dT = dev(T)
    side = torch.cuda.Stream()
    W = torch.rand(4096, 4096, device="cuda")
    V = torch.empty_like(W)
    torch.cuda.synchronize()
    for rep in range(3):
        log(f"side-stream allocation, rep {rep}")
        for what in ("sgemm", "transpose"):
            X = torch.full((M, N), 1.5, device="cuda")
            Z = torch.empty_like(X)
            for _ in range(3):
                tg.sgemm(W, W, out=V)  # several ms of work on the current stream
            Z.copy_(X)                 # reads X once that work is done
            del X                      # X's block goes back to the cache, still to be read
            if what == "sgemm":
                C = tg.sgemm(dA, dB, stream=side.cuda_stream)
            else:
                C = tg.transpose(dT, stream=side.cuda_stream)  # N×M output: the size of X
            side.synchronize()
            torch.cuda.synchronize()
            assert bool(torch.all(Z == 1.5)), f"{what} rep {rep}: the side stream wrote X's block before it was read"
            if what == "sgemm":
                assert_exact(C.cpu().numpy(), Pi, f"side-stream sgemm rep {rep}")
            else:
                assert np.array_equal(C.cpu().numpy(), T.T), f"side-stream transpose rep {rep}"
            del C, Z
