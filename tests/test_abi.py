"""The C ABI without a GPU: the library loads, exports exactly what
include/tgemm.h declares, the header stands alone in C and C++, and every
argument check returns its documented status before any HIP call is made.
"""

import ctypes
import os
import re
import subprocess

import pytest

import tiled_gemm_tgemm_amd as tg
from tiled_gemm_tgemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY):
        from tiled_gemm_tgemm_amd import build

        build.build()
    return tg.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(tgemm_\w+)\s*\(", text))


def test_header_declares_the_binding(lib):
    names = declared_functions()
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(tgemm_\w+)$", out, flags=re.M))
    assert declared_functions() <= exported
    for name in declared_functions():
        assert hasattr(lib, name)


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c11"), ("g++", "-std=c++17")])
def test_header_compiles_alone(tmp_path, compiler, std):
    ext = "c" if compiler == "gcc" else "cpp"
    src = tmp_path / f"use.{ext}"
    src.write_text('#include "tgemm.h"\nint main(void) { return tgemm_version() > 0 ? 0 : 1; }\n')
    subprocess.run([compiler, std, "-Wall", "-Werror", "-pedantic", f"-I{ROOT}/include", "-c",
                    str(src), "-o", str(tmp_path / "use.o")], check=True)


def test_static_queries(lib):
    assert tg.tgemm_version() == 200
    n = tg.tgemm_mfma_variant_count()
    assert n >= 6
    names = tg.variant_names()
    assert len(set(names)) == n and all(re.fullmatch(r"m\d+n\d+k\d+_w\dx\d(s\d)?_vec[14](_flat|_nn)?", x) for x in names)
    assert tg.tgemm_mfma_variant_name(n) is None and tg.tgemm_mfma_variant_name(-1) is None
    for st in range(4):
        assert tg.tgemm_status_string(st)
    assert "unknown" in tg.tgemm_status_string(99)


# Fake device addresses: argument checks never dereference them, and every
# case below is rejected (or finishes as a no-op) before any HIP call.
A_, B_, C_ = 0x10000000, 0x20000000, 0x30000000
INVALID, UNSUPPORTED = tg.TGEMM_ERROR_INVALID_VALUE, tg.TGEMM_ERROR_NOT_SUPPORTED
MAX_DIM = 2 ** 31 - 2 ** 16  # largest M, N, K the header allows

ENTRY = {
    "sgemm": lambda *a: tg.tgemm_sgemm(*a, None),
    "naive": lambda *a: tg.tgemm_sgemm_naive(*a, None),
    "lds": lambda *a: tg.tgemm_sgemm_lds(*a, 16, 1, None),
    "simt": lambda *a: tg.tgemm_sgemm_simt(*a, None),
    "mfma": lambda *a: tg.tgemm_sgemm_mfma(*a, 0, None),
}

CASES = [
    # (M, N, K, A, lda, B, ldb, C, ldc) -> status
    ((-1, 4, 4, A_, 4, B_, 4, C_, 4), INVALID),
    ((4, -1, 4, A_, 4, B_, 4, C_, 4), INVALID),
    ((4, 4, -1, A_, 4, B_, 4, C_, 4), INVALID),
    ((4, 4, 8, A_, 7, B_, 4, C_, 4), INVALID),      # lda < K
    ((4, 8, 4, A_, 4, B_, 7, C_, 8), INVALID),      # ldb < N
    ((4, 8, 4, A_, 4, B_, 8, C_, 7), INVALID),      # ldc < N
    ((4, 4, 4, A_, 0, B_, 4, C_, 4), INVALID),      # ld below 1
    ((4, 4, 4, 0, 4, B_, 4, C_, 4), INVALID),       # null A
    ((4, 4, 4, A_, 4, 0, 4, C_, 4), INVALID),       # null B
    ((4, 4, 4, A_, 4, B_, 4, 0, 4), INVALID),       # null C
    ((4, 4, 4, A_ + 2, 4, B_, 4, C_, 4), INVALID),  # misaligned A
    ((4, 4, 4, A_, 4, B_, 4, A_ + 8, 4), INVALID),  # C overlaps A
    ((4, 4, 4, A_, 4, B_, 4, B_ + 60, 4), INVALID),  # C overlaps B's last element
    ((2 ** 31, 4, 4, A_, 4, B_, 4, C_, 4), UNSUPPORTED),
    ((4, 4, 2 ** 31, A_, 2 ** 31, B_, 4, C_, 4), UNSUPPORTED),
    ((MAX_DIM + 1, 4, 4, A_, 4, B_, 4, C_, 4), UNSUPPORTED),       # largest size + 1
    ((0, 4, MAX_DIM + 1, A_, MAX_DIM + 1, B_, 4, C_, 4), UNSUPPORTED),
    ((0, 4, MAX_DIM, A_, MAX_DIM, B_, 4, C_, 4), tg.TGEMM_SUCCESS),  # largest K, M = 0
    ((4, 0, MAX_DIM, A_, MAX_DIM, B_, 1, C_, 1), tg.TGEMM_SUCCESS),
    ((0, 4, 4, A_, 4, B_, 4, C_, 4), tg.TGEMM_SUCCESS),  # M = 0: nothing to do
    ((4, 0, 4, A_, 4, B_, 1, C_, 1), tg.TGEMM_SUCCESS),  # N = 0
    ((0, 4, 4, 0, 4, 0, 4, 0, 4), tg.TGEMM_SUCCESS),     # no-op ignores pointers
    # operands that would run past the end of the address space cannot exist
    ((MAX_DIM, 4, 4, A_, 1 << 40, B_, 4, C_, 4), INVALID),       # A: 2^31 rows of 2^40 floats
    ((4, 4, MAX_DIM, A_, MAX_DIM, B_, 1 << 40, C_, 4), INVALID),  # B
    ((MAX_DIM, 4, 4, A_, 4, B_, 4, C_, 1 << 40), INVALID),       # C
    ((MAX_DIM, 4, 0, A_, 1, B_, 4, C_, 1 << 40), INVALID),       # C, even when K = 0 only zeroes it
]


@pytest.mark.parametrize("entry", sorted(ENTRY))
@pytest.mark.parametrize("args,status", CASES)
def test_argument_checks(lib, entry, args, status):
    assert ENTRY[entry](*args) == status


N_, T_ = tg.TGEMM_OP_N, tg.TGEMM_OP_T


@pytest.mark.parametrize("ops,args,status", [
    ((T_, N_), (8, 4, 4, A_, 7, B_, 4, C_, 4), INVALID),    # op(A)=Aᵀ: lda >= M
    ((T_, N_), (8, 4, 4, A_, 8, B_, 4, C_, 4), None),       # fine (no launch: see below)
    ((N_, T_), (4, 8, 6, A_, 6, B_, 5, C_, 8), INVALID),    # op(B)=Bᵀ: ldb >= K
    ((N_, T_), (4, 8, 6, A_, 5, B_, 6, C_, 8), INVALID),    # lda >= K still applies to A as stored
    ((2, N_), (4, 4, 4, A_, 4, B_, 4, C_, 4), UNSUPPORTED),  # unknown op
    ((N_, -1), (4, 4, 4, A_, 4, B_, 4, C_, 4), UNSUPPORTED),
    ((T_, T_), (4, 4, 4, A_, 4, B_, 4, A_ + 48, 4), INVALID),  # C overlaps Aᵀ's storage (4×4)
    ((T_, N_), (0, 4, 4, A_, 1, B_, 4, C_, 4), tg.TGEMM_SUCCESS),  # M = 0
])
def test_transposed_argument_checks(lib, ops, args, status):
    if status is None:
        # valid arguments: only ask which configuration would run (no launch)
        M, N, K, a, lda, b, ldb, c, ldc = args
        assert tg.tgemm_sgemm_variant_for_ex(*ops, M, N, K, 1 << 40, lda, 1 << 44, ldb, 1 << 46, ldc) >= 0
        return
    assert tg.tgemm_sgemm_ex(*ops, *args, None) == status
    assert tg.tgemm_sgemm_mfma_ex(*ops, *args, 0, None) == status


def test_transposed_variant_choice(lib):
    names = tg.variant_names()

    def chosen(op_a, op_b, M, N, K, lda, ldb):
        v = tg.tgemm_sgemm_variant_for_ex(op_a, op_b, M, N, K, 1 << 40, lda, 1 << 44, ldb, 1 << 46, N)
        return names[v] if v >= 0 else None

    # Aᵀ·B goes to the one-wavefront-per-SIMD 256×256 tile, which keeps two
    # register sets of staged loads (MI355X, 8192³: 153.0 against 148.2
    # TFLOP/s for 256×128; 4096³: 151.4 against 146.5)
    assert chosen(T_, N_, 4096, 4096, 4096, 4096, 4096) == "m256n256k16_w2x4_vec4"
    assert chosen(T_, N_, 8192, 8192, 8192, 8192, 8192) == "m256n256k16_w2x4_vec4"
    assert chosen(N_, T_, 4096, 4096, 4096, 4096, 4096) == "m256n128k16_w2x2_vec4"   # 151.7 against 150.8
    assert chosen(N_, T_, 8192, 8192, 8192, 8192, 8192) == "m256n256k16_w2x4_vec4"
    assert chosen(T_, T_, 512, 512, 512, 512, 512) == "m32n32k32_w1x1s8_vec4"
    # Aᵀ with M not a multiple of 4: its stored rows cannot take 16-byte loads
    assert chosen(T_, N_, 4098, 4096, 4096, 4098, 4096).endswith("vec1")
    # row-major A with K not a multiple of 4, but Aᵀ rows (length M) can
    assert chosen(T_, N_, 4096, 4096, 4095, 4096, 4096).endswith("vec4")
    # no configuration takes a transposed operand with an enormous leading dimension
    assert chosen(T_, N_, 64, 64, 64, 1 << 28, 64) is None
    assert tg.tgemm_sgemm_ex(T_, N_, 64, 64, 64, 1 << 40, 1 << 28, 1 << 44, 64, 1 << 46, 64, None) == UNSUPPORTED
    # the 64-bit-pointer fallback and the "_nn" configurations take operands as stored only
    flat = [i for i, n in enumerate(names) if n.endswith("_flat") or n.endswith("_nn")]
    assert any(n.endswith("_nn") for n in names)
    for v in flat:
        assert tg.tgemm_sgemm_mfma_ex(T_, N_, 64, 64, 64, 1 << 40, 64, 1 << 44, 64, 1 << 46, 64, v,
                                      None) == UNSUPPORTED


def test_kernel_choice_checks(lib):
    args = (64, 64, 64, A_, 64, B_, 64, C_, 64)
    n = tg.tgemm_mfma_variant_count()
    assert tg.tgemm_sgemm_mfma(*args, n, None) == UNSUPPORTED
    assert tg.tgemm_sgemm_mfma(*args, -1, None) == UNSUPPORTED
    for tile, pad in [(3, 0), (64, 0), (16, 2), (0, 0)]:
        assert tg.tgemm_sgemm_lds(*args, tile, pad, None) == UNSUPPORTED
    # a 16-byte-load variant on operands that cannot take them
    vec4 = [i for i, name in enumerate(tg.variant_names()) if name.endswith("vec4")]
    # buffer-load configurations refuse leading dimensions beyond 32-bit offsets
    buf = [i for i, name in enumerate(tg.variant_names()) if not name.endswith("_flat")]
    flat = [i for i, name in enumerate(tg.variant_names()) if name.endswith("_flat")]
    assert flat and buf
    for v in buf:
        assert tg.tgemm_sgemm_mfma(64, 64, 64, 1 << 40, 1 << 24, 1 << 44, 64, 1 << 46, 64, v,
                                   None) == UNSUPPORTED
    assert tg.tgemm_sgemm_mfma(64, 63, 64, A_, 64, B_, 63, C_, 63, vec4[0], None) == UNSUPPORTED
    assert tg.tgemm_sgemm_mfma(64, 64, 63, A_, 63, B_, 64, C_, 64, vec4[0], None) == UNSUPPORTED
    assert tg.tgemm_sgemm_mfma(64, 64, 64, A_ + 4, 64, B_, 64, C_, 64, vec4[0], None) == UNSUPPORTED


def test_variant_choice(lib):
    names = tg.variant_names()

    def chosen(M, N, K, a=1 << 40, lda=None, ldb=None, ldc=None, c=1 << 46):
        v = tg.tgemm_sgemm_variant_for(M, N, K, a, lda or K, 1 << 44, ldb or N, c, ldc or N)
        return names[v] if v >= 0 else None

    # MI355X: 8192³ 7.16-7.20 ms (256×256) against 7.18-7.19 (256×128) with 24%
    # fewer bytes moved; 4096³ 905-909 µs (256×128) against 908-912 (256×256)
    assert chosen(8192, 8192, 8192) == "m256n256k16_w2x4_vec4"
    assert chosen(4096, 4096, 4096) == "m256n128k16_w2x2_vec4"
    assert chosen(16384, 5000, 8192) == "m256n256k16_w2x4_vec4"   # 8.96 ms against 9.03
    assert chosen(8192, 4096, 1024) == "m256n128k16_w2x2_vec4"    # 472 µs against 477
    # ragged: 760 tiles of 160×128, three per CU at most, 219-222 µs against 234 for the
    # 480 tiles of 256×128 in one round
    assert chosen(3000, 5000, 1000) == "m160n128k32_w1x4_vec4_nn"
    # that tile stores C four columns at a time: not chosen when C's rows are
    # not 16-byte aligned (it would store one element at a time)
    assert chosen(3000, 5000, 1000, c=(1 << 46) + 4) != "m160n128k32_w1x4_vec4_nn"
    assert chosen(3000, 5000, 1000, ldc=5001) != "m160n128k32_w1x4_vec4_nn"
    # 79.3 µs against 77.5 for 64×64 on random inputs: the model's one miss above 2% among the
    # shapes where 64×64 competes (short K, where it overrates the larger tiles' rounds)
    assert chosen(640, 8192, 1000) == "m160n128k32_w1x4_vec4_nn"
    assert chosen(3000, 3000, 3000) == "m64n64k32_w2x2_vec4"       # 409 µs against 421 for 160×128
    # 32×32 tiles with K split over eight wavefronts: 7.3-7.5 µs against 11.7
    # for 64×64 tiles on MI355X
    assert chosen(512, 512, 512) == "m32n32k32_w1x1s8_vec4"
    assert chosen(1024, 1024, 1024) == "m64n64k32_w2x2_vec4"
    assert chosen(2048, 2048, 2048) == "m128n128k32_w2x2_vec4"  # 123.6 µs vs 127.6 for 64×64
    assert chosen(640, 640, 640) == "m32n32k32_w1x1s4_vec4"     # 11.1 µs vs 13.6 for 64×64 on MI355X
    assert chosen(2500, 2500, 2500) == "m64n64k32_w2x2_vec4"    # 272 µs vs 305 for 128×128
    assert chosen(6144, 6144, 6144) == "m128n128k32_w2x2_vec4"
    assert chosen(256, 256, 8192) == "m32n32k32_w1x1s8_vec4"    # 50.0 µs on MI355X
    assert chosen(2048, 256, 8192) == "m32n32k32_w1x1s4_vec4"   # 92.0 µs vs 131.2 for 64×64
    assert chosen(2048, 256, 8192, a=(1 << 40) + 4) == "m32n32k32_w1x1s4_vec1"  # 153 µs on MI355X
    assert chosen(64, 64, 64) == "m64n64k32_w2x2_vec4"          # 4.0 µs vs 5.0 for 32×32 tiles
    # long K on few tiles: the unsplit 64×64 tile (133 µs on MI355X)
    assert chosen(1024, 1024, 8192) == "m64n64k32_w2x2_vec4"
    assert chosen(300, 300, 300, lda=1 << 24).endswith("_flat")   # lda beyond 32-bit offsets
    assert "vec4" in chosen(3000, 5000, 1000)
    assert chosen(7, 5, 3).endswith("vec1")          # K, N not multiples of 4
    assert chosen(64, 64, 64, a=(1 << 40) + 4).endswith("vec1")  # A not 16-byte aligned
    assert chosen(0, 4, 4) is None and chosen(4, 4, 0) is None
    assert tg.tgemm_sgemm_variant_for(4, 4, 4, A_, 2, B_, 4, C_, 4) == -1  # lda < K


def test_row_store_configuration_needs_aligned_c(lib):
    """The 160×128 configuration writes C in 16-byte row pieces: over a grid
    of shapes, the automatic choice takes it only when C and ldc are 16-byte
    aligned, and takes some other configuration (not none) otherwise."""
    names = tg.variant_names()
    row_store = names.index("m160n128k32_w1x4_vec4_nn")
    picked_aligned = 0
    for M in (1000, 2560, 3000, 5000):
        for N in (1000, 2048, 5000):
            for K in (1000, 4096):
                a, b, c = 1 << 40, 1 << 44, 1 << 46
                v = tg.tgemm_sgemm_variant_for(M, N, K, a, K, b, N, c, N)
                picked_aligned += v == row_store
                for c_off, ldc in ((4, N), (0, N + 1), (8, N + 2)):
                    w = tg.tgemm_sgemm_variant_for(M, N, K, a, K, b, N, c + c_off, ldc)
                    assert w >= 0 and w != row_store, (M, N, K, c_off, ldc)
    assert picked_aligned > 0


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name in ("TGEMM_OP_N", "TGEMM_OP_T", "TGEMM_TRANSPOSE_BLOCKED", "TGEMM_TRANSPOSE_NAIVE",
                 "TGEMM_TRANSPOSE_TILED", "TGEMM_TRANSPOSE_TILED_PADDED", "TGEMM_SUCCESS",
                 "TGEMM_ERROR_INVALID_VALUE", "TGEMM_ERROR_NOT_SUPPORTED", "TGEMM_ERROR_HIP"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(_lib, name), name


TRANSPOSE_CASES = [
    ((-1, 4, A_, 4, B_, 1), INVALID),
    ((4, -1, A_, 1, B_, 4), INVALID),
    ((4, 8, A_, 7, B_, 4), INVALID),                # lda < N
    ((4, 8, A_, 8, B_, 3), INVALID),                # ldb < M
    ((4, 8, 0, 8, B_, 4), INVALID),                 # null A
    ((4, 8, A_, 8, 0, 4), INVALID),                 # null B
    ((4, 8, A_ + 2, 8, B_, 4), INVALID),            # misaligned A
    ((4, 8, A_, 8, B_ + 1, 4), INVALID),            # misaligned B
    ((4, 8, A_, 8, A_ + 4 * 31, 4), INVALID),       # B starts on A's last element
    ((4, 8, B_ - 4 * 31, 8, B_, 4), INVALID),       # A ends on B's first element
    ((MAX_DIM + 1, 1, A_, 1, B_, MAX_DIM + 1), UNSUPPORTED),
    ((4, 8, A_, 1 << 41, B_, 4), UNSUPPORTED),
    ((0, 8, A_, 8, B_, 1), tg.TGEMM_SUCCESS),       # M = 0: nothing to do
    ((4, 0, 0, 1, 0, 4), tg.TGEMM_SUCCESS),         # N = 0 ignores pointers
    ((MAX_DIM, 4, A_, 1 << 40, B_, MAX_DIM), INVALID),  # A runs past the address space
    ((4, MAX_DIM, A_, MAX_DIM, B_, 1 << 40), INVALID),  # B likewise
]


@pytest.mark.parametrize("args,status", TRANSPOSE_CASES)
def test_transpose_argument_checks(lib, args, status):
    for kernel in range(4):
        assert tg.tgemm_transpose(*args, kernel, None) == status, kernel


def test_transpose_kernel_choice_checks(lib):
    for kernel in (-1, 4, 99):
        assert tg.tgemm_transpose(4, 8, A_, 8, B_, 4, kernel, None) == UNSUPPORTED


def test_host_workspace_size(lib):
    MiB = 1 << 20
    # B, then two A panels and two C panels of (about M/4 rounded up to 256) rows
    assert tg.tgemm_sgemm_host_workspace_size(8192, 8192, 8192, 0) == 256 * MiB + 2 * 64 * MiB + 2 * 64 * MiB
    assert tg.tgemm_sgemm_host_workspace_size(8192, 8192, 8192, 1024) == 256 * MiB + 4 * 32 * MiB
    r = 256  # M = 300: about 75 rows, rounded up to one 256-row tile
    assert tg.tgemm_sgemm_host_workspace_size(300, 10, 7, 0) == 512 + 2 * (r * 7 * 4) + 2 * (r * 10 * 4)
    assert tg.tgemm_sgemm_host_workspace_size(100, 10, 7, 0) == 512 + 2 * 2816 + 2 * 4096  # panel = M
    assert tg.tgemm_sgemm_host_workspace_size(0, 10, 7, 0) == 0
    assert tg.tgemm_sgemm_host_workspace_size(10, 10, 0, 0) == 0
    assert tg.tgemm_sgemm_host_workspace_size(-1, 10, 7, 0) == -1
    assert tg.tgemm_sgemm_host_workspace_size(10, 10, 7, -5) == -1
    assert tg.tgemm_sgemm_host_workspace_size(MAX_DIM + 1, 10, 7, 0) == -1


W_ = 0x40000000  # fake 256-byte-aligned device workspace
HOST_CASES = [
    ((4, 4, 4, A_, 4, B_, 4, C_, 4, W_, 1 << 20, -1), INVALID),       # negative panel_rows
    ((4, 4, 4, A_, 3, B_, 4, C_, 4, W_, 1 << 20, 0), INVALID),        # lda < K
    ((4, 4, 4, A_, 4, B_, 4, C_, 4, 0, 1 << 20, 0), INVALID),         # no workspace
    ((4, 4, 4, A_, 4, B_, 4, C_, 4, W_ + 16, 1 << 20, 0), INVALID),   # misaligned workspace
    ((4, 4, 4, A_, 4, B_, 4, C_, 4, W_, 64, 0), INVALID),             # workspace too small
    ((4, 4, 4, 0, 4, B_, 4, C_, 4, W_, 1 << 20, 0), INVALID),         # null A
    ((4, 4, 4, A_, 4, B_, 4, A_ + 8, 4, W_, 1 << 20, 0), INVALID),    # C overlaps A
    ((MAX_DIM + 1, 4, 4, A_, 4, B_, 4, C_, 4, W_, 1 << 20, 0), UNSUPPORTED),
    ((0, 4, 4, A_, 4, B_, 4, C_, 4, 0, 0, 0), tg.TGEMM_SUCCESS),      # M = 0: nothing to do
    ((MAX_DIM, 4, 4, A_, 1 << 40, B_, 4, C_, 4, W_, 1 << 20, 0), INVALID),  # A past the address space
    ((MAX_DIM, 4, 0, A_, 1, B_, 4, C_, 1 << 40, 0, 0, 0), INVALID),        # C likewise, K = 0
]


@pytest.mark.parametrize("args,status", HOST_CASES)
def test_host_argument_checks(lib, args, status):
    assert tg.tgemm_sgemm_host(*args, None, None, None) == status


def test_host_empty_sum_is_written_on_the_host(lib):
    """K = 0 needs no device at all: C (with a leading dimension) becomes +0."""
    import numpy as np

    C = np.full((3, 7), np.nan, np.float32)
    st = tg.tgemm_sgemm_host(3, 5, 0, 0, 1, 0, 5, C.ctypes.data, 7, 0, 0, 0, None, None, None)
    assert st == tg.TGEMM_SUCCESS
    assert np.all(C[:, :5] == 0) and not np.any(np.signbit(C[:, :5])) and np.all(np.isnan(C[:, 5:]))


def test_splitk_workspace_size_and_choice(lib):
    assert tg.tgemm_sgemm_splitk_workspace_size(100, 60, 1000, 4) == 4 * 100 * 60 * 4
    assert tg.tgemm_sgemm_splitk_workspace_size(100, 60, 1000, 64) == 64 * 100 * 60 * 4
    for bad in [(100, 60, 1000, 1), (100, 60, 1000, 0), (100, 60, 1000, -2), (100, 60, 1000, 65),
                (0, 60, 1000, 4), (100, 0, 1000, 4), (100, 60, 0, 4), (-1, 60, 1000, 4),
                (MAX_DIM + 1, 4, 4, 4)]:
        assert tg.tgemm_sgemm_splitk_workspace_size(*bad) == 0, bad
    # many tiles: no split; few tiles with long K: a split (50.0 µs at 8
    # slices against 80.5 for the best unsplit kernel at 256×256×8192)
    assert tg.tgemm_sgemm_splitk_choose(8192, 8192, 8192) == 1
    assert tg.tgemm_sgemm_splitk_choose(4096, 4096, 4096) == 1
    for shape in [(256, 256, 16384), (512, 512, 16384), (2048, 256, 8192)]:
        s = tg.tgemm_sgemm_splitk_choose(*shape)
        assert s in (2, 4, 8, 16, 32, 64), (shape, s)
    assert tg.tgemm_sgemm_splitk_choose(0, 4, 4) == 1 and tg.tgemm_sgemm_splitk_choose(4, 4, -1) == 1


def test_splitk_argument_checks(lib):
    M, N, K = 64, 64, 4096
    args = (M, N, K, A_, K, B_, N, C_, N)
    W_ = 0x40000000
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, 4)
    assert need == 4 * M * N * 4
    for splits in (0, -1, 65):
        assert tg.tgemm_sgemm_splitk(*args, splits, W_, need, None) == INVALID
    assert tg.tgemm_sgemm_splitk(*args, 4, None, need, None) == INVALID          # no workspace
    assert tg.tgemm_sgemm_splitk(*args, 4, W_ + 4, need, None) == INVALID       # misaligned
    assert tg.tgemm_sgemm_splitk(*args, 4, W_, need - 4, None) == INVALID       # too small
    assert tg.tgemm_sgemm_splitk(*args, 4, C_, need, None) == INVALID           # overlaps C
    assert tg.tgemm_sgemm_splitk(*args, 4, A_ + 4096, need, None) == INVALID    # overlaps A
    assert tg.tgemm_sgemm_splitk(*args, 4, 2 ** 64 - 256, need, None) == INVALID  # wraps around
    # the product's own checks come first
    assert tg.tgemm_sgemm_splitk(M, N, K, A_, K - 1, B_, N, C_, N, 4, W_, need, None) == INVALID
    assert tg.tgemm_sgemm_splitk(-1, N, K, A_, K, B_, N, C_, N, 4, W_, need, None) == INVALID
    # empty products finish without a launch, whatever the workspace
    assert tg.tgemm_sgemm_splitk(0, N, K, A_, K, B_, N, C_, N, 4, None, 0, None) == tg.TGEMM_SUCCESS
    assert tg.tgemm_sgemm_splitk(M, 0, K, A_, K, B_, 1, C_, 1, 4, None, 0, None) == tg.TGEMM_SUCCESS


def test_splitk_ex_argument_checks(lib):
    M, N, K = 64, 64, 4096
    W_ = 0x40000000
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, 4)
    for op in (2, -1):
        assert tg.tgemm_sgemm_splitk_ex(op, N_, M, N, K, A_, K, B_, N, C_, N, 4, W_, need, None) == UNSUPPORTED
        assert tg.tgemm_sgemm_splitk_ex(N_, op, M, N, K, A_, K, B_, N, C_, N, 4, W_, need, None) == UNSUPPORTED
    # Aᵀ stored K×M: lda must reach M, not K
    assert tg.tgemm_sgemm_splitk_ex(T_, N_, M, N, K, A_, M - 1, B_, N, C_, N, 4, W_, need, None) == INVALID
    # Bᵀ stored N×K: ldb must reach K
    assert tg.tgemm_sgemm_splitk_ex(N_, T_, M, N, K, A_, K, B_, K - 1, C_, N, 4, W_, need, None) == INVALID
    # the workspace may not overlap a transposed A's K×M extent
    assert tg.tgemm_sgemm_splitk_ex(T_, N_, M, N, K, A_, M, B_, N, C_, N, 4, A_ + 4 * M * (K - 1), need,
                                    None) == INVALID


def test_splitk_workspace_size_never_wraps(lib):
    # 64·(2^31 - 2^16)²·4 bytes does not fit in 64 bits: reported as 0, and a
    # call with any workspace is refused before anything is queued
    assert tg.tgemm_sgemm_splitk_workspace_size(MAX_DIM, MAX_DIM, 4096, 64) == 0
    assert tg.tgemm_sgemm_splitk_workspace_size(MAX_DIM, MAX_DIM, 4096, 2) == 0     # 2^65 bytes
    assert tg.tgemm_sgemm_splitk_workspace_size(MAX_DIM, 1 << 20, 4096, 64) == 64 * MAX_DIM * (1 << 20) * 4
    assert tg.tgemm_sgemm_splitk(MAX_DIM, MAX_DIM, 4096, 1 << 40, 4096, 1 << 41, MAX_DIM, 1 << 46, MAX_DIM,
                                 64, 1 << 60, 2 ** 64 - 2 ** 61, None) == INVALID


def test_splitk_choice_matches_the_measured_best():
    # split counts against one timing loop on MI355X (integer inputs, µs, slices allowed while
    # each holds at least 1024 values of k): the measured fastest or within 2.5% of it
    assert tg.tgemm_sgemm_splitk_choose(384, 640, 4096) == 4      # 22.7; unsplit 28.2, 2 slices 30.3
    assert tg.tgemm_sgemm_splitk_choose(1024, 512, 4096) == 2     # 37.3; 4 slices 37.5, unsplit 50.6
    assert tg.tgemm_sgemm_splitk_choose(768, 768, 8192) == 8      # 84.9; 4 slices 94.1
    assert tg.tgemm_sgemm_splitk_choose(1024, 1024, 8192) == 4    # 125.6; unsplit 122.5, 2 slices 123.3
    assert tg.tgemm_sgemm_splitk_choose(256, 256, 16384) == 16    # 24.6; 4 slices 33.4
    assert tg.tgemm_sgemm_splitk_choose(2048, 2048, 8192) == 1    # unsplit 453; 2 slices 465
    assert tg.tgemm_sgemm_splitk_choose(1024, 1024, 1024) == 1    # slices would be under 1024 long


def test_splitk_noalloc_argument_checks(lib):
    """The allocation-free split-K entry point checks as tgemm_sgemm_splitk_ex
    does and refuses, before any device work, a product whose partial sums
    would not fit its fixed scratch."""
    M, N, K = 64, 64, 4096
    cap = tg.TGEMM_SPLITK_NOALLOC_BYTES
    assert cap == 32 << 20
    for op in (2, -1):
        assert tg.tgemm_sgemm_splitk_noalloc(op, N_, M, N, K, A_, K, B_, N, C_, N, 4, None) == UNSUPPORTED
        assert tg.tgemm_sgemm_splitk_noalloc(N_, op, M, N, K, A_, K, B_, N, C_, N, 4, None) == UNSUPPORTED
    for splits in (0, -1, 65):
        assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, M, N, K, A_, K, B_, N, C_, N, splits, None) == INVALID
    assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, M, N, K, A_, K - 1, B_, N, C_, N, 4, None) == INVALID
    assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, M, N, K, A_, K, B_, N, A_ + 8, N, 4, None) == INVALID
    # beyond the scratch: 2048×2048 in 4 slices needs 64 MiB; 1024×1024 in 16 needs 64 MiB
    assert tg.tgemm_sgemm_splitk_workspace_size(2048, 2048, 8192, 4) > cap
    big = (1 << 40, 8192, 1 << 42, 2048, 1 << 44, 2048)
    assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, 2048, 2048, 8192, *big, 4, None) == UNSUPPORTED
    assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, 1024, 1024, 8192, 1 << 40, 8192, 1 << 42, 1024, 1 << 44,
                                         1024, 16, None) == UNSUPPORTED
    # empty products finish without a launch
    assert tg.tgemm_sgemm_splitk_noalloc(N_, N_, 0, N, K, A_, K, B_, N, C_, N, 4, None) == tg.TGEMM_SUCCESS
