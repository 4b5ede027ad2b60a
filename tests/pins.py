"""Pins of the CPU oracle: checks that tie it to something other than itself.

Each pin returns None when it holds and a short failure message otherwise, so
the same battery runs on the real oracle (every pin must hold) and on copies
of oracle.c with a planted mistake (some pin must fail).  Each pin names what
fixes the expected answer: exact rational arithmetic, exact integer sums, a
closed form, an algebraic identity, the worked example on page 1, or the
IEEE-754 definition of round-to-nearest-even.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle

TWO_M53 = 2.0 ** -53
TWO_M24 = 2.0 ** -24


# ---------------------------------------------------------------- helpers

def exact_product(A, B):
    """Exact rational product and exact sum of |products| (pure Python)."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    P = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return P, S


def round_to_f32(x: Fraction) -> float:
    """Round an exact rational to the nearest float32, ties to even (IEEE 754).

    Written from the definition: find the binade, scale to an integer
    significand, round half to even.  Covers normal and subnormal results;
    overflow raises.
    """
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, -126)  # subnormal results share the quantum 2^-149
    quantum = Fraction(2) ** (e - 23)
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = n * quantum
    if value >= Fraction(2) ** 128:
        raise OverflowError("float32 overflow")
    return sign * float(value)


def seeded(shape, dist, seed):
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        x = rng.uniform(-1, 1, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "int":
        x = rng.integers(-4, 5, size=shape)
    elif dist == "wide":
        # wide exponent range: products and sums span many binades
        x = rng.standard_normal(size=shape) * 2.0 ** rng.integers(-20, 21, size=shape)
    else:
        raise ValueError(dist)
    return np.ascontiguousarray(x.astype(np.float32))


TINY_SHAPES = [(1, 1, 1), (1, 3, 2), (3, 1, 4), (2, 5, 3), (4, 4, 4), (5, 3, 7), (7, 6, 8),
               (3, 2, 1)]


# ---------------------------------------------------------------- pins

def pin_bruteforce_rational(lib):
    """Exact rationals on tiny shapes: |P − exact| <= K·2^-53·S, and S likewise."""
    for dist in ("uniform", "normal", "wide", "int"):
        for s, (M, N, K) in enumerate(TINY_SHAPES):
            A = seeded((M, K), dist, 100 + s)
            B = seeded((K, N), dist, 200 + s)
            P, S = oracle.gemm(A, B, lib=lib)
            Pe, Se = exact_product(A, B)
            for i in range(M):
                for j in range(N):
                    tol = Fraction(K) * Fraction(TWO_M53) * Se[i][j]
                    if abs(Fraction(float(P[i, j])) - Pe[i][j]) > tol:
                        return f"P[{i},{j}] {dist} {M}x{N}x{K}: {P[i, j]} vs {float(Pe[i][j])}"
                    if abs(Fraction(float(S[i, j])) - Se[i][j]) > tol:
                        return f"S[{i},{j}] {dist} {M}x{N}x{K}: {S[i, j]} vs {float(Se[i][j])}"
                    if dist == "int" and Fraction(float(P[i, j])) != Pe[i][j]:
                        return f"integer P[{i},{j}] not exact"
    return None


def pin_integer_paths(lib):
    """Integer inputs: float64 path == int64 path == exact numpy float64 matmul."""
    for s, (M, N, K) in enumerate([(17, 23, 31), (64, 48, 96), (33, 65, 129)]):
        A = seeded((M, K), "int", 300 + s)
        B = seeded((K, N), "int", 400 + s)
        P, _ = oracle.gemm(A, B, lib=lib)
        Pi = oracle.gemm_i64(A, B, lib=lib)
        ref = A.astype(np.int64) @ B.astype(np.int64)  # exact integer library matmul
        if not np.array_equal(Pi, ref):
            return f"int64 path differs from integer matmul at {M}x{N}x{K}"
        if not np.array_equal(P, ref.astype(np.float64)):
            return f"float64 path differs from integer matmul at {M}x{N}x{K}"
    return None


def pin_identities(lib):
    """I·B = B and A·I = A bitwise; permutations move rows/columns exactly."""
    rng = np.random.default_rng(7)
    M, N, K = 9, 11, 13
    A = seeded((M, K), "wide", 11)
    B = seeded((K, N), "wide", 12)
    P, _ = oracle.gemm(np.eye(K, dtype=np.float32), B, with_abs=False, lib=lib)
    if not np.array_equal(P, B.astype(np.float64)):
        return "I·B != B"
    P, _ = oracle.gemm(A, np.eye(K, dtype=np.float32), with_abs=False, lib=lib)
    if not np.array_equal(P, A.astype(np.float64)):
        return "A·I != A"
    perm = rng.permutation(K)
    Pm = np.eye(K, dtype=np.float32)[perm]  # row r of Pm is e_{perm[r]}
    P, _ = oracle.gemm(Pm, B, with_abs=False, lib=lib)
    if not np.array_equal(P, B[perm].astype(np.float64)):
        return "permutation·B != B[perm]"
    P, _ = oracle.gemm(A, Pm.T.copy(), with_abs=False, lib=lib)
    if not np.array_equal(P, A[:, perm].astype(np.float64)):
        return "A·permutationᵀ != A[:, perm]"
    return None


def pin_one_hot(lib):
    """A = e_(i0,k0), B = e_(k0,j0): the product is exactly one 1 at (i0, j0)."""
    M, N, K = 5, 7, 6
    for i0, k0, j0 in [(0, 0, 0), (4, 5, 6), (2, 3, 1), (1, 0, 5), (3, 5, 0)]:
        A = np.zeros((M, K), np.float32)
        B = np.zeros((K, N), np.float32)
        A[i0, k0] = 1
        B[k0, j0] = 1
        P, S = oracle.gemm(A, B, lib=lib)
        want = np.zeros((M, N))
        want[i0, j0] = 1
        if not np.array_equal(P, want) or not np.array_equal(S, want):
            return f"one-hot ({i0},{k0},{j0}) misplaced"
    return None


def pin_transpose(lib):
    """(A·B)ᵀ == Bᵀ·Aᵀ bitwise: the same products summed in the same k order."""
    for dist in ("uniform", "wide"):
        A = seeded((6, 10), dist, 21)
        B = seeded((10, 8), dist, 22)
        P, S = oracle.gemm(A, B, lib=lib)
        Q, T = oracle.gemm(B.T.copy(), A.T.copy(), lib=lib)
        if not np.array_equal(P.T, Q) or not np.array_equal(S.T, T):
            return f"(AB)ᵀ != BᵀAᵀ ({dist})"
    return None


def pin_closed_forms(lib):
    """Zeros give +0; ones give K; A_ik = 1, B_kj = j give K·j; S of ±1 entries is K."""
    M, N, K = 4, 6, 37
    P, S = oracle.gemm(np.zeros((M, K), np.float32), np.zeros((K, N), np.float32), lib=lib)
    if np.any(P != 0) or np.any(np.signbit(P)) or np.any(S != 0):
        return "zeros·zeros != +0"
    P, S = oracle.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32), lib=lib)
    if np.any(P != K) or np.any(S != K):
        return "ones·ones != K"
    B = np.tile(np.arange(N, dtype=np.float32), (K, 1))
    P, _ = oracle.gemm(np.ones((M, K), np.float32), B, lib=lib)
    if not np.array_equal(P, np.tile(K * np.arange(N, dtype=np.float64), (M, 1))):
        return "ones·[j] != K·j"
    signs = np.where(np.arange(M * K).reshape(M, K) % 3 == 0, -1, 1).astype(np.float32)
    P, S = oracle.gemm(signs, np.ones((K, N), np.float32), lib=lib)
    if np.any(S != K) or not np.array_equal(P[:, 0], signs.sum(axis=1).astype(np.float64)):
        return "±1 rows: wrong signed or absolute sum"
    return None


def pin_worked_example(lib):
    """Page 1's 4x4 example with M_ik = 4i+k+1, N_kj = 4k+j+1.

    Closed form derived by hand from the sums of k and k² over k = 0..3:
    P_ij = (4i+1)(4j+28) + 6j + 62, i.e. rows 90..120, 202..280, 314..440,
    426..600.
    """
    Mx = np.array([[4 * i + k + 1 for k in range(4)] for i in range(4)], np.float32)
    Nx = np.array([[4 * k + j + 1 for j in range(4)] for k in range(4)], np.float32)
    want = np.array([[(4 * i + 1) * (4 * j + 28) + 6 * j + 62 for j in range(4)]
                     for i in range(4)], np.float64)
    if want[0, 0] != 90 or want[3, 3] != 600:
        return "closed form itself is off"
    P, _ = oracle.gemm(Mx, Nx, lib=lib)
    if not np.array_equal(P, want):
        return "worked example differs from the closed form"
    if not np.array_equal(oracle.gemm_i64(Mx, Nx, lib=lib), want.astype(np.int64)):
        return "integer path differs on the worked example"
    return None


def pin_window(lib):
    """A window of the product equals the same slice of the full product, bitwise."""
    A = seeded((20, 30), "normal", 31)
    B = seeded((30, 25), "normal", 32)
    P, S = oracle.gemm(A, B, lib=lib)
    for i0, i1, j0, j1 in [(0, 20, 0, 25), (3, 9, 4, 21), (19, 20, 24, 25), (5, 5, 2, 7)]:
        Pw, Sw = oracle.gemm_window(A, B, i0, i1, j0, j1, lib=lib)
        if not np.array_equal(Pw, P[i0:i1, j0:j1]) or not np.array_equal(Sw, S[i0:i1, j0:j1]):
            return f"window ({i0},{i1},{j0},{j1}) differs from the full product"
    return None


def pin_leading_dimensions(lib):
    """The C entry points with A and B embedded in wider row-major buffers
    (lda > K, ldb > N, the padding NaN) give, bit for bit, the products of
    the contiguous operands: the row stride is honoured and nothing outside
    the operands is read."""
    lib = lib or oracle._load()
    M, K, N = 9, 13, 11
    A = seeded((M, K), "int", 33)
    B = seeded((K, N), "int", 34)
    lda, ldb = K + 3, N + 5
    Aw = np.full((M, lda), np.nan, np.float32)
    Bw = np.full((K, ldb), np.nan, np.float32)
    Aw[:, :K] = A
    Bw[:, :N] = B
    P, S = oracle.gemm(A, B, lib=lib)
    Pw = np.empty((M, N), np.float64)
    Sw = np.empty((M, N), np.float64)
    rc = lib.oracle_gemm_f64_window(M, N, K, Aw, lda, Bw, ldb, 0, M, 0, N, Pw, N, Sw.ctypes.data, N)
    if rc != 0 or not np.array_equal(Pw, P) or not np.array_equal(Sw, S):
        return "float64 product with lda > K, ldb > N differs from the contiguous one"
    Iw = np.empty((M, N), np.int64)
    rc = lib.oracle_gemm_i64(M, N, K, Aw, lda, Bw, ldb, Iw, N)
    if rc != 0 or not np.array_equal(Iw, oracle.gemm_i64(A, B, lib=lib)):
        return "int64 product with lda > K, ldb > N differs from the contiguous one"
    Fw = np.empty((M, N), np.float32)
    rc = lib.oracle_gemm_fma_f32(M, N, K, Aw, lda, Bw, ldb, Fw, N)
    if rc != 0 or not np.array_equal(Fw, oracle.gemm_fma_f32(A, B, lib=lib)):
        return "float32 model with lda > K, ldb > N differs from the contiguous one"
    want = oracle.checksums(A, B, lib=lib)
    got = [np.empty(M), np.empty(M), np.empty(N), np.empty(N)]
    rc = lib.oracle_checksums(M, N, K, Aw, lda, Bw, ldb, *got, np.empty(4 * K))
    if rc != 0 or not all(np.array_equal(g, w) for g, w in zip(got, want)):
        return "checksums with lda > K, ldb > N differ from the contiguous ones"
    return None


def pin_fma_model(lib):
    """The float32 model equals step-by-step exact rounding (IEEE RNE) of a·b + acc."""
    for dist, (M, N, K) in [("uniform", (3, 4, 9)), ("wide", (4, 3, 7)), ("normal", (2, 2, 16))]:
        A = seeded((M, K), dist, 41)
        B = seeded((K, N), dist, 42)
        C = oracle.gemm_fma_f32(A, B, lib=lib)
        for i in range(M):
            for j in range(N):
                acc = 0.0
                for k in range(K):
                    acc = round_to_f32(Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                                       + Fraction(acc))
                if float(C[i, j]) != acc or math.copysign(1, float(C[i, j])) != math.copysign(1, acc):
                    return f"fma model [{i},{j}] {dist}: {C[i, j]!r} vs {acc!r}"
    A = seeded((30, 50), "int", 43)
    B = seeded((50, 20), "int", 44)
    if not np.array_equal(oracle.gemm_fma_f32(A, B, lib=lib).astype(np.int64),
                          A.astype(np.int64) @ B.astype(np.int64)):
        return "fma model not exact on integers"
    return None


def pin_checksums(lib):
    """Row/column checksums equal the exact sums of the product on integer inputs,
    and stay within a few float64 ulps of them on real inputs."""
    A = seeded((23, 41), "int", 51)
    B = seeded((41, 19), "int", 52)
    row, rowabs, col, colabs = oracle.checksums(A, B, lib=lib)
    Pi = A.astype(np.int64) @ B.astype(np.int64)
    Si = np.abs(A.astype(np.int64)) @ np.abs(B.astype(np.int64))
    if not (np.array_equal(row, Pi.sum(1)) and np.array_equal(col, Pi.sum(0))):
        return "integer checksums differ from exact row/column sums"
    if not (np.array_equal(rowabs, Si.sum(1)) and np.array_equal(colabs, Si.sum(0))):
        return "integer absolute checksums differ from exact sums"
    A = seeded((7, 9), "normal", 53)
    B = seeded((9, 5), "normal", 54)
    row, rowabs, col, colabs = oracle.checksums(A, B, lib=lib)
    Pe, Se = exact_product(A, B)
    for i in range(7):
        e, ea = sum(Pe[i]), sum(Se[i])
        if abs(Fraction(float(row[i])) - e) > 64 * Fraction(TWO_M53) * ea:
            return f"row checksum {i} off"
        if abs(Fraction(float(rowabs[i])) - ea) > 64 * Fraction(TWO_M53) * ea:
            return f"row abs checksum {i} off"
    for j in range(5):
        e = sum(Pe[i][j] for i in range(7))
        ea = sum(Se[i][j] for i in range(7))
        if abs(Fraction(float(col[j])) - e) > 64 * Fraction(TWO_M53) * ea:
            return f"column checksum {j} off"
        if abs(Fraction(float(colabs[j])) - ea) > 64 * Fraction(TWO_M53) * ea:
            return f"column abs checksum {j} off"
    return None


def pin_empty(lib):
    """K = 0 gives +0 everywhere (empty sum); M = 0 or N = 0 gives empty results."""
    P, S = oracle.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32), lib=lib)
    if P.shape != (3, 4) or np.any(P != 0) or np.any(np.signbit(P)) or np.any(S != 0):
        return "K = 0 is not +0"
    if oracle.gemm(np.zeros((0, 5), np.float32), np.ones((5, 2), np.float32), lib=lib)[0].shape != (0, 2):
        return "M = 0 shape"
    if oracle.gemm_fma_f32(np.ones((2, 0), np.float32), np.ones((0, 3), np.float32), lib=lib).shape != (2, 3):
        return "fma K = 0 shape"
    return None


# ---------------------------------------------------------------- transpose

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TRANSPOSE_SHAPES = [(1, 1), (1, 17), (17, 1), (3, 4), (33, 65), (64, 64), (100, 7)]


def _bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def pin_transpose_golden(lib):
    """The hand-written 3x4 example of tests/golden/transpose_3x4.txt (page 2 §1.4)."""
    rows = {"in": [], "out": []}
    with open(os.path.join(GOLDEN, "transpose_3x4.txt")) as f:
        for line in f:
            parts = line.split()
            if parts and parts[0] in rows:
                rows[parts[0]].append([float(v) for v in parts[1:]])
    A = np.array(rows["in"], np.float32)
    want = np.array(rows["out"], np.float32)
    if not np.array_equal(_bits(oracle.transpose(A, lib=lib)), _bits(want)):
        return "golden 3x4 transpose differs (bitwise)"
    return None


def pin_transpose_closed_form(lib):
    """A(i, j) = i·N + j (exact in float32): the output at (j, i) must hold i·N + j."""
    for M, N in TRANSPOSE_SHAPES + [(0, 5), (5, 0)]:
        A = (np.arange(M)[:, None] * N + np.arange(N)[None, :]).astype(np.float32)
        B = oracle.transpose(A, lib=lib)
        want = (np.arange(M)[None, :] * N + np.arange(N)[:, None]).astype(np.float32)
        if B.shape != (N, M) or not np.array_equal(B, want):
            return f"closed form fails at {M}x{N}"
    return None


def pin_transpose_library_and_bits(lib):
    """Equal, bit for bit, to numpy's own transpose copy, on values that include
    NaNs with payloads, ±0, ±inf and subnormals; applying it twice gives A back."""
    rng = np.random.default_rng(44)
    for M, N in TRANSPOSE_SHAPES:
        words = rng.integers(0, 2 ** 32, size=(M, N), dtype=np.uint64).astype(np.uint32)
        special = np.array([0x7FC01234, 0xFFA00001, 0x80000000, 0x00000000, 0x7F800000,
                            0xFF800000, 0x00000001, 0x807FFFFF], np.uint32)
        flat = words.reshape(-1)
        flat[: min(flat.size, special.size)] = special[: flat.size]
        A = words.view(np.float32)
        B = oracle.transpose(A, lib=lib)
        if not np.array_equal(_bits(B), np.ascontiguousarray(words.T)):
            return f"differs from numpy's transpose at {M}x{N}"
        if not np.array_equal(_bits(oracle.transpose(B, lib=lib)), words):
            return f"twice is not the identity at {M}x{N}"
    return None


def pin_transpose_strides(lib):
    """Leading dimensions wider than the rows: padding of A is never read (NaN
    there would not show, so it holds values that would) and padding of B is
    never written."""
    lib_ = lib or oracle._load()
    for M, N, pa, pb in [(3, 4, 3, 5), (17, 1, 2, 1), (1, 9, 0, 4), (20, 30, 7, 2)]:
        lda, ldb = N + pa, M + pb
        Abuf = np.full((M, lda), 7.0, np.float32)
        Abuf[:, :N] = (np.arange(M)[:, None] * N + np.arange(N)[None, :])
        Bbuf = np.full((N, ldb), -3.0, np.float32)
        rc = lib_.oracle_transpose(M, N, Abuf.view(np.uint32), lda, Bbuf.view(np.uint32), ldb)
        if rc != 0:
            return f"rejected lda={lda}, ldb={ldb}"
        if not np.array_equal(Bbuf[:, :M], Abuf[:, :N].T):
            return f"wrong values with lda={lda}, ldb={ldb}"
        if np.any(Bbuf[:, M:] != -3.0):
            return f"wrote B's padding with ldb={ldb}"
    return None


ALL_PINS = [pin_bruteforce_rational, pin_integer_paths, pin_identities, pin_one_hot,
            pin_transpose, pin_closed_forms, pin_worked_example, pin_window, pin_leading_dimensions,
            pin_fma_model,
            pin_checksums, pin_empty, pin_transpose_golden, pin_transpose_closed_form,
            pin_transpose_library_and_bits, pin_transpose_strides]


def run_all(lib=None):
    """{pin name: failure message or None}."""
    out = {}
    for pin in ALL_PINS:
        try:
            out[pin.__name__] = pin(lib)
        except Exception as exc:  # a planted mistake may also make a call fail
            out[pin.__name__] = f"raised {type(exc).__name__}: {exc}"
    return out
