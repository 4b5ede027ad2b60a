"""Seeded synthetic input matrices for C = A·B and for the transpose.

This module draws numbers and nothing else: it holds none of the product's
arithmetic, so both the HIP path (bench, parity tests) and the CPU oracle can
take their inputs from it without sharing any computation.

The pages (page 1, "CUDA - Matrix Multiplication", section [Matrix
Multiplication] and "Kernel 호출"; page 2, "Lec 29 · GPU Architecture (2)",
§1.2) work on square Width×Width matrices with no data set attached, so every
workload here is a synthetic stand-in of that shape family:

* generator: ``numpy.random.default_rng(seed)`` (PCG64); A (M×K, row-major) is
  drawn first, then B (K×N), both as float64 and rounded to float32;
* ``uniform``: i.i.d. U[-1, 1); ``int4``: i.i.d. integers in {-4, ..., 4},
  inclusive, equally likely; ``normal``: i.i.d. standard normal;
* sampled output blocks (for the largest square case) are drawn from the same
  generator, continued after B, without replacement, on a grid aligned to the
  block size.

The transpose of page 2 §1.4 is studied there on a 1024×1024 matrix; its
workloads are that shape, one large enough that input and output (1 GiB
each) stream from HBM rather than the last-level cache, and a ragged one.
Their values are ``numpy.random.default_rng(seed).random(dtype=float32)``
mapped to [-1, 1) (2x - 1, exact in float32): a transpose only moves words,
so the value law matters only in that every word is distinct in practice.
"""

from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str  # "uniform" | "int4" | "normal"
    seed: int

    @property
    def flops(self) -> int:
        """Multiply-adds counted as two operations: 2·M·N·K."""
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes a GEMM must move at least once: read A and B, write C."""
        return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)


# The five synthetic workloads, named by their shapes and value law.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("square512_uniform", 512, 512, 512, "uniform", 0),
        Workload("square1024_int4", 1024, 1024, 1024, "int4", 1),
        Workload("square4096_uniform", 4096, 4096, 4096, "uniform", 2),
        # M×K = 3000×1000 times K×N = 1000×5000: no side is a tile multiple.
        Workload("rect3000x1000x5000_normal", 3000, 5000, 1000, "normal", 3),
        Workload("square8192_uniform", 8192, 8192, 8192, "uniform", 4),
    )
}


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "int4":
        x = rng.integers(-4, 5, size=shape).astype(np.float64)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    else:
        raise ValueError(f"unknown value law {dist!r}")
    return np.ascontiguousarray(x.astype(np.float32))


def random_matrices(M: int, N: int, K: int, dist: str, seed: int):
    """Return (A, B, rng): A is M×K, B is K×N, float32 row-major.

    The generator is returned in the state just after B was drawn, so that a
    caller can continue the same stream (block sampling does).
    """
    rng = np.random.default_rng(seed)
    A = _draw(rng, dist, (M, K))
    B = _draw(rng, dist, (K, N))
    return A, B, rng


def make_inputs(w: Workload):
    """(A, B) for a named workload."""
    A, B, _ = random_matrices(w.M, w.N, w.K, w.dist, w.seed)
    return A, B


def sample_blocks(w: Workload, count: int = 64, size: int = 64, rng=None):
    """Origins (row0, col0) of `count` distinct size×size output blocks.

    Blocks lie on a grid aligned to `size`; the grid index is drawn without
    replacement from the workload's generator continued after B (so the same
    seed always gives the same blocks).  Requires M and N to be multiples of
    `size`.
    """
    if w.M % size or w.N % size:
        raise ValueError("block sampling needs M and N multiples of the block size")
    if rng is None:
        _, _, rng = random_matrices(w.M, w.N, w.K, w.dist, w.seed)
    grid_cols = w.N // size
    n_blocks = (w.M // size) * grid_cols
    picks = rng.choice(n_blocks, size=count, replace=False)
    return [(int(p // grid_cols) * size, int(p % grid_cols) * size) for p in picks]


def make_inputs_and_blocks(w: Workload, count: int = 64, size: int = 64):
    """(A, B, blocks) in one pass over the generator."""
    A, B, rng = random_matrices(w.M, w.N, w.K, w.dist, w.seed)
    return A, B, sample_blocks(w, count, size, rng)


@dataclasses.dataclass(frozen=True)
class TransposeWorkload:
    name: str
    M: int  # input rows (output columns)
    N: int  # input columns (output rows)
    seed: int

    @property
    def algorithmic_bytes(self) -> int:
        """Every element read once and written once: 2·4·M·N."""
        return 8 * self.M * self.N


TRANSPOSE_WORKLOADS = {
    w.name: w
    for w in (
        TransposeWorkload("transpose1024_uniform", 1024, 1024, 10),
        TransposeWorkload("transpose16384_uniform", 16384, 16384, 11),
        # neither side a multiple of any tile; M·N about 15 M elements
        TransposeWorkload("transpose3001x5003_uniform", 3001, 5003, 12),
    )
}


def random_matrix(M: int, N: int, seed: int) -> np.ndarray:
    """M×N float32, i.i.d. on the grid of multiples of 2^-23 in [-1, 1)."""
    rng = np.random.default_rng(seed)
    x = rng.random((M, N), dtype=np.float32)
    x *= np.float32(2.0)
    x -= np.float32(1.0)
    return x


def make_transpose_input(w: TransposeWorkload) -> np.ndarray:
    return random_matrix(w.M, w.N, w.seed)
