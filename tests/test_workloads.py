"""The seeded input generator: deterministic, right shapes, right value sets."""

import numpy as np
import pytest

from tiled_gemm_tgemm_amd import workloads as wl


def test_five_workloads_shapes():
    shapes = {w.name: (w.M, w.N, w.K, w.dist, w.seed) for w in wl.WORKLOADS.values()}
    assert shapes == {
        "square512_uniform": (512, 512, 512, "uniform", 0),
        "square1024_int4": (1024, 1024, 1024, "int4", 1),
        "square4096_uniform": (4096, 4096, 4096, "uniform", 2),
        "rect3000x1000x5000_normal": (3000, 5000, 1000, "normal", 3),
        "square8192_uniform": (8192, 8192, 8192, "uniform", 4),
    }


def test_deterministic_and_seed_sensitive():
    a1, b1, _ = wl.random_matrices(40, 30, 20, "uniform", 9)
    a2, b2, _ = wl.random_matrices(40, 30, 20, "uniform", 9)
    a3, _, _ = wl.random_matrices(40, 30, 20, "uniform", 10)
    assert a1.tobytes() == a2.tobytes() and b1.tobytes() == b2.tobytes()
    assert a1.tobytes() != a3.tobytes()
    assert a1.dtype == np.float32 and a1.shape == (40, 20) and b1.shape == (20, 30)
    assert a1.flags.c_contiguous and b1.flags.c_contiguous


def test_value_laws():
    a, b, _ = wl.random_matrices(300, 300, 300, "int4", 1)
    vals = set(np.unique(np.concatenate([a.ravel(), b.ravel()])).tolist())
    assert vals == set(float(v) for v in range(-4, 5))
    a, b, _ = wl.random_matrices(300, 300, 300, "uniform", 0)
    assert a.min() >= -1 and a.max() <= 1 and abs(float(a.mean())) < 0.01
    a, b, _ = wl.random_matrices(300, 300, 300, "normal", 3)
    assert abs(float(a.mean())) < 0.01 and abs(float(a.std()) - 1) < 0.01
    with pytest.raises(ValueError):
        wl.random_matrices(2, 2, 2, "cauchy", 0)


def test_workload_inputs_first_values_stable():
    """The first rows come straight from PCG64 with these seeds; a change in
    the draw order (A before B) or the law would move them."""
    w = wl.WORKLOADS["square512_uniform"]
    A, B = wl.make_inputs(w)
    A2, B2, _ = wl.random_matrices(512, 512, 512, "uniform", 0)
    assert np.array_equal(A, A2) and np.array_equal(B, B2)
    rng = np.random.default_rng(0)
    first = rng.uniform(-1, 1, size=(512, 512)).astype(np.float32)
    assert np.array_equal(A, first)


def test_sampled_blocks():
    w = wl.Workload("t", 512, 1024, 64, "uniform", 4)
    blocks = wl.sample_blocks(w, count=64, size=64)
    assert len(blocks) == 64 and len(set(blocks)) == 64
    assert all(r % 64 == 0 and c % 64 == 0 and 0 <= r < 512 and 0 <= c < 1024 for r, c in blocks)
    assert blocks == wl.sample_blocks(w, count=64, size=64)
    _, _, blocks2 = wl.make_inputs_and_blocks(w)
    assert blocks2 == blocks
    with pytest.raises(ValueError):
        wl.sample_blocks(wl.Workload("r", 100, 64, 8, "uniform", 0))


def test_transpose_workloads():
    ws = wl.TRANSPOSE_WORKLOADS
    assert [(w.M, w.N) for w in ws.values()] == [(1024, 1024), (16384, 16384), (3001, 5003)]
    assert ws["transpose16384_uniform"].algorithmic_bytes == 2 * 4 * 16384 ** 2
    a = wl.random_matrix(300, 200, 10)
    assert a.dtype == np.float32 and a.shape == (300, 200)
    assert np.array_equal(a, wl.random_matrix(300, 200, 10))
    assert not np.array_equal(a, wl.random_matrix(300, 200, 11))
    assert a.min() >= -1.0 and a.max() < 1.0
    # on the 2^-23 grid (2x - 1 of a float32 multiple of 2^-24 is exact)
    assert np.array_equal(a * np.float32(2 ** 23), np.round(a * np.float32(2 ** 23)))
    assert len(np.unique(a)) > 0.99 * a.size
