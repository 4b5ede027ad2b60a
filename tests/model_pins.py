"""Pins of the step-by-step models in oracle/models.py: checks that tie
them to the pages' own facts and to the pinned product oracle.

Fixtures under tests/golden/ hold what the pages print (with citations):
the 4x4 / TILE_WIDTH=2 worked example of page 1, the load counts of page 2
§1.2, the bank rules of page 2 §1.3-1.4 and the transpose's bursts and
conflicts of page 2 §1.4.  Each pin takes the models module as its argument
and raises when it does not hold, so the same battery runs on the real
models (every pin must hold, tests/test_models.py) and on copies with a
planted mistake (some pin must fail, tests/test_model_mutants.py).
"""

import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def _pair(s):
    a, b = s.split(",")
    return int(a), int(b)


def worked_example_inputs():
    Mx = [[4 * i + k + 1 for k in range(4)] for i in range(4)]
    Nx = [[4 * k + j + 1 for j in range(4)] for k in range(4)]
    return Mx, Nx


def pin_index_map(models):
    tm = models.thread_map(4, 2)
    assert len(tm) == 4 and all(len(c) == 4 for c in tm.values())
    seen = 0
    for parts in _lines("worked_example_4x4_tile2.txt"):
        if parts[0] != "block":
            continue
        by, bx = int(parts[1]), int(parts[2])
        assert sorted(tm[(bx, by)]) == sorted(_pair(p) for p in parts[3:])
        seen += 1
    assert seen == 2
    # every output is computed exactly once
    cells = [c for cs in tm.values() for c in cs]
    assert sorted(cells) == [(i, j) for i in range(4) for j in range(4)]


def pin_phase_terms(models):
    Mx, Nx = worked_example_inputs()
    run = models.tiled_run(Mx, Nx, 2)
    n_terms = 0
    for parts in _lines("worked_example_4x4_tile2.txt"):
        if parts[0] != "term":
            continue
        cell, phase = _pair(parts[1]), int(parts[2]) - 1
        want = []
        for t in parts[3:]:
            m_idx, n_idx = t.split(";")
            want.append((*_pair(m_idx), *_pair(n_idx)))
        assert run["terms"][cell][phase] == want
        # the number the page's symbolic sum stands for, from the inputs
        value = sum(Fraction(Mx[i][k] * Nx[k2][j]) for i, k, k2, j in want)
        assert run["partial"][cell][phase] == value
        n_terms += 1
    assert n_terms == 8
    # Block(0,0)'s per-phase partial sums with these inputs
    assert [run["partial"][(0, 0)][p] for p in (0, 1)] == [11, 79]
    assert [run["partial"][(0, 1)][p] for p in (0, 1)] == [14, 86]
    assert [run["partial"][(1, 0)][p] for p in (0, 1)] == [35, 167]
    assert [run["partial"][(1, 1)][p] for p in (0, 1)] == [46, 182]


def pin_tiled_equals_oracle(models):
    """Tiling regroups the products but sums the same ones: exact equality
    in rationals with the oracle on integer inputs, for several tiles."""
    Mx, Nx = worked_example_inputs()
    run = models.tiled_run(Mx, Nx, 2)
    P, _ = oracle.gemm(np.array(Mx, np.float32), np.array(Nx, np.float32))
    assert np.array_equal(np.array([[float(v) for v in r] for r in run["P"]]), P)
    rng = np.random.default_rng(3)
    for width, tile in [(8, 2), (8, 4), (12, 3), (16, 8)]:
        A = rng.integers(-4, 5, (width, width)).astype(np.float32)
        B = rng.integers(-4, 5, (width, width)).astype(np.float32)
        run = models.tiled_run(A.tolist(), B.tolist(), tile)
        naive, _, _ = models.naive_run(A.tolist(), B.tolist(), tile)
        P, _ = oracle.gemm(A, B)
        got = np.array([[float(v) for v in r] for r in run["P"]])
        assert np.array_equal(got, P)
        assert np.array_equal(np.array([[float(v) for v in r] for r in naive]), P)


def pin_load_counts(models):
    Mx, Nx = worked_example_inputs()
    for parts in _lines("load_counts.txt"):
        kind = parts[0]
        if kind == "naive_column_reads_per_block":
            width, tile, want = map(int, parts[1:])
            _, _, by_block = models.naive_run([[1] * width] * width, [[1] * width] * width, tile)
            for (bx, by), cnt in by_block.items():
                for k in range(width):
                    for j in range(bx * tile, bx * tile + tile):
                        assert cnt[("N", k, j)] == want
        elif kind == "naive_column_reads_total":
            width, tile, want = map(int, parts[1:])
            _, loads, _ = models.naive_run([[1] * width] * width, [[1] * width] * width, tile)
            assert all(loads[("N", k, j)] == want for k in range(width) for j in range(width))
        elif kind == "total_reads":
            name, n, b, formula = parts[1], int(parts[2]), int(parts[3]), parts[4]
            ones = [[1] * n] * n
            if name == "naive":
                _, loads, _ = models.naive_run(ones, ones, b)
            else:
                loads = models.tiled_run(ones, ones, b)["loads"]
            assert sum(loads.values()) == eval(formula, {"n": n, "b": b})
        elif kind == "per_matrix_reads":
            _, n, b, formula = parts[0], int(parts[2]), int(parts[3]), parts[4]
            ones = [[1] * n] * n
            loads = models.tiled_run(ones, ones, b)["loads"]
            assert sum(v for key, v in loads.items() if key[0] == "M") == eval(formula, {"n": n, "b": b})
            assert sum(v for key, v in loads.items() if key[0] == "N") == eval(formula, {"n": n, "b": b})
        elif kind == "reduction":
            b = int(parts[1])
            # the ratio of the two formulas, at a width divisible by b
            n = 2 * b
            assert Fraction(2 * n ** 2 * (n // b), 2 * n ** 3) == Fraction(parts[2])
        else:
            raise AssertionError(f"unknown fixture line {parts}")


def pin_bank_model(models):
    for parts in _lines("bank_model.txt"):
        if parts[0] == "case":
            banks, want = int(parts[2]), int(parts[3])
            words = [int(w) for w in parts[4:]]
            assert models.conflict_degree(words, banks) == want, parts[1]
        elif parts[0] == "column":
            name, banks, want, col = parts[1], int(parts[2]), int(parts[3]), int(parts[4])
            width = int(name.split("x")[1])
            words = [r * width + col for r in range(32)]
            assert models.conflict_degree(words, banks) == want, name
    # a 32-way conflict means 31 replays
    assert models.conflict_degree([r * 32 for r in range(32)], 32) - 1 == 31


def pin_transpose_models(models):
    """The page's transpose kernels, thread by thread: both produce the
    transpose (equal to the oracle's), and their per-warp DRAM bursts and
    shared-memory conflicts are the page's (tests/golden/transpose_coalescing.txt)."""
    M, N = 64, 96  # several tiles each way, not square
    for parts in _lines("transpose_coalescing.txt"):
        assert parts[0] == "kernel"
        kind, pad, rd, wr, conflict = parts[1], int(parts[2]), int(parts[3]), int(parts[4]), int(parts[5])
        run = models.transpose_run(M, N, kind, pad=pad)
        A = np.array(run["A"], np.float32)
        assert np.array_equal(np.array(run["B"], np.float32), oracle.transpose(A)), kind
        assert {models.bursts(a) for a in run["reads"]} == {rd}, (kind, pad, "reads")
        assert {models.bursts(a) for a in run["writes"]} == {wr}, (kind, pad, "writes")
        worst = max((models.conflict_degree(w, 32) for w in run["lds_reads"]), default=0)
        assert worst == conflict, (kind, pad, "shared-memory reads")
        # every element read once and written once
        assert sum(len(a) for a in run["reads"]) == M * N == sum(len(a) for a in run["writes"])


PINS = [pin_index_map, pin_phase_terms, pin_tiled_equals_oracle, pin_load_counts, pin_bank_model,
        pin_transpose_models]


def run_all(models):
    """{pin name: None if it holds, else what failed}"""
    out = {}
    for pin in PINS:
        try:
            pin(models)
            out[pin.__name__] = None
        except Exception as e:  # a pin that raises, for whatever reason, does not hold
            out[pin.__name__] = f"{type(e).__name__}: {e}"
    return out
