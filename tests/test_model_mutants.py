"""Plant one plausible mistake at a time in a copy of oracle/models.py (on the
CPU) and check that at least one model pin catches it: outputs mapped to the
wrong thread, a phase or a product term dropped, a tile filled from the
wrong row, a global read miscounted, the bank rule without broadcast or with
the wrong bank index, bursts counted in the wrong unit, and transposes that
ignore the padding, leave the block offsets unswapped or write to the wrong
address must each fail something."""

import importlib.util

import pytest

from oracle import models

import model_pins

MUTANTS = {
    "thread_map_row_col_swapped": ("col = bx * tile + tx\n                    row = by * tile + ty",
                                   "col = by * tile + ty\n                    row = bx * tile + tx"),
    "naive_drops_last_k": ("for k in range(width):\n                m = M[row][k]",
                           "for k in range(width - 1):\n                m = M[row][k]"),
    "naive_block_tally_transposed": ('by_block[(bx, by)][("N", k, col)] += 1',
                                     'by_block[(by, bx)][("N", k, col)] += 1'),
    "tiled_n_tile_from_wrong_row": ("sub_n[ty][tx] = (m * tile + ty, col, N[m * tile + ty][col])",
                                    "sub_n[ty][tx] = (m * tile + tx, col, N[m * tile + tx][col])"),
    "tiled_last_phase_dropped": ("for m in range(phases):", "for m in range(phases - 1):"),
    "tiled_reads_n_tile_transposed": ("nk, nj, nv = sub_n[k][tx]", "nk, nj, nv = sub_n[tx][k]"),
    "tiled_m_reads_counted_twice": ('loads[("M", row, m * tile + tx)] += 1', 'loads[("M", row, m * tile + tx)] += 2'),
    "bank_without_broadcast": ("per_bank[w % nbanks].add(w)", "per_bank[w % nbanks].add((w, len(per_bank[w % nbanks])))"),
    "bank_index_divides": ("per_bank[w % nbanks].add(w)", "per_bank[w // nbanks].add(w)"),
    "bursts_counted_in_words": ("return len({a // burst_bytes for a in byte_addresses})",
                                "return len({a // (4 * burst_bytes) for a in byte_addresses})"),
    "transpose_pad_ignored_on_read": ("word = tx * (tile + pad) + ty + j", "word = tx * tile + ty + j"),
    "transpose_offsets_not_swapped": ("r, c = x0 + ty + j, y0 + tx", "r, c = y0 + ty + j, x0 + tx"),
    "transpose_naive_write_address": ("wr.append(4 * (x * M + y))", "wr.append(4 * (y * M + x))"),
}


def load_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(models.__file__).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"models_{name}.py"
    path.write_text(src.replace(before, after))
    spec = importlib.util.spec_from_file_location(f"models_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_real_models_hold_every_pin():
    assert not any(model_pins.run_all(models).values())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_model_pins_catch_mutant(name, tmp_path):
    failures = {k: v for k, v in model_pins.run_all(load_mutant(name, tmp_path)).items() if v}
    assert failures, f"no model pin caught the planted mistake {name}"
