"""Step-by-step CPU models of the pages' two kernels and of their memory rules.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle``): nothing in the
GPU product path imports this.  Pure Python loops; meant for small inputs.

* ``thread_map``: which output each thread of each block computes, from the
  index formulas col = blockIdx.x·blockDim.x + threadIdx.x and
  row = blockIdx.y·blockDim.y + threadIdx.y (page 1, section
  [Matrix Multiplication], "Work Flow").
* ``naive_run``: the one-thread-per-output kernel (page 1, "가장 단순한 CUDA
  행렬 곱셈 Kernel"; page 2 §1.2): every thread reads its whole row of M and
  column of N from global memory.  Counts every global read.
* ``tiled_run``: the shared-memory tiled kernel (page 1, section
  [Shared Memory], "Work Flow - Compute Block(0, 0)" and "Tiled Matrix
  Multiplication Kernel"; page 2 §1.2): per phase every thread copies one M
  and one N element into the two tiles, all threads wait, then each adds the
  tile's products to its register sum, all threads wait again.  Records the
  terms each output adds in each phase and counts every global read.
* ``conflict_degree``: the shared-memory bank rule of page 2 §1.3 (banks of
  4-byte words, consecutive words in consecutive banks; several threads
  touching different words of one bank are serialised, the same word is a
  broadcast).
* ``transpose_run``: the transpose kernels of page 2 §1.4 (naive, and tiled
  through shared memory with optional padding), thread by thread, recording
  the addresses each warp instruction touches; ``bursts`` counts the DRAM
  burst sections such an instruction needs (page 2 §1.4, DRAM bursts).

All three kernels' models assume what the pages assume: square Width×Width
matrices with Width a multiple of the tile (page 1, "Kernel 호출").
"""

from __future__ import annotations

from collections import Counter, defaultdict
from fractions import Fraction


def thread_map(width: int, tile: int):
    """{(bx, by): [(row, col) for ty, tx]} for a width×width output, tile×tile blocks."""
    if width % tile:
        raise ValueError("the pages' launch assumes Width is a multiple of TILE_WIDTH")
    grid = width // tile
    out = {}
    for by in range(grid):
        for bx in range(grid):
            cells = []
            for ty in range(tile):
                for tx in range(tile):
                    col = bx * tile + tx
                    row = by * tile + ty
                    cells.append((row, col))
            out[(bx, by)] = cells
    return out


def naive_run(M, N, tile: int):
    """Run the naive kernel's arithmetic in exact rationals.

    Returns (P, loads) where P[i][j] is a Fraction and loads counts global
    reads per element: loads[("M", i, k)] and loads[("N", k, j)], together
    with per-block counts loads_by_block[(bx, by)][("N", k, j)].
    """
    width = len(M)
    P = [[Fraction(0)] * width for _ in range(width)]
    loads = Counter()
    by_block = defaultdict(Counter)
    for (bx, by), cells in thread_map(width, tile).items():
        for row, col in cells:
            value = Fraction(0)
            for k in range(width):
                m = M[row][k]
                n = N[k][col]
                loads[("M", row, k)] += 1
                loads[("N", k, col)] += 1
                by_block[(bx, by)][("M", row, k)] += 1
                by_block[(bx, by)][("N", k, col)] += 1
                value += Fraction(m) * Fraction(n)
            P[row][col] = value
    return P, loads, by_block


def tiled_run(M, N, tile: int):
    """Run the tiled kernel phase by phase in exact rationals.

    Returns a dict with
      P        -- final result, Fractions;
      terms    -- terms[(row, col)][phase] = list of (i, k, k2, j) index
                  quadruples meaning M(i,k)·N(k2,j) added in that phase;
      partial  -- partial[(row, col)][phase] = sum added in that phase;
      loads    -- Counter of global reads per element, as in naive_run;
      by_block -- per-block Counter of global reads.
    """
    width = len(M)
    if width % tile:
        raise ValueError("the pages' kernel assumes Width is a multiple of TILE_WIDTH")
    phases = width // tile
    P = [[Fraction(0)] * width for _ in range(width)]
    terms = defaultdict(lambda: defaultdict(list))
    partial = defaultdict(dict)
    loads = Counter()
    by_block = defaultdict(Counter)
    for (bx, by), cells in thread_map(width, tile).items():
        pvalue = {cell: Fraction(0) for cell in cells}
        for m in range(phases):
            # every thread of the block copies one M and one N element
            sub_m = [[None] * tile for _ in range(tile)]
            sub_n = [[None] * tile for _ in range(tile)]
            for ty in range(tile):
                for tx in range(tile):
                    row = by * tile + ty
                    col = bx * tile + tx
                    sub_m[ty][tx] = (row, m * tile + tx, M[row][m * tile + tx])
                    sub_n[ty][tx] = (m * tile + ty, col, N[m * tile + ty][col])
                    loads[("M", row, m * tile + tx)] += 1
                    loads[("N", m * tile + ty, col)] += 1
                    by_block[(bx, by)][("M", row, m * tile + tx)] += 1
                    by_block[(bx, by)][("N", m * tile + ty, col)] += 1
            # (first barrier: both tiles complete)
            for ty in range(tile):
                for tx in range(tile):
                    cell = (by * tile + ty, bx * tile + tx)
                    added = Fraction(0)
                    for k in range(tile):
                        mi, mk, mv = sub_m[ty][k]
                        nk, nj, nv = sub_n[k][tx]
                        terms[cell][m].append((mi, mk, nk, nj))
                        added += Fraction(mv) * Fraction(nv)
                    partial[cell][m] = added
                    pvalue[cell] += added
            # (second barrier: nobody still reads the tiles when they are refilled)
        for cell, v in pvalue.items():
            P[cell[0]][cell[1]] = v
    return {"P": P, "terms": terms, "partial": partial, "loads": loads, "by_block": by_block}


def conflict_degree(word_addresses, nbanks: int = 32) -> int:
    """Largest number of distinct words that one request maps to a single bank.

    `word_addresses` are the 4-byte word indices the threads of one request
    touch; word w lies in bank w mod nbanks.  Threads reading the same word
    count once (broadcast).  The request is served in that many passes, i.e.
    with degree − 1 replays; 1 means conflict-free.
    """
    per_bank = defaultdict(set)
    for w in word_addresses:
        per_bank[w % nbanks].add(w)
    return max((len(s) for s in per_bank.values()), default=0)


def bursts(byte_addresses, burst_bytes: int = 32) -> int:
    """Number of burst-aligned sections of `burst_bytes` that one warp
    instruction's accesses (4-byte words at these byte addresses) touch;
    a fully coalesced access of 32 words touches 128 / 32 = 4."""
    return len({a // burst_bytes for a in byte_addresses})


def transpose_run(M, N, kind: str, tile: int = 32, rows: int = 8, pad: int = 0, warp: int = 32):
    """Run a transpose kernel of page 2 §1.4 on an M×N matrix of distinct
    values, thread by thread.

    Blocks of tile×rows threads each own a tile×tile tile; thread (tx, ty)
    handles the elements of rows ty, ty + rows, ... of the tile (the page's
    loop over j).  "naive": read input (y, x), write output (x, y) directly.
    "tiled": read input (y, x) into tile[ty + j][tx]; all threads wait; with
    the block offsets swapped, write output row (x0 + ty + j), column
    (y0 + tx) from tile[tx][ty + j].  pad adds words to each tile row.

    Returns {"B": the output as nested lists, "reads"/"writes": one list of
    byte addresses per warp instruction (row-major, 4-byte elements, leading
    dimensions N and M), "lds_reads": one list of tile word indices per warp
    instruction that reads the tile}.  Assumes M, N multiples of tile.
    """
    assert kind in ("naive", "tiled") and M % tile == 0 and N % tile == 0 and tile % rows == 0
    A = [[i * N + j for j in range(N)] for i in range(M)]
    B = [[None] * M for _ in range(N)]
    reads, writes, lds_reads = [], [], []
    nthreads = tile * rows
    for by in range(M // tile):
        for bx in range(N // tile):
            x0, y0 = bx * tile, by * tile
            tile_words = {}
            for j in range(0, tile, rows):
                # one instruction per warp: threads t = ty*tile + tx, in warps of `warp`
                for w0 in range(0, nthreads, warp):
                    rd, wr = [], []
                    for t in range(w0, w0 + warp):
                        tx, ty = t % tile, t // tile
                        y, x = y0 + ty + j, x0 + tx
                        rd.append(4 * (y * N + x))
                        if kind == "naive":
                            B[x][y] = A[y][x]
                            wr.append(4 * (x * M + y))
                        else:
                            tile_words[(ty + j) * (tile + pad) + tx] = A[y][x]
                    reads.append(rd)
                    if wr:
                        writes.append(wr)
            if kind == "tiled":
                # (barrier) then the write-out, block offsets swapped
                for j in range(0, tile, rows):
                    for w0 in range(0, nthreads, warp):
                        wr, lr = [], []
                        for t in range(w0, w0 + warp):
                            tx, ty = t % tile, t // tile
                            word = tx * (tile + pad) + ty + j
                            r, c = x0 + ty + j, y0 + tx
                            B[r][c] = tile_words[word]
                            wr.append(4 * (r * M + c))
                            lr.append(word)
                        writes.append(wr)
                        lds_reads.append(lr)
    return {"A": A, "B": B, "reads": reads, "writes": writes, "lds_reads": lds_reads}
