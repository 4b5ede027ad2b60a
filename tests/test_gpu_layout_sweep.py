"""Seeded sweep over operand layouts (GPU): shapes, storage orders, leading
dimensions and base alignments drawn at random, every entry point that takes
them, exact integer results.

What is computed is page 1's product ("[Multi-Core & GPU Programming] CUDA -
Matrix Multiplication", section [Matrix Multiplication]); with integer inputs
whose partial sums stay below 2^24 every order of summation gives the exact
product, so each result must equal the oracle's int64 product bit for bit.

Each case stores A and B (as stored or transposed) inside larger buffers:
the operand starts 0-3 floats past a 256-byte boundary, rows are padded by a
few floats, and every float of the buffer that is not an operand element
(padding between rows, before and after) is NaN, so a read that strays
outside the operand and reaches C shows as a non-finite or wrong output.  C
lives in a buffer of sentinels laid out the same way; after the call only
its M×N window may have changed.  The draws are seeded, so the cases are
the same on every run.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import tiled_gemm_tgemm_amd as tg
from tiled_gemm_tgemm_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = np.float32(-1.25e30)
CASES = 40


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    tg.library()
    yield


def draw_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(CASES):
        if i % 2 == 0:
            # small and degenerate: sizes log-uniform in [1, 640]
            M, N, K = (int(round(np.exp(rng.uniform(0.0, np.log(640.0))))) for _ in range(3))
        else:
            # several tiles with ragged tails: sizes uniform in [100, 700]
            M, N, K = (int(rng.integers(100, 701)) for _ in range(3))
        if i % 10 == 9:
            which = int(rng.integers(3))
            M, N, K = [1 if j == which else v for j, v in enumerate((M, N, K))]
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        pads = [int(rng.choice([0, 0, 1, 3, 4, 8])) for _ in range(3)]
        offs = [int(rng.choice([0, 0, 1, 2, 3])) for _ in range(3)]
        if i % 4 == 3:
            # operands that the 16-byte-load configurations take: sizes, leading
            # dimensions and bases in whole float4s
            M, N, K = (-(-v // 4) * 4 for v in (M, N, K))
            pads = [p - p % 4 for p in pads]
            offs = [0, 0, offs[2]]
        cases.append((i, M, N, K, ta, tb, pads, offs))
    return cases


class Stored:
    """A rows×cols matrix X kept at float offset `off` of a device buffer,
    rows `ld` floats apart, every other float of the buffer `fill`."""

    def __init__(self, X, off, pad, fill):
        rows, cols = X.shape
        self.ld = max(cols + pad, 1)
        self.off = off
        size = off + rows * self.ld + 64
        host = np.full(size, fill, dtype=np.float32)
        view = host[off:off + rows * self.ld].reshape(rows, self.ld)
        view[:, :cols] = X
        self.host = host
        self.rows, self.cols = rows, cols
        self.buf = torch.from_numpy(host).cuda()

    @property
    def ptr(self):
        return self.buf.data_ptr() + 4 * self.off

    def window(self):
        """(values of the matrix window, copy of the buffer with the window cleared)"""
        got = self.buf.cpu().numpy()
        view = got[self.off:self.off + self.rows * self.ld].reshape(self.rows, self.ld)
        win = view[:, :self.cols].copy()
        rest = got.copy()
        rest[self.off:self.off + self.rows * self.ld].reshape(self.rows, self.ld)[:, :self.cols] = SENTINEL
        return win, rest


def entry_points(M, N, K, ta, tb):
    """(label, callable(op_a, op_b, A, lda, B, ldb, C, ldc, stream) -> status) for every entry point
    that takes this storage order."""
    calls = [("auto", lambda oa, ob, a, la, b, lb, c, lc, s: tg.tgemm_sgemm_ex(oa, ob, M, N, K, a, la, b, lb, c,
                                                                              lc, s))]
    for v, name in enumerate(tg.variant_names()):
        calls.append((name, lambda oa, ob, a, la, b, lb, c, lc, s, v=v: tg.tgemm_sgemm_mfma_ex(
            oa, ob, M, N, K, a, la, b, lb, c, lc, v, s)))
    if not ta and not tb:
        calls += [
            ("naive", lambda oa, ob, a, la, b, lb, c, lc, s: tg.tgemm_sgemm_naive(M, N, K, a, la, b, lb, c, lc, s)),
            ("lds16p1", lambda oa, ob, a, la, b, lb, c, lc, s: tg.tgemm_sgemm_lds(M, N, K, a, la, b, lb, c, lc,
                                                                                  16, 1, s)),
            ("lds32p0", lambda oa, ob, a, la, b, lb, c, lc, s: tg.tgemm_sgemm_lds(M, N, K, a, la, b, lb, c, lc,
                                                                                  32, 0, s)),
            ("simt", lambda oa, ob, a, la, b, lb, c, lc, s: tg.tgemm_sgemm_simt(M, N, K, a, la, b, lb, c, lc, s)),
        ]
    return calls


@pytest.mark.parametrize("case", draw_cases(), ids=lambda c: f"c{c[0]}_{c[1]}x{c[2]}x{c[3]}_"
                         f"{'T' if c[4] else 'N'}{'T' if c[5] else 'N'}")
def test_layout_sweep_integer_exact(case):
    i, M, N, K, ta, tb, pads, offs = case
    log(f"layout case {i}: M={M} N={N} K={K} ta={ta} tb={tb} pads={pads} offsets={offs}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 100 + i)
    want = oracle.gemm_i64(A, B).astype(np.float64)
    sa = Stored(A.T if ta else A, offs[0], pads[0], np.nan)
    sb = Stored(B.T if tb else B, offs[1], pads[1], np.nan)
    op_a = tg.TGEMM_OP_T if ta else tg.TGEMM_OP_N
    op_b = tg.TGEMM_OP_T if tb else tg.TGEMM_OP_N
    stream = torch.cuda.current_stream().cuda_stream
    ran = []
    for label, call in entry_points(M, N, K, ta, tb):
        sc = Stored(np.zeros((M, N), np.float32), offs[2], pads[2], SENTINEL)
        sc.buf.fill_(float(SENTINEL))
        st = call(op_a, op_b, sa.ptr, sa.ld, sb.ptr, sb.ld, sc.ptr, sc.ld, stream)
        if st == tg.TGEMM_ERROR_NOT_SUPPORTED and label != "auto":
            continue  # this configuration does not take these operands (alignment, order)
        assert st == tg.TGEMM_SUCCESS, f"{label}: status {tg.tgemm_status_string(st)}"
        torch.cuda.synchronize()
        got, rest = sc.window()
        bad = got.astype(np.float64) != want
        if bad.any():
            r, c = np.argwhere(bad)[0]
            pytest.fail(f"case {i} {label}: {bad.sum()} elements differ; first ({r},{c}) {got[r, c]} vs "
                        f"{want[r, c]}")
        assert np.all(rest == SENTINEL), f"case {i} {label}: C written outside its window"
        ran.append(label)
    # every 4-byte-load configuration takes any layout (the operand-as-stored
    # ones only as stored); 16-byte-load ones need whole float4s
    trans = ta or tb
    must = {"auto"} | {n for n in tg.variant_names()
                       if n.endswith("_vec1") or (n.endswith("_vec1_flat") and not trans)}
    if not trans:
        must |= {"naive", "lds16p1", "lds32p0", "simt"}
    whole4 = (offs[0] == 0 and offs[1] == 0 and pads[0] % 4 == 0 and pads[1] % 4 == 0
              and (M if ta else K) % 4 == 0 and (K if tb else N) % 4 == 0)
    if whole4:
        must |= {n for n in tg.variant_names() if "_vec4" in n and not (trans and n.endswith(("_nn", "_flat")))}
    missing = must - set(ran)
    assert not missing, f"case {i}: refused by {sorted(missing)}"
    log(f"  exact through {len(ran)} entry points")


@pytest.mark.parametrize("case", draw_cases()[:12], ids=lambda c: f"c{c[0]}")
def test_layout_sweep_splitk_integer_exact(case):
    i, M, N, K, ta, tb, pads, offs = case
    splits = 2 + i % 3
    log(f"layout split-K case {i}: M={M} N={N} K={K} ta={ta} tb={tb} splits={splits}")
    A, B, _ = wl.random_matrices(M, N, K, "int4", 100 + i)
    want = oracle.gemm_i64(A, B).astype(np.float64)
    sa = Stored(A.T if ta else A, offs[0], pads[0], np.nan)
    sb = Stored(B.T if tb else B, offs[1], pads[1], np.nan)
    sc = Stored(np.zeros((M, N), np.float32), offs[2], pads[2], SENTINEL)
    sc.buf.fill_(float(SENTINEL))
    need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = tg.tgemm_sgemm_splitk_ex(tg.TGEMM_OP_T if ta else tg.TGEMM_OP_N, tg.TGEMM_OP_T if tb else tg.TGEMM_OP_N,
                                  M, N, K, sa.ptr, sa.ld, sb.ptr, sb.ld, sc.ptr, sc.ld, splits, ws.data_ptr(), need,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == tg.TGEMM_SUCCESS, tg.tgemm_status_string(st)
    torch.cuda.synchronize()
    got, rest = sc.window()
    assert np.array_equal(got.astype(np.float64), want), f"case {i}: split-K result differs"
    assert np.all(rest == SENTINEL), f"case {i}: split-K wrote C outside its window"


def scaled_inputs(M, N, K, seed):
    """Real inputs over a wide range: N(0,1) values with each row of A and
    each column of B scaled by 2^e, e uniform in [-12, 12] (exact in float32,
    no subnormal products), and for every third seed the second half of A's
    columns equal to the first half and the second half of B's rows the
    negated first half perturbed by about 2^-10, so that the sums cancel and
    C is about 2^-10 of S."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)) * np.exp2(rng.integers(-12, 13, (M, 1)))
    B = rng.standard_normal((K, N)) * np.exp2(rng.integers(-12, 13, (1, N)))
    if seed % 3 == 0 and K >= 2:
        h = K // 2
        A[:, h:2 * h] = A[:, :h]
        B[h:2 * h] = -B[:h] * (1.0 + np.exp2(-10) * rng.uniform(-1.0, 1.0, (h, N)))
    return A.astype(np.float32), B.astype(np.float32)


@pytest.mark.parametrize("case", draw_cases()[:20], ids=lambda c: f"c{c[0]}_{c[1]}x{c[2]}x{c[3]}")
def test_layout_sweep_real_within_bound(case):
    i, M, N, K, ta, tb, pads, offs = case
    log(f"layout real case {i}: M={M} N={N} K={K} ta={ta} tb={tb} pads={pads} offsets={offs}")
    A, B = scaled_inputs(M, N, K, 300 + i)
    P, S = oracle.gemm(A, B)
    bound = 4.0 * K * 2.0 ** -24 * S
    fma = oracle.gemm_fma_f32(A, B) if not (ta or tb) else None
    sa = Stored(A.T if ta else A, offs[0], pads[0], np.nan)
    sb = Stored(B.T if tb else B, offs[1], pads[1], np.nan)
    op_a = tg.TGEMM_OP_T if ta else tg.TGEMM_OP_N
    op_b = tg.TGEMM_OP_T if tb else tg.TGEMM_OP_N
    stream = torch.cuda.current_stream().cuda_stream
    ran = 0
    worst = 0.0
    for label, call in entry_points(M, N, K, ta, tb):
        sc = Stored(np.zeros((M, N), np.float32), offs[2], pads[2], SENTINEL)
        sc.buf.fill_(float(SENTINEL))
        st = call(op_a, op_b, sa.ptr, sa.ld, sb.ptr, sb.ld, sc.ptr, sc.ld, stream)
        if st == tg.TGEMM_ERROR_NOT_SUPPORTED and label != "auto":
            continue
        assert st == tg.TGEMM_SUCCESS, f"{label}: status {tg.tgemm_status_string(st)}"
        torch.cuda.synchronize()
        got, rest = sc.window()
        assert np.all(np.isfinite(got)), f"case {i} {label}: non-finite output"
        err = np.abs(got.astype(np.float64) - P)
        bad = err > bound
        if bad.any():
            r, c = np.argwhere(bad)[0]
            pytest.fail(f"case {i} {label}: {bad.sum()} elements outside the bound; first ({r},{c}) "
                        f"C={got[r, c]!r} P={P[r, c]!r} bound={bound[r, c]!r}")
        if label in ("naive", "lds16p1", "lds32p0", "simt"):
            # one fused multiply-add per k in ascending order: the oracle's float32 model bit for bit
            assert np.array_equal(got.view(np.uint32), fma.view(np.uint32)), f"case {i} {label}: differs from the FMA chain"
        assert np.all(rest == SENTINEL), f"case {i} {label}: C written outside its window"
        pos = S > 0
        if pos.any():
            worst = max(worst, float((err[pos] / (K * 2.0 ** -24 * S[pos])).max()))
        ran += 1
    log(f"  within the bound through {ran} entry points; worst ratio {worst:.4f} of K·2^-24·S")
