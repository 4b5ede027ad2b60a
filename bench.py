#!/usr/bin/env python3
"""Benchmark of libtgemm's fp32 C = A·B on one MI355X; prints one JSON line.

A step is one call of the product (tgemm_sgemm) on seeded synthetic inputs
that are already resident in device memory.  Default workload: 8192³ with
U[-1,1] inputs (seed 4).  The other four workloads (512³, 1024³ integers,
4096³, 3000×1000×5000) are timed the same way and reported under "also",
each with its own step count (--small-steps for the launch-bound two,
--ragged-steps for the ragged one); the three smaller ones are timed again
with cold caches under "cold".

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
                  [--kernel auto|naive|lds16|lds32|simt|mfma:<variant>]
                  [--also NAME,...] [--no-cpu-baseline] [--copy-bytes N]
  python bench.py --transpose blocked|naive|tiled|tiled_padded [--workload NAME]
  python bench.py --host [--workload NAME] [--panel-rows R]
  python bench.py --shape MxNxK --kernel splitk[S] --also ''   (K split across work-groups)

With --transpose the line measures B = Aᵀ (tgemm_transpose) instead, default
workload 16384×16384: GB/s of algorithmic traffic (every element read once
and written once) against the 8 TB/s HBM peak, a device-to-device copy of the
same size timed beside it, and the oracle's transpose on the host.

With --host the line measures the product of operands in pinned HOST memory
(tgemm_sgemm_host: transfers overlapped with the computation), host to host,
against the same steps run one after the other on one stream.

Warm-up: at least --warmup calls and at least --warmup-seconds of back-to-back
calls (the GPU clock takes a few tens of milliseconds of load to settle).

Reported:
* value / ms_per_step — wall clock over the timed steps, between two device
  synchronisations, throughput = 2·M·N·K / time;
* roofline — the product kernel's average duration per launch, from one pair
  of HIP events recorded around the timed steps on the stream they are
  launched on, its algorithmic flops (2·M·N·K per launch) over that time,
  against the MI355X dense fp32 matrix peak (kernel_ms also gives the
  spread of single calls, each between its own events, from as many calls
  after the timed region); the
  measured HBM traffic per launch comes from the committed rocprofv3 counter
  summary when it was taken on the current kernel source, else null;
* engine_clock — the XCDs' mean engine clock read with amd-smi while the
  product runs (after the timed steps), and the kernel's fraction of the
  peak at that clock (CUs × 256 flops × clock); null without amd-smi;
* cpu_baseline — the CPU oracle (float64, test infrastructure) timed on this
  host's cores on a bounded sample: whole rows of the same product;
* vendor_blas — context only: torch.matmul in float32 with TF32 off (the ROCm
  BLAS library behind it) timed the same way on the same resident operands,
  with the largest difference from this library's output (--no-vendor skips it).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp32 GEMM TFLOPS + % of MI355X FP32 matrix peak at 4096³ and 8192³"
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# vector-ALU fp32 ceiling without packed instructions: 256 CUs × 4 SIMDs ×
# 16 lanes × 2 flops per FMA × 2.4 GHz
PEAK_FP32_VECTOR_FMA_TFLOPS = 78.6
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")
TRANSPOSE_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "transpose_traffic.json")
TRANSPOSE_SOURCE = "tiled_gemm_tgemm_amd/csrc/transpose.hip"
# the sources of the product kernel whose counters profiles/traffic.json holds
KERNEL_SOURCES = ["tiled_gemm_tgemm_amd/csrc/mfma_sgemm.hip", "tiled_gemm_tgemm_amd/csrc/mfma_common.h"]


def code_of(path: str) -> bytes:
    """A C++/HIP source with its comments and blank lines removed, so that a
    change of wording alone does not make a counter record stale.  Removes
    // and /* */ comments outside string and character literals."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [l.rstrip() for l in "".join(out).split("\n")]
    return "\n".join(l for l in lines if l.strip()).encode()


def kernel_source_hash() -> str:
    """SHA-256 of the product kernel's code (comments aside)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update(code_of(os.path.join(ROOT, rel)))
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--warmup-seconds", type=float, default=0.5,
                   help="keep warming up (untimed) until this much time has passed, so the GPU "
                        "clock has settled before the timed steps")
    p.add_argument("--workload", default="square8192_uniform")
    p.add_argument("--kernel", default="auto",
                   help="auto | naive | simt | lds<T>[p1] | mfma:<variant> | splitk[<slices>]")
    p.add_argument("--shape", default=None,
                   help="MxNxK: time a U[-1,1) product of that shape (seed 0) instead of --workload")
    p.add_argument("--also", default="square512_uniform,square1024_int4,square4096_uniform,rect3000x1000x5000_normal",
                   help="comma-separated extra workloads timed the same way ('' for none)")
    p.add_argument("--small-steps", type=int, default=500,
                   help="timed calls for the launch-bound workloads (512^3, 1024^3)")
    p.add_argument("--ragged-steps", type=int, default=50, help="timed calls for 3000x1000x5000")
    p.add_argument("--cold-also", default="square512_uniform,square1024_int4,square4096_uniform",
                   help="workloads also timed with cold caches under 'cold' ('' for none)")
    p.add_argument("--cold-steps", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-vendor", action="store_true",
                   help="skip timing the vendor BLAS (torch.matmul, fp32) beside the product")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="host threads for the cpu_baseline leg (0: the OpenMP default, all cores)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--op-a", choices=("N", "T"), default="N",
                   help="T: A is stored transposed (K×M) and passed as TGEMM_OP_T")
    p.add_argument("--op-b", choices=("N", "T"), default="N",
                   help="T: B is stored transposed (N×K) and passed as TGEMM_OP_T")
    p.add_argument("--no-engine-clock", action="store_true",
                   help="skip the amd-smi clock reading (a child process); use it under a profiler "
                        "that loads itself into every child")
    p.add_argument("--cold", action="store_true",
                   help="before every timed call, overwrite a 512 MiB buffer so that L2 and the "
                        "256 MB Infinity Cache hold none of the operands (kernel time only)")
    p.add_argument("--transpose", default=None,
                   choices=("blocked", "naive", "tiled", "tiled_padded"),
                   help="measure the transpose kernel instead of the product")
    p.add_argument("--host", action="store_true",
                   help="measure tgemm_sgemm_host (host operands, copies overlapped with the product)")
    p.add_argument("--panel-rows", type=int, default=0, help="panel height for --host (0: the library's)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="after the timed steps, run one plain device-to-device copy of this many "
                        "bytes (a known-size reference for hardware byte counters)")
    return p.parse_args()


def kernel_call(name: str):
    """(callable(A, B, C), description) for a --kernel choice."""
    import tiled_gemm_tgemm_amd as tg

    if name == "auto":
        # the C entry point itself, its arguments marshalled once per set of
        # tensors (the Python wrapper's checks cost more than a 512^3 call)
        lib = tg.library()
        cache = {}

        def call(A, B, C):
            key = (A.data_ptr(), B.data_ptr(), C.data_ptr())
            if key not in cache:
                import torch

                op_a, lda = tg._layout(A, "A")
                op_b, ldb = tg._layout(B, "B")
                cache.clear()
                cache[key] = (op_a, op_b, A.shape[0], B.shape[1], A.shape[1], A.data_ptr(), lda, B.data_ptr(),
                              ldb, C.data_ptr(), max(C.stride(0), C.shape[1], 1),
                              torch.cuda.current_stream(A.device).cuda_stream)
            st = lib.tgemm_sgemm_ex(*cache[key])
            if st != tg.TGEMM_SUCCESS:
                raise tg.TgemmError(st, "tgemm_sgemm_ex")
            return C

        return call, "tgemm_sgemm"
    if name == "naive":
        return (lambda A, B, C: tg.sgemm(A, B, out=C, kernel="naive")), "tgemm_sgemm_naive"
    if name == "simt":
        return (lambda A, B, C: tg.sgemm(A, B, out=C, kernel="simt")), "tgemm_sgemm_simt"
    if name.startswith("lds"):
        tile = int(name[3:].split("p")[0])
        pad = 1 if name.endswith("p1") else 0
        return ((lambda A, B, C: tg.sgemm(A, B, out=C, kernel="lds", tile=tile, pad=pad)),
                f"tgemm_sgemm_lds(tile={tile},pad={pad})")
    if name.startswith("splitk"):
        # tgemm_sgemm_splitk with `splits` slices ("splitk8") or the library's
        # choice ("splitk"); the workspace is allocated on the first call,
        # which is a warm-up call, outside any timed region
        splits = int(name[6:]) if name[6:] else None
        state = {}

        def call(A, B, C):
            import torch

            if "ws" not in state:
                M, K = A.shape
                N = B.shape[1]
                state["s"] = splits or tg.tgemm_sgemm_splitk_choose(M, N, K)
                need = tg.tgemm_sgemm_splitk_workspace_size(M, N, K, state["s"])
                state["ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            return tg.sgemm_splitk(A, B, out=C, splits=state["s"], workspace=state["ws"])

        return call, f"tgemm_sgemm_splitk(splits={splits if splits else 'chosen'})"
    if name.startswith("mfma:"):
        v = name.split(":", 1)[1]
        names = tg.variant_names()
        idx = names.index(v) if v in names else int(v)
        return ((lambda A, B, C: tg.sgemm(A, B, out=C, kernel="mfma", variant=idx)),
                f"tgemm_sgemm_mfma({names[idx]})")
    raise SystemExit(f"unknown --kernel {name}")


def time_workload(w, kernel: str, steps: int, warmup: int, warmup_seconds: float = 0.0,
                  cold: bool = False, op_a: str = "N", op_b: str = "N"):
    """Time `steps` calls on resident inputs; returns a dict of measurements."""
    import numpy as np
    import torch

    import tiled_gemm_tgemm_amd as tg
    from tiled_gemm_tgemm_amd import workloads as wl

    A_h, B_h = wl.make_inputs(w)
    # a transposed operand is stored transposed and handed over as a view
    A = torch.from_numpy(np.ascontiguousarray(A_h.T)).cuda().t() if op_a == "T" else torch.from_numpy(A_h).cuda()
    B = torch.from_numpy(np.ascontiguousarray(B_h.T)).cuda().t() if op_b == "T" else torch.from_numpy(B_h).cuda()
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    call, desc = kernel_call(kernel)
    variant = None
    if kernel == "auto":
        ops = (tg.TGEMM_OP_T if op_a == "T" else tg.TGEMM_OP_N, tg.TGEMM_OP_T if op_b == "T" else tg.TGEMM_OP_N)
        v = tg.tgemm_sgemm_variant_for_ex(*ops, w.M, w.N, w.K, A.data_ptr(), w.M if op_a == "T" else w.K,
                                          B.data_ptr(), w.K if op_b == "T" else w.N, C.data_ptr(), w.N)
        variant = tg.tgemm_mfma_variant_name(v)
        if op_a == "T" or op_b == "T":
            desc = f"tgemm_sgemm_ex(op_a={op_a},op_b={op_b})"
    warm = 0
    t_warm = time.perf_counter()
    while warm < warmup or time.perf_counter() - t_warm < warmup_seconds:
        call(A, B, C)
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()  # the stream every call is queued on
    torch.cuda.synchronize()

    def per_call_events(n, flush=None):
        """n calls, each between its own pair of events (ms per call)."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for i in range(n):
            if flush is not None:
                flush.fill_(float(i))
            starts[i].record(stream)
            call(A, B, C)
            ends[i].record(stream)
        torch.cuda.synchronize()
        return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    if cold:
        # a 512 MiB fill before every call; the wall clock would cover the
        # fills too, so the figure is the calls' own event time
        flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
        # the first fill of a new buffer maps its pages (~5 ms) and the calls
        # after it run up to 20% slow for ~15 ms: the flush-and-call loop is
        # warmed up as the plain calls were before it is timed
        i = 0
        t_cold = time.perf_counter()
        while i < warmup or time.perf_counter() - t_cold < warmup_seconds:
            flush.fill_(float(i))
            call(A, B, C)
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        per = per_call_events(steps, flush)
        wall_ms = kernel_ms = float(per.mean())
    else:
        # the timed region: `steps` calls back to back, one event pair on the
        # calls' stream around all of them (events between calls would add
        # their own host cost to every call of the small products)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            call(A, B, C)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wall_ms = (t1 - t0) * 1e3 / steps
        kernel_ms = ev0.elapsed_time(ev1) / steps
        # the spread of single calls, from as many more calls outside the timed region
        per = per_call_events(steps)
    return {
        "workload": w, "A_host": A_h, "B_host": B_h, "A": A, "B": B, "C": C, "desc": desc, "variant": variant,
        "warmup_launches": warm,
        "wall_ms": wall_ms, "kernel_ms": kernel_ms, "kernel_ms_per_call": float(per.mean()),
        "kernel_ms_min": float(per.min()), "kernel_ms_median": float(np.median(per)),
        "kernel_ms_p90": float(np.percentile(per, 90)),
        "tflops_wall": w.flops / (wall_ms * 1e-3) / 1e12,
        "tflops_kernel": w.flops / (kernel_ms * 1e-3) / 1e12,
    }


def engine_clock(m, kernel: str, load_seconds: float = 2.0):
    """Mean engine clock (GHz) of the XCDs while the product runs.  The same
    call is launched back to back for `load_seconds`, then two child
    `amd-smi metric -c --json` reads are taken while the launches go on; the
    second is used (the tool reports a sampled value that can lag the load).
    None where amd-smi is missing, fails, reports other than exactly one GPU,
    or reports an XCD below its minimum clock (a sample of an idle engine)."""
    import shutil
    import subprocess

    import torch

    exe = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if exe is None:
        return None
    # amd-smi is a Python script started through "#!/usr/bin/env python3";
    # run it with this interpreter directly, as a child process, so that no
    # launcher replaces one program with another on the way
    cmd = [exe]
    real = os.path.realpath(exe)
    try:
        with open(real, "rb") as f:
            first = f.readline()
        if first.startswith(b"#!") and b"python" in first:
            cmd = [sys.executable, real]
    except OSError:
        pass
    call, _ = kernel_call(kernel)
    A, B, C = m["A"], m["B"], m["C"]
    n = 0

    def busy_until(done):
        nonlocal n
        t0 = time.perf_counter()
        while not done() and time.perf_counter() - t0 < 30.0:
            call(A, B, C)
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()

    t_load = time.perf_counter()
    busy_until(lambda: time.perf_counter() - t_load >= load_seconds)
    reading = None
    for _ in range(2):
        child = subprocess.Popen(cmd + ["metric", "-c", "--json"], stdout=subprocess.PIPE,
                                 stderr=subprocess.DEVNULL, text=True)
        busy_until(lambda: child.poll() is not None)
        try:
            out, _ = child.communicate(timeout=10)
            reading = json.loads(out)["gpu_data"] if child.returncode == 0 else None
        except (subprocess.TimeoutExpired, ValueError, KeyError, TypeError):
            child.kill()
            reading = None
    torch.cuda.synchronize()
    return mean_engine_clock(reading)


def mean_engine_clock(gpu_data):
    """Mean of the XCD engine clocks (GHz) in amd-smi's `metric -c --json`
    "gpu_data" list; None unless it holds exactly one GPU whose gfx_* clocks
    are all at or above their minimum (below it, the engine was asleep)."""
    if not gpu_data or len(gpu_data) != 1:
        return None
    mhz = []
    for k, v in gpu_data[0].get("clock", {}).items():
        if not k.startswith("gfx_") or not isinstance(v, dict) or not isinstance(v.get("clk"), dict):
            continue
        lo = v.get("min_clk")
        if isinstance(lo, dict) and v["clk"]["value"] < lo["value"]:
            return None
        mhz.append(v["clk"]["value"])
    return sum(mhz) / len(mhz) / 1e3 if mhz else None


def vendor_blas(m, steps: int, warmup_seconds: float):
    """torch.matmul (fp32, TF32 off) on the same resident operands, timed like the product."""
    import torch

    torch.backends.cuda.matmul.allow_tf32 = False
    w, A, B = m["workload"], m["A"], m["B"]
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    t_warm = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t_warm < warmup_seconds:
        torch.matmul(A, B, out=C)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    # as the product's timed region: the calls back to back between one pair of events
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        torch.matmul(A, B, out=C)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    diff = float((C - m["C"]).abs().max().item())
    return {"what": "torch.matmul float32, TF32 off (ROCm BLAS); context, not a target",
            "kernel_ms_mean": round(ms, 4), "tflops": round(tflops, 3),
            "pct_of_fp32_matrix_peak": round(100.0 * tflops / PEAK_FP32_MATRIX_TFLOPS, 2),
            "tgemm_over_vendor": round(m["tflops_kernel"] / tflops, 4),
            "max_abs_diff_vs_tgemm": diff}


def traffic_for(workload_name: str, variant: str):
    """Measured HBM bytes per launch from the committed counter record, or
    None: the record holds, per workload, the configuration it was taken on,
    and the hash of the product kernel's code when it was taken."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    with open(TRAFFIC_RECORD) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    entry = rec.get("workloads", {}).get(workload_name)
    if not entry or entry.get("kernel") != variant:
        return None  # not measured, or on another configuration
    return entry.get("hbm_bytes_per_launch")


def error_ratios(C, P, S, K: int):
    """Rounding diagnostics of a real-valued product against the oracle's
    float64 P and S = sum_k |a_ik b_kj|: max |dC| / (K 2^-24 S) (the
    acceptance bound is 4), its RMS, and the RMS of dC / (sqrt(K) 2^-24 S),
    which takes out the growth with K that independent roundings give."""
    import numpy as np

    d = np.abs(np.asarray(C, np.float64) - P)
    u = 2.0 ** -24
    pos = S > 0
    if not np.all(d[~pos] == 0):
        return {"max_ratio": float("inf"), "within_bound": False}
    r = d[pos] / (K * u * S[pos])
    r_sqrt = d[pos] / (np.sqrt(K) * u * S[pos])
    return {"max_ratio": round(float(r.max()), 4) if r.size else 0.0,
            "rms_ratio": round(float(np.sqrt(np.mean(r * r))), 5) if r.size else 0.0,
            "rms_ratio_sqrt_k": round(float(np.sqrt(np.mean(r_sqrt * r_sqrt))), 4) if r.size else 0.0,
            "within_bound": bool(r.size == 0 or r.max() <= 4.0)}


def transpose_traffic_for(workload_name: str, kernel: str):
    """Measured bytes per launch of a transpose kernel from the committed record, or None."""
    if not os.path.exists(TRANSPOSE_TRAFFIC_RECORD):
        return None
    with open(TRANSPOSE_TRAFFIC_RECORD) as f:
        rec = json.load(f)
    digest = hashlib.sha256(code_of(os.path.join(ROOT, TRANSPOSE_SOURCE))).hexdigest()
    if rec.get("kernel_source_sha256") != digest or rec.get("kernel") != kernel:
        return None
    entry = rec.get("workloads", {}).get(workload_name)
    return entry.get("hbm_bytes_per_launch") if entry else None


def cpu_model(path: str = "/proc/cpuinfo"):
    """The host CPU's model name from /proc/cpuinfo (None where it has none)."""
    try:
        with open(path) as f:
            for text in f:
                key, sep, value = text.partition(":")
                if sep and key.strip() == "model name":
                    return value.strip()
    except OSError:
        pass
    return None


def cpu_baseline(m, target_s: float, others=(), one_thread_workload=None):
    """The oracle (float64 sums of exact float32 products, plus the sums of
    |products|) timed on this host's cores.  `value`: whole rows of the
    headline product, grown to ~target_s.  `full_oracle`: the whole product
    of each workload in `others` (name -> (A, B, GPU result on the host)),
    timed, and the GPU result checked against it (exact equality on integer
    inputs, else the rounding diagnostics); then an extrapolated time for the
    whole headline product at the largest of those products' oracle rate,
    and the one-thread rate on `one_thread_workload`."""
    import numpy as np
    import torch

    import oracle

    w = m["workload"]
    A, B = m["A_host"], m["B_host"]
    rows = 2
    while True:
        t0 = time.perf_counter()
        P, S = oracle.gemm_window(A, B, 0, rows, 0, w.N)
        t = time.perf_counter() - t0
        if t >= target_s or rows >= w.M:
            break
        # grow the sample towards the target from the measured rate
        grow = min(max(1.1 * target_s / max(t, 1e-3), 2.0), 64.0)
        rows = min(w.M, int(rows * grow))
    macs = rows * w.N * w.K
    C_rows = m["C"][:rows].cpu().numpy().astype(np.float64)
    out = {
        "value": 2.0 * macs / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
        "kind": "oracle", "cpu": cpu_model(), "cpus_allowed": len(os.sched_getaffinity(0)),
        "sample": f"first {rows} rows of C ({rows}x{w.N}, K={w.K}) of {w.name}: float64 sums "
                  f"with exact float32 products, plus the sums of |products|; {t:.2f} s",
        "sample_rows_within_bound": bool(np.all(np.abs(C_rows - P) <= 4.0 * w.K * 2.0 ** -24 * S)),
        "sample_rows_error": error_ratios(C_rows, P, S, w.K),
    }
    full = {}
    best_rate = None
    for name, (wo, Ah, Bh, Ch) in others.items():
        t0 = time.perf_counter()
        P, S = oracle.gemm(Ah, Bh)
        t = time.perf_counter() - t0
        entry = {"seconds": round(t, 3), "gflops": round(wo.flops / t / 1e9, 2)}
        if wo.dist == "int4":
            t0 = time.perf_counter()
            Pi = oracle.gemm_i64(Ah, Bh)
            entry["int64_seconds"] = round(time.perf_counter() - t0, 3)
            entry["gpu_exact"] = bool(np.array_equal(Ch.astype(np.int64), Pi) and np.array_equal(P, Pi))
        else:
            entry["gpu_error"] = error_ratios(Ch, P, S, wo.K)
        full[name] = entry
        if best_rate is None or wo.flops > best_rate[1]:
            best_rate = (wo.flops / t, wo.flops, name)
        del P, S
    if full:
        out["full_oracle"] = full
        rate, _, name = best_rate
        out["extrapolated_full_headline"] = {
            "what": f"the whole {w.name} product by the oracle, extrapolated (not run) from the "
                    f"{name} oracle rate: 2MNK / rate",
            "seconds": round(w.flops / rate, 1)}
    if one_thread_workload is not None:
        wo, Ah, Bh = one_thread_workload
        saved = torch.get_num_threads()
        # the oracle's OpenMP regions share the runtime torch configured at import
        torch.set_num_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.gemm(Ah, Bh)
            t = time.perf_counter() - t0
            threads = oracle.num_threads()
        finally:
            torch.set_num_threads(saved)
        out["one_thread"] = {"workload": wo.name, "seconds": round(t, 3), "gflops": round(wo.flops / t / 1e9, 2),
                             "threads": threads}
    return out


def time_transpose(w, kernel: str, steps: int, warmup: int, warmup_seconds: float):
    """Time `steps` transposes of a resident input; also a plain copy of the same size."""
    import numpy as np
    import torch

    import tiled_gemm_tgemm_amd as tg
    from tiled_gemm_tgemm_amd import workloads as wl

    A_h = wl.make_transpose_input(w)
    A = torch.from_numpy(A_h).cuda()
    B = torch.empty((w.N, w.M), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(call):
        warm, t_warm = 0, time.perf_counter()
        while warm < warmup or time.perf_counter() - t_warm < warmup_seconds:
            call()
            warm += 1
            if warm % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            call()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        per = np.array([s_.elapsed_time(e) for s_, e in zip(starts, ends)])
        return warm, wall_ms, per

    warm, wall_ms, per = timed(lambda: tg.transpose(A, out=B, kernel=kernel))
    copy_dst = torch.empty_like(A)
    _, _, per_copy = timed(lambda: copy_dst.copy_(A))
    del copy_dst
    return {"workload": w, "A_host": A_h, "B": B, "warmup_launches": warm, "wall_ms": wall_ms,
            "kernel_ms": float(per.mean()), "kernel_ms_min": float(per.min()),
            "kernel_ms_median": float(np.median(per)), "kernel_ms_p90": float(np.percentile(per, 90)),
            "copy_ms": float(per_copy.mean())}


def transpose_main(args, props):
    import numpy as np
    import torch

    from tiled_gemm_tgemm_amd import workloads as wl

    name = args.workload if args.workload in wl.TRANSPOSE_WORKLOADS else "transpose16384_uniform"
    w = wl.TRANSPOSE_WORKLOADS[name]
    m = time_transpose(w, args.transpose, args.steps, args.warmup, args.warmup_seconds)
    gbs = lambda ms: w.algorithmic_bytes / (ms * 1e-3) / 1e9  # noqa: E731
    achieved = gbs(m["kernel_ms"])
    line = {
        "metric": "fp32 matrix transpose GB/s (bytes read + written) vs the 8 TB/s HBM peak",
        "value": round(gbs(m["wall_ms"]), 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": m["warmup_launches"],
        "ms_per_step": round(m["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "seed": w.seed,
                   "kernel": f"tgemm_transpose({args.transpose})"},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": transpose_traffic_for(w.name, args.transpose),
        },
        "kernel_ms": {"mean": round(m["kernel_ms"], 4), "min": round(m["kernel_ms_min"], 4),
                      "median": round(m["kernel_ms_median"], 4), "p90": round(m["kernel_ms_p90"], 4)},
        "copy_reference": {"what": "device-to-device copy of the same M·N floats",
                           "gbs": round(gbs(m["copy_ms"]), 1), "ms": round(m["copy_ms"], 4),
                           "transpose_over_copy": round(m["copy_ms"] / m["kernel_ms"], 4)},
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
                   "hip": torch.version.hip},
    }
    if not args.no_cpu_baseline:
        import oracle

        A = m["A_host"]
        reps, t = 0, 0.0
        while t < args.cpu_seconds or reps == 0:
            t0 = time.perf_counter()
            Bo = oracle.transpose(A)
            t += time.perf_counter() - t0
            reps += 1
        same = bool(np.array_equal(Bo.view(np.uint32), m["B"].cpu().numpy().view(np.uint32)))
        line["cpu_baseline"] = {
            "value": round(reps * w.algorithmic_bytes / t / 1e9, 2), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full transposes of {w.name} ({w.M}x{w.N}) by the oracle; {t:.2f} s",
            "gpu_result_bit_exact": same,
        }
    print(json.dumps(line), flush=True)
    return 0


def host_main(args, props):
    """Host-to-host product with overlapped transfers vs the same steps in series."""
    import numpy as np
    import torch

    import tiled_gemm_tgemm_amd as tg
    from tiled_gemm_tgemm_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    A_h, B_h = wl.make_inputs(w)
    A = torch.from_numpy(A_h).pin_memory()
    B = torch.from_numpy(B_h).pin_memory()
    C = torch.empty((w.M, w.N), dtype=torch.float32).pin_memory()
    need = tg.tgemm_sgemm_host_workspace_size(w.M, w.N, w.K, args.panel_rows)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    streams = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    dA = torch.empty((w.M, w.K), device="cuda")
    dB = torch.empty((w.K, w.N), device="cuda")
    dC = torch.empty((w.M, w.N), device="cuda")
    torch.cuda.synchronize()

    def overlapped():
        tg.sgemm_host(A, B, out=C, panel_rows=args.panel_rows, streams=streams, workspace=ws)

    def serial():
        dA.copy_(A, non_blocking=True)
        dB.copy_(B, non_blocking=True)
        tg.sgemm(dA, dB, out=dC)
        C.copy_(dC, non_blocking=True)
        torch.cuda.synchronize()

    def h2d():
        dA.copy_(A, non_blocking=True)
        torch.cuda.synchronize()

    def d2h():
        C.copy_(dC, non_blocking=True)
        torch.cuda.synchronize()

    def timed(fn):
        warm, t_warm = 0, time.perf_counter()
        while warm < args.warmup or time.perf_counter() - t_warm < args.warmup_seconds:
            fn()
            warm += 1
        ts = []
        for _ in range(args.steps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.mean(ts)), float(np.min(ts))

    t_ov, t_ov_min = timed(overlapped)
    t_se, _ = timed(serial)
    serial_c = C.numpy().copy()
    overlapped()
    same = bool(np.array_equal(C.numpy(), serial_c))
    t_h2d, _ = timed(h2d)
    t_d2h, _ = timed(d2h)
    h2d_gbs = 4 * w.M * w.K / t_h2d / 1e9
    d2h_gbs = 4 * w.M * w.N / t_d2h / 1e9
    in_bytes, out_bytes = 4 * (w.M * w.K + w.K * w.N), 4 * w.M * w.N
    tflops = w.flops / t_ov / 1e12
    line = {
        "metric": "host-to-host fp32 GEMM TFLOP/s, PCIe transfers included (overlapped with the product)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_ov * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "seed": w.seed,
                   "kernel": "tgemm_sgemm_host", "panel_rows": args.panel_rows or "library default",
                   "host_memory": "pinned"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP32_MATRIX_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_MATRIX_TFLOPS, 4), "traffic": None},
        "overlap": {
            "overlapped_ms": round(t_ov * 1e3, 3), "overlapped_min_ms": round(t_ov_min * 1e3, 3),
            "serial_ms": round(t_se * 1e3, 3), "speedup": round(t_se / t_ov, 3),
            "h2d_gbs": round(h2d_gbs, 1), "d2h_gbs": round(d2h_gbs, 1),
            "transfer_floor_ms": round(max(in_bytes / (h2d_gbs * 1e9), out_bytes / (d2h_gbs * 1e9)) * 1e3, 3),
            "results_equal_serial": same,
        },
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
                   "hip": torch.version.hip},
    }
    print(json.dumps(line), flush=True)
    return 0


def plain_also(args) -> bool:
    """Whether the extra workloads run the default product (cold figures and
    counter records belong to it)."""
    return args.kernel == "auto" and args.op_a == "N" and args.op_b == "N" and not args.cold


def steps_for(w, args) -> int:
    """Timed calls for a workload: the launch-bound small products and the
    ragged one get more, so their means rest on enough calls."""
    if w.flops <= 2 * 1024 ** 3:
        return max(args.steps, args.small_steps)
    if w.name.startswith("rect"):
        return max(args.steps, args.ragged_steps)
    return args.steps


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs "
              "are not supported.", file=sys.stderr)
        return 2
    import torch

    from tiled_gemm_tgemm_amd import _lib, build, workloads as wl

    if not os.path.exists(_lib.LIBRARY):
        build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    props = torch.cuda.get_device_properties(0)
    if args.transpose:
        return transpose_main(args, props)
    if args.host:
        return host_main(args, props)

    if args.shape:
        M, N, K = (int(x) for x in args.shape.lower().split("x"))
        w = wl.Workload(f"shape{M}x{N}x{K}_uniform", M, N, K, "uniform", 0)
    else:
        w = wl.WORKLOADS[args.workload]
    m = time_workload(w, args.kernel, args.steps, args.warmup, args.warmup_seconds, args.cold,
                      args.op_a, args.op_b)
    plain = args.kernel == "auto" and args.op_a == "N" and args.op_b == "N" and not args.cold
    traffic = traffic_for(w.name, m["variant"]) if plain else None
    achieved = m["tflops_kernel"]
    # kernels that multiply on the vector ALUs are held to the fma rate
    on_valu = args.kernel in ("naive", "simt") or args.kernel.startswith("lds")
    bound, peak = ("alu", PEAK_FP32_VECTOR_FMA_TFLOPS) if on_valu else ("mfma", PEAK_FP32_MATRIX_TFLOPS)
    line = {
        "metric": METRIC,
        "value": round(m["tflops_wall"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": m["warmup_launches"],
        "ms_per_step": round(m["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "caches": "cold (512 MiB flush before each call; kernel time)" if args.cold else "warm",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "values": w.dist,
                   "seed": w.seed, "kernel": m["desc"], "variant": m["variant"],
                   "op_a": args.op_a, "op_b": args.op_b},
        "pct_of_fp32_matrix_peak": round(100.0 * m["tflops_wall"] / PEAK_FP32_MATRIX_TFLOPS, 2),
        "roofline": {
            "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "kernel_ms": {"mean": round(m["kernel_ms"], 4), "per_call_mean": round(m["kernel_ms_per_call"], 4),
                      "min": round(m["kernel_ms_min"], 4), "median": round(m["kernel_ms_median"], 4),
                      "p90": round(m["kernel_ms_p90"], 4)},
        "algorithmic_hbm_gbs": round(w.algorithmic_bytes / (m["kernel_ms"] * 1e-3) / 1e9, 1),
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
                   "hip": torch.version.hip},
    }
    if not args.cold and not args.no_engine_clock:
        ghz = engine_clock(m, args.kernel)
        # flops per clock and CU: 256 on the fp32 matrix cores, 128 as unpacked vector FMAs
        per_clk = 256 if bound == "mfma" else 128
        at_clock = props.multi_processor_count * per_clk * ghz / 1e3 if ghz else None
        line["engine_clock"] = None if ghz is None else {
            "ghz": round(ghz, 3),
            "what": "mean XCD engine clock from amd-smi, read after 2 s of the same call back to back "
                    "(after the timed steps, while it still runs)",
            "peak_at_this_clock": round(at_clock, 2),
            "frac_of_peak_at_this_clock": round(achieved / at_clock, 4),
        }
    # the vendor library computes the plain product; compare only what it computes
    vendor = not args.no_vendor and (args.kernel == "auto" or args.kernel.startswith("splitk")) and not args.cold
    if vendor:
        line["vendor_blas"] = vendor_blas(m, args.steps, args.warmup_seconds)
    also = {}
    others = {}  # inputs and GPU results kept for the oracle leg
    cold_names = [x for x in args.cold_also.split(",") if x] if plain_also(args) else []
    for name in [x for x in args.also.split(",") if x and x != w.name]:
        wa = wl.WORKLOADS[name]
        steps = steps_for(wa, args)
        ma = time_workload(wa, args.kernel, steps, args.warmup, args.warmup_seconds, args.cold,
                           args.op_a, args.op_b)
        entry = {
            "tflops": round(ma["tflops_wall"], 3),
            "ms_per_step": round(ma["wall_ms"], 5),
            "steps": steps,
            "pct_of_fp32_matrix_peak": round(100.0 * ma["tflops_wall"] / PEAK_FP32_MATRIX_TFLOPS, 2),
            "kernel_ms_mean": round(ma["kernel_ms"], 5),
            "kernel_ms_per_call_mean": round(ma["kernel_ms_per_call"], 5),
            "kernel_ms_median": round(ma["kernel_ms_median"], 5),
            "roofline_frac": round(ma["tflops_kernel"] / PEAK_FP32_MATRIX_TFLOPS, 4),
            "algorithmic_hbm_gbs": round(wa.algorithmic_bytes / (ma["kernel_ms"] * 1e-3) / 1e9, 1),
            "algorithmic_hbm_frac": round(wa.algorithmic_bytes / (ma["kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
            "variant": ma["variant"],
        }
        t_bytes = traffic_for(wa.name, ma["variant"]) if plain else None
        if t_bytes:
            gbs = t_bytes / (ma["kernel_ms"] * 1e-3) / 1e9
            entry["measured_hbm"] = {"bytes_per_launch": t_bytes, "gbs": round(gbs, 1),
                                     "frac_of_8tbs": round(gbs / PEAK_HBM_GBS, 5)}
        if vendor:
            entry["vendor_blas"] = vendor_blas(ma, steps, args.warmup_seconds)
        if name in cold_names:
            mc = time_workload(wa, args.kernel, args.cold_steps, args.warmup, args.warmup_seconds, True,
                               args.op_a, args.op_b)
            entry["cold"] = {"what": "512 MiB written before every call (L2 and the Infinity Cache hold none "
                                     "of the operands); kernel time",
                             "steps": args.cold_steps, "kernel_ms_mean": round(mc["kernel_ms"], 5),
                             "kernel_ms_median": round(mc["kernel_ms_median"], 5),
                             "tflops": round(mc["tflops_kernel"], 3),
                             "roofline_frac": round(mc["tflops_kernel"] / PEAK_FP32_MATRIX_TFLOPS, 4),
                             "algorithmic_hbm_gbs": round(wa.algorithmic_bytes / (mc["kernel_ms"] * 1e-3) / 1e9, 1)}
            del mc
        also[name] = entry
        if not args.no_cpu_baseline:
            others[name] = (wa, ma["A_host"], ma["B_host"], ma["C"].cpu().numpy())
        del ma
    if also:
        line["also"] = also
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_reference_bytes"] = 4 * n
        del src, dst
    if not args.no_cpu_baseline:
        if args.cpu_threads > 0:
            # the oracle's OpenMP regions share the runtime torch configured at
            # import; this sets the thread count they run with
            torch.set_num_threads(args.cpu_threads)
        one = None
        if "square512_uniform" in others:
            wo, Ah, Bh, _ = others["square512_uniform"]
            one = (wo, Ah, Bh)
        line["cpu_baseline"] = cpu_baseline(m, args.cpu_seconds, others, one)
        # the GPU results of the other workloads against the whole oracle product
        for name, entry in line["cpu_baseline"].get("full_oracle", {}).items():
            also[name]["parity"] = {k: v for k, v in entry.items() if k in ("gpu_exact", "gpu_error")}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
