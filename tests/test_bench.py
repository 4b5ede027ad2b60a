"""Host logic of bench.py that runs without a GPU: the one-GPU contract, the
kernel-code hash that keys the committed traffic record, and the reading of
amd-smi's clock report."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in (res.stdout + res.stderr)
    assert not res.stdout.lstrip().startswith("{")  # no JSON line is printed


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text('int f(int x) {\n    return x + 1;  // one\n}\n/* block */\nconst char *s = "// kept";\n')
    b.write_text('// a new header comment\nint f(int x) {\n\n    return x + 1;  // reworded\n}\n'
                 'const char *s = "// kept";\n')
    assert bench.code_of(str(a)) == bench.code_of(str(b))
    b.write_text('int f(int x) {\n    return x + 2;\n}\nconst char *s = "// kept";\n')
    assert bench.code_of(str(a)) != bench.code_of(str(b))
    # text inside string literals is code, not comment
    b.write_text('int f(int x) {\n    return x + 1;\n}\nconst char *s = "// changed";\n')
    assert bench.code_of(str(a)) != bench.code_of(str(b))


def test_traffic_record_is_used_only_for_the_kernel_it_was_taken_on(tmp_path, monkeypatch):
    record = {"kernel_source_sha256": bench.kernel_source_hash(),
              "workloads": {"square8192_uniform": {"kernel": "m256n128k16_w2x2_vec4",
                                                   "hbm_bytes_per_launch": 123456789}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(record))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.traffic_for("square8192_uniform", "m256n128k16_w2x2_vec4") == 123456789
    assert bench.traffic_for("square4096_uniform", "m256n128k16_w2x2_vec4") is None
    assert bench.traffic_for("square8192_uniform", "m128n128k32_w2x2_vec4") is None
    record["kernel_source_sha256"] = "0" * 64
    path.write_text(json.dumps(record))
    assert bench.traffic_for("square8192_uniform", "m256n128k16_w2x2_vec4") is None


def test_committed_traffic_record_matches_the_current_kernel():
    """profiles/traffic.json must be re-measured whenever the product kernel's
    code changes; otherwise bench.py reports roofline.traffic as null."""
    with open(bench.TRAFFIC_RECORD) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def _xcd(clk, lo=500):
    return {"clk": {"value": clk, "unit": "MHz"}, "min_clk": {"value": lo, "unit": "MHz"},
            "max_clk": {"value": 2400, "unit": "MHz"}}


def _gpu(clocks):
    c = {f"gfx_{i}": _xcd(v) for i, v in enumerate(clocks)}
    c["mem_0"] = _xcd(2000, 2000)
    c["vclk_0"] = {"clk": {"value": 59, "unit": "MHz"}, "min_clk": "N/A"}
    return {"gpu": 0, "clock": c}


def test_engine_clock_is_the_mean_over_the_xcds():
    assert bench.mean_engine_clock([_gpu([2392, 2377, 2400, 2359, 2394, 2374, 2396, 2366])]) == \
        pytest.approx(19058 / 8 / 1e3, abs=1e-12)


@pytest.mark.parametrize("data", [
    [],                                            # no GPU reported
    None,
    [_gpu([2400] * 8), _gpu([2400] * 8)],          # which one is ours is unknown
    [_gpu([2392, 95, 2400, 2359, 2394, 2374, 2396, 2366])],  # one XCD asleep: an idle sample
    [{"gpu": 0, "clock": {}}],
])
def test_engine_clock_rejects_readings_it_cannot_trust(data):
    assert bench.mean_engine_clock(data) is None


def test_error_ratios_against_known_differences():
    import numpy as np

    K = 1000
    S = np.full((2, 3), 8.0)
    P = np.zeros((2, 3))
    u = 2.0 ** -24
    C = np.array([[0.0, K * u * 8.0, -2 * K * u * 8.0], [0.5 * K * u * 8.0, 0.0, 0.0]])
    r = bench.error_ratios(C, P, S, K)
    assert r["max_ratio"] == 2.0 and r["within_bound"]
    assert abs(r["rms_ratio"] - np.sqrt((1 + 4 + 0.25) / 6)) < 1e-4
    assert abs(r["rms_ratio_sqrt_k"] - np.sqrt(K) * np.sqrt((1 + 4 + 0.25) / 6)) < 1e-2
    C[0, 0] = 5 * K * u * 8.0
    assert not bench.error_ratios(C, P, S, K)["within_bound"]
    # where S is zero the product must be exactly zero
    S[1, 1] = 0.0
    C[0, 0] = 0.0
    C[1, 1] = 1e-30
    assert bench.error_ratios(C, P, S, K)["within_bound"] is False


def test_step_counts_per_workload():
    from tiled_gemm_tgemm_amd import workloads as wl

    class A:  # noqa: N801 - the three options steps_for reads
        steps, small_steps, ragged_steps = 20, 500, 50
    W = wl.WORKLOADS
    assert bench.steps_for(W["square512_uniform"], A) == 500
    assert bench.steps_for(W["square1024_int4"], A) == 500
    assert bench.steps_for(W["rect3000x1000x5000_normal"], A) == 50
    assert bench.steps_for(W["square4096_uniform"], A) == 20
    assert bench.steps_for(W["square8192_uniform"], A) == 20


def test_cpu_model_is_read_from_cpuinfo(tmp_path):
    info = tmp_path / "cpuinfo"
    info.write_text("processor\t: 0\nvendor_id\t: AuthenticAMD\nmodel name\t: AMD EPYC 9575F 64-Core Processor\n"
                    "processor\t: 1\nmodel name\t: AMD EPYC 9575F 64-Core Processor\n")
    assert bench.cpu_model(str(info)) == "AMD EPYC 9575F 64-Core Processor"
    info.write_text("processor\t: 0\nfeatures\t: fp asimd\n")
    assert bench.cpu_model(str(info)) is None
    assert bench.cpu_model(str(tmp_path / "missing")) is None
