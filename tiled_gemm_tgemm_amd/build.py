"""Build libtgemm.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Every source is compiled to its own object in parallel, then linked into
``tiled_gemm_tgemm_amd/libtgemm.so``.  Flags:

* ``--offload-arch=gfx950`` — MI355X only;
* ``-O3 -std=c++17``;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` — keep the compiler
  from forming packed fp32 instructions (hipcc's host pass warns that it does
  not know the feature; that is harmless).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libtgemm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "host_pipeline.cpp", "naive.hip", "lds_tiled.hip", "simt_tiled.hip", "transpose.hip", "splitk_sum.hip",
           "mfma_sgemm.hip", "mfma_sgemm_flat.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wextra",
          "-Wno-unused-parameter",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtgemm)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass always warns about the device-only target feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(output: str = LIBRARY, extra=()) -> str:
    """Compile and link libtgemm.so; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, extra), SOURCES))
    tmp = output + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
