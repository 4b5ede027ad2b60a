"""Compile the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure only.  Flags: -O2, OpenMP for the row split, and
-ffp-contract=off so that gcc never fuses a multiply and an add on its own
(the only fused multiply-add in the oracle is the explicit fmaf of the float32
model); no -ffast-math, so no reassociation.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def build(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile `source` into the shared library `output`; return its path."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
