"""Compile the CPU oracle (plain C, gcc) into oracle/libdsoracle.so.

Test infrastructure: the oracle is built so that tests and the benchmark's CPU
baseline can run it; the product library never loads it.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ds_oracle.c")
LIB = os.path.join(HERE, "libdsoracle.so")

# No -ffast-math and no contraction: every float expression rounds as written.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*(sys.argv[1:2] or [])))
