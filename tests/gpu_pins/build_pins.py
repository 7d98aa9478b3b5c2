"""Build tests/gpu_pins/libdspins.so: test-only kernels over the library's device
building blocks (see ds_pins.hip).  Same compiler and flags as the library."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "ds_pins.hip")
LIB = os.path.join(HERE, "libdspins.so")


def build() -> str:
    sys.path.insert(0, ROOT)
    from vocab_wise_logit_amd import build as libbuild

    tmp = LIB + ".tmp"
    cmd = [libbuild.hipcc(), *libbuild.HIPFLAGS, "-shared", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
