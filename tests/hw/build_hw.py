"""Build tests/hw/libhwconv.so, the exhaustive check of the gfx950 conversion instructions
(test infrastructure; see hw_conversions.hip).  Same compiler and flags as the library."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hw_conversions.hip")
LIB = os.path.join(HERE, "libhwconv.so")


def build() -> str:
    sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
    from nvfp4_block_scaled_amax_amd import build as b
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [b.hipcc()] + b.flags() + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
