"""Build libnvfp4_amax.so (HIP, gfx950) in-tree with hipcc.

Flags that the arithmetic depends on:
  -ffp-contract=off      no fused multiply-add except where the source writes fma
  -packed-fp32-ops off   no v_pk_{add,mul,fma}_f32 generated for this code
  (defaults kept)        correctly rounded fp32 division, fp32 denormals preserved
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "nvfp4_amax.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnvfp4_amax.so")
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-I" + INCLUDE]


def build_library(verbose: bool = False) -> str:
    """Compile the kernels and the C ABI into LIB (atomically replaced)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
