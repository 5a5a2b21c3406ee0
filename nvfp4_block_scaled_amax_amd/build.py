"""Build libnvfp4_amax.so (HIP, gfx950) in-tree with hipcc.

Flags that the arithmetic depends on:
  -ffp-contract=off      no fused multiply-add except where the source writes fma
  -packed-fp32-ops off   no v_pk_{add,mul,fma}_f32 generated for this code
  (defaults kept)        correctly rounded fp32 division, fp32 denormals preserved

The build also reads the compiler's per-kernel resource report and fails if any kernel
spills to scratch memory: the single-read kernel keeps up to 28 blocks per lane in
registers at the 256-VGPR limit, and a spill there would be slow without being wrong.
"""
from __future__ import annotations

import os
import re
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


def scratch_users(report: str) -> list:
    """Kernels with a nonzero ScratchSize in a -Rpass-analysis=kernel-resource-usage report."""
    users, name = [], None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            users.append((name, int(m.group(1))))
    return users


def build_library(verbose: bool = False) -> str:
    """Compile the kernels and the C ABI into LIB (atomically replaced)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-Rpass-analysis=kernel-resource-usage", "-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = (res.stdout + res.stderr).splitlines()
    kept, skip = [], 0
    for l in lines:              # drop the resource remarks with their source-line context
        if "kernel-resource-usage" in l:
            skip = 2
        elif skip and re.match(r"^\s*\d*\s*\|", l):
            skip -= 1
        elif "packed-fp32-ops" not in l:
            skip = 0
            kept.append(l)
    out = "\n".join(kept)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    spills = scratch_users("\n".join(lines))
    if spills:
        os.remove(tmp)
        raise RuntimeError("kernels spill to scratch memory: %s" % spills)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
