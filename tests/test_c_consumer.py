"""The C ABI from a plain C program, with no Python or torch in between (no GPU needed).

A C99 file is compiled with gcc against include/nvfp4_amax.h alone, linked against the built
libnvfp4_amax.so and run.  It checks the ABI version, the status strings, the fused-path query
and that argument errors come back as status codes before any device work (so the calls never
reach a GPU).  This pins that the header is valid C and self-contained, and that every entry
point it declares resolves at link time.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import nvfp4_block_scaled_amax_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "nvfp4_amax.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

int main(void) {
  /* fake, never dereferenced, 16-byte aligned addresses: validation fails first */
  const uint16_t* in = (const uint16_t*)(uintptr_t)0x100000;
  uint8_t* codes = (uint8_t*)(uintptr_t)0x900000;
  uint8_t* scales = (uint8_t*)(uintptr_t)0x1100000;
  float* alpha = (float*)(uintptr_t)0x1900000;
  uint16_t* out = (uint16_t*)(uintptr_t)0x2100000;

  CHECK(nvfp4_abi_version() == NVFP4_ABI_VERSION);
  CHECK(strcmp(nvfp4_status_str(NVFP4_OK), "ok") == 0);
  CHECK(strcmp(nvfp4_status_str((nvfp4_status)99), "unknown status") == 0);

  CHECK(nvfp4_quantize(NULL, 4, 32, NVFP4_BLOCK, NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE,
                       codes, scales, alpha, NULL) == NVFP4_ERR_NULL);
  CHECK(nvfp4_quantize(in, 4, 24, NVFP4_BLOCK, NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE,
                       codes, scales, alpha, NULL) == NVFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(in, 4, 32, 32, NVFP4_RTN6, NVFP4_RULE_MSE,
                       codes, scales, alpha, NULL) == NVFP4_ERR_BLOCK);
  CHECK(nvfp4_quantize(in, 4, 32, NVFP4_BLOCK, (nvfp4_mode)7, NVFP4_RULE_MSE,
                       codes, scales, alpha, NULL) == NVFP4_ERR_ENUM);
  CHECK(nvfp4_fakequant(in, 4, 32, NVFP4_BLOCK, NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MAE,
                        (uint16_t*)((uintptr_t)out + 2), alpha, NULL) == NVFP4_ERR_ALIGN);
  CHECK(nvfp4_amax(in, 1, 4, 32, (float*)((uintptr_t)in + 4), NULL) == NVFP4_ERR_ALIAS);
  CHECK(nvfp4_dequantize(codes, scales, alpha, 1, 4, 30, out, NULL) == NVFP4_ERR_SHAPE);

  /* the fused-path query is host logic: a 256x256 tensor takes the single-read path */
  CHECK(nvfp4_fused_single_read(1, 256, 256, NVFP4_FOUR_OVER_SIX, NVFP4_RULE_MSE, 0) >= 0);
  printf("c consumer ok\n");
  return 0;
}
"""


@pytest.fixture(scope="module")
def libdir():
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_block_scaled_amax_amd import build
        build.build_library()
    return os.path.dirname(nv.LIB_PATH)


def test_c_program_compiles_links_and_runs(tmp_path, libdir):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lnvfp4_amax", "-Wl,-rpath," + libdir,
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer ok" in r.stdout
