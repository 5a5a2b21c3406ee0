"""The whole path driven from plain C on the GPU, checked against the oracle's C interface.

A C99 program built with gcc allocates device memory with the HIP runtime, copies a seeded
input in, calls nvfp4_quantize / nvfp4_fakequant / nvfp4_dequantize through the C ABI on the
default stream, copies the results back and compares them byte for byte with orc_quantize
(the CPU oracle, linked as a test-only library).  No Python or torch is involved in the run,
so this pins that the boundary alone is enough to use the library.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest
import torch

import nvfp4_block_scaled_amax_amd as nv

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "nvfp4_amax.h"
#include "nvfp4_oracle.h"

#define HIPCHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); return 2; } } while (0)

enum { E = 2, ROWS = 48, COLS = 272 };   /* 17 blocks per row: 1632 blocks, ragged grids */
#define N ((size_t)E * ROWS * COLS)
#define NB (N / 16)

/* seeded bf16 bit patterns: random sign, exponents 2^-7 .. 2^3, random fraction; every
 * 97th element 2^6 larger (block outliers) */
static uint32_t rng = 12345u;
static uint32_t next(void) { rng ^= rng << 13; rng ^= rng >> 17; rng ^= rng << 5; return rng; }

static int compare(const char* what, const uint8_t* a, const uint8_t* b, size_t n) {
  size_t bad = 0, first = 0;
  for (size_t i = 0; i < n; ++i) if (a[i] != b[i]) { if (!bad) first = i; ++bad; }
  if (bad) printf("%s: %zu of %zu bytes differ, first at %zu\n", what, bad, n, first);
  return bad != 0;
}

int main(void) {
  uint16_t* x = malloc(N * 2);
  for (size_t i = 0; i < N; ++i) {
    uint32_t r = next();
    uint32_t e = 120u + r % 11u + (i % 97 == 0 ? 6u : 0u);
    x[i] = (uint16_t)(((r >> 8) & 1u) << 15 | e << 7 | ((r >> 16) & 0x7Fu));
  }
  const int modes[3] = {NVFP4_FOUR_OVER_SIX, NVFP4_FOUR_OVER_SIX, NVFP4_RTN6};
  const int rules[3] = {NVFP4_RULE_MSE, NVFP4_RULE_MAE, NVFP4_RULE_MSE};
  uint16_t *dx, *dy, *dz; uint8_t *dc, *ds; float* da;
  HIPCHECK(hipMalloc((void**)&dx, N * 2));
  HIPCHECK(hipMalloc((void**)&dy, N * 2));
  HIPCHECK(hipMalloc((void**)&dz, N * 2));
  HIPCHECK(hipMalloc((void**)&dc, N / 2));
  HIPCHECK(hipMalloc((void**)&ds, NB));
  HIPCHECK(hipMalloc((void**)&da, E * sizeof(float)));
  HIPCHECK(hipMemcpy(dx, x, N * 2, hipMemcpyHostToDevice));
  uint8_t *c = malloc(N / 2), *s = malloc(NB), *rc = malloc(N / 2), *rs = malloc(NB);
  uint16_t *y = malloc(N * 2), *z = malloc(N * 2), *ry = malloc(N * 2);
  float a[E], ra[E], b[E];
  int fails = 0;
  for (int k = 0; k < 3; ++k) {
    nvfp4_status st = nvfp4_quantize_batched(dx, E, ROWS, COLS, NVFP4_BLOCK, (nvfp4_mode)modes[k],
                                             (nvfp4_rule)rules[k], dc, ds, da, NULL);
    if (st != NVFP4_OK) { printf("quantize: %s\n", nvfp4_status_str(st)); return 3; }
    st = nvfp4_dequantize(dc, ds, da, E, ROWS, COLS, dz, NULL);
    if (st != NVFP4_OK) { printf("dequantize: %s\n", nvfp4_status_str(st)); return 3; }
    HIPCHECK(hipDeviceSynchronize());
    HIPCHECK(hipMemcpy(c, dc, N / 2, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(s, ds, NB, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(a, da, sizeof a, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(z, dz, N * 2, hipMemcpyDeviceToHost));
    st = nvfp4_fakequant_batched(dx, E, ROWS, COLS, NVFP4_BLOCK, (nvfp4_mode)modes[k],
                                 (nvfp4_rule)rules[k], dy, da, NULL);
    if (st != NVFP4_OK) { printf("fakequant: %s\n", nvfp4_status_str(st)); return 3; }
    HIPCHECK(hipDeviceSynchronize());
    HIPCHECK(hipMemcpy(y, dy, N * 2, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(b, da, sizeof b, hipMemcpyDeviceToHost));
    if (orc_quantize(x, E, ROWS, COLS, modes[k], rules[k], rc, rs, ra, ry, NULL, 4) != 0) {
      printf("oracle rejected the input\n");
      return 4;
    }
    fails += compare("codes", c, rc, N / 2);
    fails += compare("scales", s, rs, NB);
    fails += compare("alpha", (const uint8_t*)a, (const uint8_t*)ra, sizeof a);
    fails += compare("fake-quant alpha", (const uint8_t*)b, (const uint8_t*)ra, sizeof b);
    fails += compare("fake-quant", (const uint8_t*)y, (const uint8_t*)ry, N * 2);
    fails += compare("dequantize", (const uint8_t*)z, (const uint8_t*)ry, N * 2);
    printf("case %d (mode %d rule %d): %s\n", k, modes[k], rules[k], fails ? "MISMATCH" : "same");
  }
  hipFree(dx); hipFree(dy); hipFree(dz); hipFree(dc); hipFree(ds); hipFree(da);
  if (!fails) printf("c consumer on the GPU ok\n");
  return fails ? 1 : 0;
}
"""


def test_c_program_matches_the_oracle_on_the_gpu(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    nv.lib()                                   # raises if the HIP library is missing
    libdir = os.path.dirname(nv.LIB_PATH)
    orcdir = os.path.join(ROOT, "oracle")
    assert os.path.exists(os.path.join(orcdir, "libnvfp4_oracle.so")), "oracle not built"
    src = tmp_path / "gpu_consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "gpu_consumer"
    rocm_lib = os.path.join(ROCM, "lib")
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           "-I", orcdir, "-I", os.path.join(ROCM, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lnvfp4_amax", "-Wl,-rpath," + libdir,
           "-L", orcdir, "-lnvfp4_oracle", "-Wl,-rpath," + orcdir,
           "-L", rocm_lib, "-lamdhip64", "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("[c-consumer] running %s" % exe, flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer on the GPU ok" in r.stdout
