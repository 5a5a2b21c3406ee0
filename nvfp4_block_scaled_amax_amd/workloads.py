"""Seeded synthetic bf16 workloads for NVFP4 quantization.

This module holds input generation only -- no quantization arithmetic.  Both the
HIP path and the CPU oracle consume what it produces.

The pages quantize LLM weights, activations and gradients (Nemotron 3 Nano,
Llama 3, Qwen 3 in the Four Over Six explainer, "Key contributions and
results"; W4A16 / W4A4 students in the Nemotron NVFP4 pages).  No checkpoint or
dataset is available, so each workload below is a synthetic stand-in with the
shape and value distribution of one such tensor kind:

  tiny    256 x 256        N(0, 1)                                     seed 0
  weight  4096 x 14336     0.02 * N(0, 1); 0.1 % of positions (distinct,
                           uniform) multiplied by 20                    seed 1
  act     8192 x 4096      0.5 * Student-t(nu = 3); 8 distinct columns
                           multiplied by 50                             seed 2
  large   16384 x 14336    N(0, 1); each entry independently with
                           p = 0.01 replaced by Laplace(0, b = 10)      seed 3
  moe     64 x 2048 x 5120 expert e: sigma_e * N(0, 1), sigma_e
                           log-uniform in [0.005, 0.05]                 seed 4

Random numbers come from numpy's PCG64 (``default_rng(seed)``) in float64 or
float32 and are rounded to bfloat16 with torch's round-to-nearest-even cast.
Generation is chunked so the largest workload (1.34 GB of bf16) never holds a
full float64 copy.  All generators accept other shapes, so the tests can draw
small tensors of the same distribution.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np
import torch

_CHUNK = 1 << 24  # elements per generation chunk


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple            # (rows, cols) or (E, rows, cols); blocks run along cols
    seed: int
    runs: tuple             # ((mode, rule, output), ...) -- output "packed" | "fakequant"
    description: str


WORKLOADS = {
    "tiny": Workload("tiny", (256, 256), 0,
                     (("rtn6", "mse", "packed"), ("four_over_six", "mse", "packed")),
                     "256x256 bf16, N(0,1)"),
    "weight": Workload("weight", (4096, 14336), 1,
                       (("four_over_six", "mse", "packed"), ("rtn6", "mse", "packed")),
                       "4096x14336 bf16 weight, N(0,0.02^2), 0.1% entries x20"),
    "act": Workload("act", (8192, 4096), 2,
                    (("four_over_six", "mae", "fakequant"),),
                    "8192 tokens x 4096 bf16 activation, 0.5*t(3), 8 channels x50"),
    "large": Workload("large", (16384, 14336), 3,
                      (("four_over_six", "mse", "packed"), ("four_over_six", "mae", "packed"),
                       ("four_over_six", "maxerr", "packed"), ("rtn6", "mse", "packed")),
                      "16384x14336 bf16, N(0,1) with 1% Laplace(0,10) outliers"),
    "moe": Workload("moe", (64, 2048, 5120), 4,
                    (("four_over_six", "mse", "packed"),),
                    "64 experts x 2048x5120 bf16, per-expert sigma log-uniform [0.005,0.05]"),
}


def _to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _fill(n: int, draw) -> torch.Tensor:
    """Fill n bf16 values chunk by chunk; draw(k) returns k float32/float64 values."""
    out = torch.empty(n, dtype=torch.bfloat16)
    for lo in range(0, n, _CHUNK):
        k = min(_CHUNK, n - lo)
        out[lo:lo + k] = _to_bf16(draw(k))
    return out


def normal(shape, seed: int, sigma: float = 1.0) -> torch.Tensor:
    """sigma * N(0, 1)."""
    rng = np.random.default_rng(seed)
    n = math.prod(shape)
    return _fill(n, lambda k: rng.standard_normal(k, dtype=np.float32) *
                 np.float32(sigma)).view(shape)


def weight(shape, seed: int = 1) -> torch.Tensor:
    """0.02 * N(0,1), then round(0.001 * N) distinct uniform positions multiplied by 20."""
    rng = np.random.default_rng(seed)
    n = math.prod(shape)
    base = np.empty(n, np.float32)
    for lo in range(0, n, _CHUNK):
        k = min(_CHUNK, n - lo)
        base[lo:lo + k] = rng.standard_normal(k, dtype=np.float32) * np.float32(0.02)
    pos = rng.choice(n, size=int(round(0.001 * n)), replace=False)
    base[pos] *= np.float32(20.0)
    return _to_bf16(base).view(shape)


def activation(shape, seed: int = 2) -> torch.Tensor:
    """0.5 * Student-t(3); 8 distinct channels (last-dim columns) multiplied by 50."""
    rng = np.random.default_rng(seed)
    rows, cols = shape
    cols_hot = rng.choice(cols, size=min(8, cols), replace=False)
    x = (rng.standard_t(3, size=(rows, cols)) * 0.5).astype(np.float32)
    x[:, cols_hot] *= np.float32(50.0)
    return _to_bf16(x).view(shape)


def large(shape, seed: int = 3) -> torch.Tensor:
    """N(0,1); each entry independently with p = 0.01 replaced by Laplace(0, 10)."""
    rng = np.random.default_rng(seed)
    n = math.prod(shape)

    def draw(k):
        x = rng.standard_normal(k, dtype=np.float32)
        hit = rng.random(k, dtype=np.float32) < np.float32(0.01)
        x[hit] = rng.laplace(0.0, 10.0, size=int(hit.sum())).astype(np.float32)
        return x
    return _fill(n, draw).view(shape)


def moe(shape, seed: int = 4) -> torch.Tensor:
    """E experts; expert e is sigma_e * N(0,1), sigma_e = exp(U(ln 0.005, ln 0.05))."""
    rng = np.random.default_rng(seed)
    E, rows, cols = shape
    sig = np.exp(rng.uniform(math.log(0.005), math.log(0.05), size=E)).astype(np.float32)
    out = torch.empty((E, rows * cols), dtype=torch.bfloat16)
    for e in range(E):
        out[e] = _fill(rows * cols, lambda k: rng.standard_normal(k, dtype=np.float32) *
                       sig[e])
    return out.view(shape)


_GEN = {"tiny": lambda s, seed: normal(s, seed), "weight": weight, "act": activation,
        "large": large, "moe": moe}


def generate(name: str, shape=None, seed=None) -> torch.Tensor:
    """The named workload (full size by default) as a CPU bf16 tensor."""
    w = WORKLOADS[name]
    return _GEN[name](tuple(shape) if shape is not None else w.shape,
                      w.seed if seed is None else seed)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (no copy for contiguous CPU tensors)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def sha256(t: torch.Tensor) -> str:
    """SHA-256 of the tensor's bf16 bytes (row-major), the fingerprint of an input of record."""
    return hashlib.sha256(memoryview(bits(t).reshape(-1))).hexdigest()
