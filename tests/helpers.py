"""Shared test helpers: bf16 bit conversions and the golden-file reader.

No quantization arithmetic lives here."""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16_bits(values) -> np.ndarray:
    """Exact bf16 bit patterns of values that bf16 represents exactly (asserted)."""
    f = np.asarray(values, dtype=np.float32)
    t = torch.from_numpy(f.copy()).to(torch.bfloat16)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back.view(np.uint32), f.view(np.uint32)), "not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def read_examples(name: str = "worked_examples.txt"):
    """Parse the worked-example fixture into a list of dicts."""
    out, cur = [], None
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            vals = rest.split()
            if key == "example":
                cur = {"name": vals[0]}
                out.append(cur)
            elif key in ("mode",):
                cur[key] = vals[0]
            elif key == "rules":
                cur[key] = vals
            elif key in ("input", "y"):
                cur[key] = [float(v) if v != "-0" else -0.0 for v in vals]
            elif key == "alpha_bits":
                cur[key] = int(vals[0], 16)
            elif key in ("scales", "codes"):
                cur[key] = [int(v, 16) for v in vals]
            elif key == "qstar":
                cur[key] = [int(v) for v in vals]
            elif key == "stats":
                cur[key] = [2.0 ** int(v[2:]) if v.startswith("2^") else float(v) for v in vals]
            else:
                raise ValueError("unknown key %r in %s" % (key, name))
    return out
