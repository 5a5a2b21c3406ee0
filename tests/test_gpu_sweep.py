"""A seeded sweep over every entry point on random shapes and value ranges (GPU).

Each case draws a shape (batched or not, ragged last workgroups), a distribution from the
workload generators rescaled by 2^-126 .. 2^100 (bf16 subnormals, alpha below 2^-118 and
subnormal scale bytes, which take the reference path, are reached), a mode and a rule, and runs the dynamic packed and
fake-quant calls, the fixed-scale calls, the single-read calls, dequantize and diagnostics.
Every output is compared with the oracle bit for bit (the diagnostics' statistics within their
rounding bound)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W
from test_gpu_parity import check_stats

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
RUNS = [("rtn6", "mse"), ("four_over_six", "mse"), ("four_over_six", "mae"),
        ("four_over_six", "maxerr")]
NAMES = ["tiny", "weight", "act", "large", "moe"]


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_amax_amd as m
    m.lib()
    return m


def _case(k):
    rng = np.random.default_rng(5000 + k)
    rows = int(rng.integers(1, 65))
    cols = int(rng.integers(1, 129)) * 16
    E = int(rng.integers(2, 5)) if k % 3 == 0 else None
    shape = (E, rows, cols) if E else (rows, cols)
    name = NAMES[k % len(NAMES)]
    scale = float(2.0 ** rng.integers(-126, 101))   # no overflow: |x| stays below 2^120
    if name == "moe":                               # the generator takes [E, rows, cols]
        gshape = shape if len(shape) == 3 else (1,) + shape
    else:                                           # the others take [rows, cols]
        gshape = (rows * (E or 1), cols)
    x = (W.generate(name, gshape, seed=6000 + k).float() * scale).to(torch.bfloat16)
    x = x.view(shape)
    mode, rule = RUNS[int(rng.integers(0, 4))]
    return shape, name, scale, x, mode, rule


@pytest.mark.parametrize("k", range(40))
def test_every_entry_point_on_a_random_case(nv, orc, k):
    shape, name, scale, xt, mode, rule = _case(k)
    print("[sweep] %d %s %s x%g %s/%s" % (k, name, shape, scale, mode, rule), flush=True)
    sys.stdout.flush()
    x = W.bits(xt)
    E = shape[0] if len(shape) == 3 else 1
    xg = xt.cuda()
    ref = orc.quantize(x, mode, rule, nthreads=NTHREADS, want_y=True, want_qstar=True)
    ref_alpha = ref["alpha"][:E].view(np.uint32)

    c, s, a = nv.quantize(xg, mode, rule)
    y, a2 = nv.fakequant(xg, mode, rule)
    am = nv.amax(xg)
    c3, s3, a3 = nv.quantize_from_amax(xg, am, mode, rule)
    y4, _ = nv.fakequant_from_amax(xg, am, mode, rule)
    c5, s5, a5 = nv.quantize_fused(xg, mode, rule)
    y6, a6 = nv.fakequant_fused(xg, mode, rule)
    yd = nv.dequantize(c, s, a)
    c7, s7, a7, q7, n7, st7 = nv.quantize_diag(xg, mode, rule)
    torch.cuda.synchronize()

    u16 = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    for tag, cc, ss, aa in (("dynamic", c, s, a), ("from_amax", c3, s3, a3),
                            ("fused", c5, s5, a5), ("diag", c7, s7, a7)):
        assert np.array_equal(aa.cpu().numpy().view(np.uint32), ref_alpha), tag
        assert np.array_equal(cc.cpu().numpy(), ref["codes"]), tag
        assert np.array_equal(ss.cpu().numpy(), ref["scales"]), tag
    for tag, yy in (("fakequant", y), ("fakequant_from_amax", y4), ("fakequant_fused", y6),
                    ("dequantize", yd)):
        assert np.array_equal(u16(yy), ref["y"]), tag
    assert np.array_equal(a2.cpu().numpy().view(np.uint32), ref_alpha)
    assert np.array_equal(a6.cpu().numpy().view(np.uint32), ref_alpha)
    assert np.array_equal(q7.cpu().numpy(), ref["qstar"])
    assert np.array_equal(n7.cpu().numpy(), (ref["qstar"].reshape(E, -1) == 4).sum(axis=1))
    check_stats(st7.cpu().numpy(), orc.quantize_stats(x, mode, rule, nthreads=NTHREADS),
                x.size // E, "sweep%d" % k)
