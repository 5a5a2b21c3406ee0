"""The gfx950 conversion instructions the block pass uses, checked on every binary32 input
against their definitions (tests/hw/hw_conversions.hip, built by __graft_entry__.build()).

The fast path takes its FP4 rounding, FP4 decode, E4M3 scale byte and bf16 fake-quant output
from these instructions; the reference path and the oracle compute the same roundings in
software.  Zero mismatches over all inputs make the two interchangeable."""
from __future__ import annotations

import ctypes
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libhwconv.so")
# (which, what, inputs compared): every pattern but NaNs (2 * (2^23 - 1)); 256 bytes x 4
# positions x 2 codes; +0 up to +inf; every pattern but infinities and NaNs (2 * 2^23); every
# pattern above 448 up to +inf.
CASES = [(0, "v_cvt_scalef32_pk_fp4_f32: E2M1 round to nearest even, all 2^32 inputs, 4 bytes",
          2**32 - 2 * (2**23 - 1)),
         (1, "v_cvt_scalef32_pk_f32_fp4: the 16 codes in each byte position", 256 * 4 * 2),
         (2, "v_cvt_pk_fp8_f32 after the 448 clamp: E4M3 round to nearest even, inputs >= 0",
          0x7F800001),
         (3, "v_cvt_pk_bf16_f32: bf16 round to nearest even, all finite inputs",
          2**32 - 2 * 2**23),
         (4, "v_cvt_pk_fp8_f32 with no clamp: every input above 448, up to +inf, gives 0x7E or 0x7F",
          0x7F800001 - 0x43E00001)]


@pytest.fixture(scope="module")
def hw():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        raise RuntimeError("tests/hw/libhwconv.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.hwconv_check.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_ulonglong)]
    L.hwconv_check.restype = ctypes.c_int
    return L


@pytest.mark.parametrize("which,what,inputs", CASES,
                         ids=["fp4-encode", "fp4-decode", "e4m3", "bf16", "e4m3-over-448"])
def test_conversion_matches_definition_on_every_input(hw, which, what, inputs):
    print("[hw] %s" % what, flush=True)
    sys.stdout.flush()
    out = (ctypes.c_ulonglong * 5)()
    assert hw.hwconv_check(which, out) == 0, "HIP error"
    assert out[0] == 0, "%s: %d mismatches, first input %08x hw %08x sw %08x" % (
        what, out[0], out[1], out[2], out[3])
    assert out[4] == inputs, "compared %d inputs, expected %d" % (out[4], inputs)
