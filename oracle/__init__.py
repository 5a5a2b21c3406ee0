"""CPU oracle for NVFP4 block-scaled quantization (rtn6 and Four Over Six).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``nvfp4_block_scaled_amax_amd``) never imports it, and the two share no code.

The arithmetic lives in ``nvfp4_oracle.cpp`` (plain C++17, brute-force rounding,
binary32 steps in the order the pages describe).  This module builds it with g++
and wraps it with ctypes over numpy arrays.

What pins each function (tests/test_oracle_pins.py, tests/test_oracle_shadow.py,
tests/test_oracle_mutants.py):
  e2m1_*, e4m3_*, bf16_rne   the printed FP4 value set, an independent threshold
                             formulation, torch's float8_e4m3fn and bfloat16 casts
  alpha                      closed forms and exact rationals
  quantize_block, candidate, worked examples derived by hand, exact-rational brute
  quantize                   force, the pages' 66.6 % and 75 % facts, invariants
  amax                       an independent numpy max over batches with NaN, +-Inf,
                             -0 and subnormals
  quantize_blocks            equal to quantize on every block id and on shuffled
                             subsets of batches with a different alpha per tensor
  dequantize                 closed forms; equal to the fake-quant output
  quantize_stats             hand-derived statistics and exact-rational sums
  shadow_block,              exact-rational brute force of the exact-quotient
  shadow_compare             reading, closed forms, and equality with the binary32
                             reading where no rounding intervenes
The planted-mistake tests build mutated copies of the C++ source and check that
the pins above reject each of them.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.cpp")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")

RTN6, FOUR_OVER_SIX = 0, 1
MSE, MAE, MAXERR = 0, 1, 2
MODES = {"rtn6": RTN6, "four_over_six": FOUR_OVER_SIX}
RULES = {"mse": MSE, "mae": MAE, "maxerr": MAXERR}


def build(force: bool = False) -> str:
    """Compile the oracle shared library with g++ (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "nvfp4_oracle.h"))):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
            "-shared", "-pthread", "-Wall", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


class _BlockDebug(ctypes.Structure):
    _fields_ = [("qstar", ctypes.c_int), ("s6", ctypes.c_uint8), ("s4", ctypes.c_uint8),
                ("err6", ctypes.c_float), ("err4", ctypes.c_float)]


class _ShadowCounts(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "blocks", "scale_diff", "choice_diff", "block_diff", "code_diff", "y_diff",
        "exact_ties", "inexact")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _bind(build())
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Route every function of this module to another build of the oracle for the duration
    (the planted-mistake tests load mutated copies of the source this way)."""
    global _lib
    saved = _lib
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def _bind(path: str) -> ctypes.CDLL:
    if True:
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_e2m1_decode.argtypes, L.orc_e2m1_decode.restype = [i32], f32
        L.orc_e2m1_round_mag.argtypes, L.orc_e2m1_round_mag.restype = [f32], i32
        L.orc_e2m1_round_mag_many.argtypes = [P, i64, P]
        L.orc_e4m3_decode.argtypes, L.orc_e4m3_decode.restype = [i32], ctypes.c_double
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [f32], i32
        L.orc_e4m3_encode_many.argtypes = [P, i64, P]
        L.orc_bf16_rne.argtypes, L.orc_bf16_rne.restype = [f32], ctypes.c_uint16
        L.orc_bf16_rne_many.argtypes = [P, i64, P]
        L.orc_alpha.argtypes, L.orc_alpha.restype = [f32, i32], f32
        L.orc_amax.argtypes, L.orc_amax.restype = [P, i64, i64, P], i32
        L.orc_quantize_block.argtypes = [P, f32, i32, i32, P, P, P, ctypes.POINTER(_BlockDebug)]
        L.orc_candidate.argtypes = [P, f32, i32, i32, P, P, P, P]
        L.orc_quantize.argtypes = [P, i64, i64, i64, i32, i32, P, P, P, P, P, i32]
        L.orc_quantize.restype = i32
        L.orc_quantize_blocks.argtypes = [P, i64, i64, i64, i32, i32, P, P, i64, P, P, P, P]
        L.orc_quantize_blocks.restype = i32
        L.orc_dequantize.argtypes = [P, P, P, i64, i64, i64, P]
        L.orc_dequantize.restype = i32
        L.orc_quantize_stats.argtypes = [P, i64, i64, i64, i32, i32, P, i32]
        L.orc_quantize_stats.restype = i32
        L.orc_inexact_subtractions.restype = i64
        L.orc_shadow_block.argtypes = [P, f32, i32, i32, i32, P, P, P, P]
        L.orc_shadow_compare.argtypes = [P, i64, i64, i64, i32, i32, i32,
                                         ctypes.POINTER(_ShadowCounts), i32]
        L.orc_shadow_compare.restype = i32
        L.orc_shadow_inexact.restype = i64
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _mode(m):
    return MODES[m] if isinstance(m, str) else int(m)


def _rule(r):
    return RULES[r] if isinstance(r, str) else int(r)


# ---- formats ------------------------------------------------------------------------
def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(code)


def e2m1_round_mag(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e2m1_round_mag_many(_p(a), a.size, _p(out))
    return out


def e4m3_decode(byte: int) -> float:
    return lib().orc_e4m3_decode(byte)


def e4m3_encode(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().orc_e4m3_encode_many(_p(s), s.size, _p(out))
    return out


def bf16_rne(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_bf16_rne_many(_p(f), f.size, _p(out))
    return out


def alpha(amax: float, mode) -> np.float32:
    return np.float32(lib().orc_alpha(float(amax), _mode(mode)))


# ---- tensors ------------------------------------------------------------------------
def amax(x_bits: np.ndarray, E: int = 1) -> np.ndarray:
    """x_bits: uint16 bf16 bit patterns, E tensors of equal size; returns float32 [E]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(E, np.float32)
    assert lib().orc_amax(_p(x), E, x.size // E, _p(out)) == 0
    return out


def quantize_block(x16_bits, alpha_, mode, rule):
    """One block; returns (codes[8] u8, scale u8, y[16] u16, debug dict)."""
    x = np.ascontiguousarray(x16_bits, dtype=np.uint16)
    assert x.size == 16
    codes = np.zeros(8, np.uint8)
    scale = np.zeros(1, np.uint8)
    y = np.zeros(16, np.uint16)
    dbg = _BlockDebug()
    lib().orc_quantize_block(_p(x), float(alpha_), _mode(mode), _rule(rule), _p(codes),
                             _p(scale), _p(y), ctypes.byref(dbg))
    return codes, int(scale[0]), y, dict(qstar=dbg.qstar, s6=dbg.s6, s4=dbg.s4,
                                         err6=dbg.err6, err4=dbg.err4)


def candidate(x16_bits, alpha_, Q: int, rule):
    """One candidate (Q = 6 or 4) alone: (magnitude codes[16], scale, xhat[16] f32, err)."""
    x = np.ascontiguousarray(x16_bits, dtype=np.uint16)
    mag = np.zeros(16, np.uint8)
    scale = np.zeros(1, np.uint8)
    xh = np.zeros(16, np.float32)
    err = np.zeros(1, np.float32)
    lib().orc_candidate(_p(x), float(alpha_), int(Q), _rule(rule), _p(mag), _p(scale),
                        _p(xh), _p(err))
    return mag, int(scale[0]), xh, np.float32(err[0])


def quantize(x_bits: np.ndarray, mode="four_over_six", rule="mse", nthreads: int = 1,
             want_y: bool = True, want_qstar: bool = False):
    """x_bits: uint16 array [rows, cols] or [E, rows, cols] (bf16 bit patterns).

    Returns dict(codes, scales, alpha, y, qstar) with the layouts of the C ABI."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    batched = x.ndim == 3
    E = x.shape[0] if batched else 1
    rows, cols = x.shape[-2], x.shape[-1]
    lead = (E,) if batched else ()
    codes = np.empty(lead + (rows, cols // 2), np.uint8)
    scales = np.empty(lead + (rows, cols // 16), np.uint8)
    al = np.empty(E, np.float32)
    y = np.empty(x.shape, np.uint16) if want_y else None
    q = np.empty(lead + (rows, cols // 16), np.uint8) if want_qstar else None
    rc = lib().orc_quantize(_p(x), E, rows, cols, _mode(mode), _rule(rule), _p(codes),
                            _p(scales), _p(al), _p(y) if y is not None else None,
                            _p(q) if q is not None else None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments (rc=%d)" % rc)
    return dict(codes=codes, scales=scales, alpha=al if batched else al[:1], y=y, qstar=q)


def quantize_blocks(x_bits: np.ndarray, alpha_: np.ndarray, ids: np.ndarray,
                    mode="four_over_six", rule="mse"):
    """Selected flat block ids of [E][rows][cols/16]; alpha_ is float32 [E]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    E = x.shape[0] if x.ndim == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    al = np.ascontiguousarray(alpha_, dtype=np.float32)
    codes = np.empty((ids.size, 8), np.uint8)
    scales = np.empty(ids.size, np.uint8)
    y = np.empty((ids.size, 16), np.uint16)
    q = np.empty(ids.size, np.uint8)
    rc = lib().orc_quantize_blocks(_p(x), E, rows, cols, _mode(mode), _rule(rule), _p(al),
                                   _p(ids), ids.size, _p(codes), _p(scales), _p(y), _p(q))
    if rc != 0:
        raise ValueError("oracle rejected arguments (rc=%d)" % rc)
    return dict(codes=codes, scales=scales, y=y, qstar=q)


def dequantize(codes: np.ndarray, scales: np.ndarray, alpha_: np.ndarray) -> np.ndarray:
    """Packed NVFP4 -> bf16 bit patterns; codes [..., rows, cols/2], scales [..., rows,
    cols/16], alpha [E]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    al = np.ascontiguousarray(alpha_, dtype=np.float32)
    E = c.shape[0] if c.ndim == 3 else 1
    rows, cols = c.shape[-2], c.shape[-1] * 2
    y = np.empty(c.shape[:-1] + (cols,), np.uint16)
    if lib().orc_dequantize(_p(c), _p(s), _p(al), E, rows, cols, _p(y)) != 0:
        raise ValueError("oracle rejected arguments")
    return y


# Columns of quantize_stats (same order as the oracle's ORC_STAT_* constants).
STATS = ("sse", "sae", "maxerr", "sse_near", "sse_f32scale", "near_count")


def quantize_stats(x_bits: np.ndarray, mode="four_over_six", rule="mse",
                   nthreads: int = 1) -> np.ndarray:
    """Per-tensor error statistics of the quantization -> float64 [E, 6], columns STATS:
    sum e^2, sum |e|, max |e|, sum e^2 over elements above 2/3 of their block max, sum e^2
    with binary32 block scales instead of E4M3, and the count of elements above 2/3 of
    their block max.  NaN rows for poisoned tensors."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    E = x.shape[0] if x.ndim == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    out = np.empty((E, len(STATS)), np.float64)
    rc = lib().orc_quantize_stats(_p(x), E, rows, cols, _mode(mode), _rule(rule), _p(out),
                                  int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments (rc=%d)" % rc)
    return out


def inexact_subtractions() -> int:
    return int(lib().orc_inexact_subtractions())


# ---- exact-quotient shadow (a diagnostic reading, not the parity target) -------------
def shadow_block(x16_bits, a, mode, rule, exact_alpha: bool = False):
    """One block under the exact-quotient reading: (codes[8] u8, scale u8, y[16] u16, qstar).
    a is the binary32 alpha, or with exact_alpha the tensor amax (alpha = amax / (6*M)
    exactly)."""
    x = np.ascontiguousarray(x16_bits, dtype=np.uint16)
    assert x.size == 16
    codes = np.zeros(8, np.uint8)
    scale = np.zeros(1, np.uint8)
    y = np.zeros(16, np.uint16)
    q = ctypes.c_int(0)
    lib().orc_shadow_block(_p(x), float(a), _mode(mode), _rule(rule), int(bool(exact_alpha)),
                           _p(codes), _p(scale), _p(y), ctypes.byref(q))
    return codes, int(scale[0]), y, q.value


def shadow_compare(x_bits: np.ndarray, mode="four_over_six", rule="mse",
                   exact_alpha: bool = False, nthreads: int = 1) -> dict:
    """Counts of what differs between the binary32 reading and the exact-quotient reading
    (after the binary32 alpha, or with exact_alpha fully exact) over whole tensors
    ([rows, cols] or [E, rows, cols])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    E = x.shape[0] if x.ndim == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    c = _ShadowCounts()
    rc = lib().orc_shadow_compare(_p(x), E, rows, cols, _mode(mode), _rule(rule),
                                  int(bool(exact_alpha)), ctypes.byref(c), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments (rc=%d)" % rc)
    return {name: int(getattr(c, name)) for name, _ in _ShadowCounts._fields_}


def shadow_inexact() -> int:
    """Failed exactness checks of the shadow's own arithmetic in shadow_block calls (0)."""
    return int(lib().orc_shadow_inexact())
