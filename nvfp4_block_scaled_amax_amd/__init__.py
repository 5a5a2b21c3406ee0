"""NVFP4 block-scaled quantization (rtn6 and Four Over Six) on MI355X.

A thin ctypes binding over ``libnvfp4_amax.so`` (see ``include/nvfp4_amax.h``
for the operation, layouts and errors).  This module only marshals arguments:
torch provides device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  If the library is not built,
every call raises -- there is no fallback.

    codes, scales, alpha = quantize(x, "four_over_six", "mse")
    y, alpha = fakequant(x, "four_over_six", "mae")

x is a contiguous bf16 CUDA tensor [rows, cols] or [E, rows, cols] (a leading
expert dimension selects the batched entry points), cols % 16 == 0.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["quantize", "fakequant", "amax", "quantize_from_amax", "fakequant_from_amax",
           "dequantize", "quantize_diag", "quantize_fused", "fakequant_fused",
           "quantize_fused_noalloc", "fused_blocks_per_lane", "set_fused_wait_limit",
           "diag_ws_words", "lib",
           "NVFP4Error", "MODES", "RULES", "STATS", "FUSED_WS_WORDS", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_amax.so")
MODES = {"rtn6": 0, "four_over_six": 1}
RULES = {"mse": 0, "mae": 1, "maxerr": 2}
BLOCK = 16


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().nvfp4_status_str(status).decode()
        super().__init__("%s: %s (status %d)" % (where, msg, status))
        self.status = status


_lib = None
ABI_VERSION = 5                  # NVFP4_ABI_VERSION of include/nvfp4_amax.h
FUSED_WS_WORDS = 544             # NVFP4_FUSED_WS_WORDS: workspace int32 words per tensor


def diag_ws_words(E: int) -> int:
    """NVFP4_DIAG_WS_WORDS(E): int32 words of quantize_diag's statistics workspace."""
    return 32 * E + 12 * max(E, 1024)


# Columns of the per-tensor statistics of quantize_diag (NVFP4_STAT_* order).
STATS = ("sse", "sae", "maxerr", "sse_near", "sse_f32scale", "near_count")


def lib() -> ctypes.CDLL:
    """The C ABI with argument types set.  Raises if the HIP library is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnvfp4_amax.so is not built (run __graft_entry__.build() or "
                               "python -m nvfp4_block_scaled_amax_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.nvfp4_abi_version.restype = i32
        if L.nvfp4_abi_version() != ABI_VERSION:
            raise RuntimeError("libnvfp4_amax.so has ABI version %d, this binding needs %d: "
                               "rebuild it" % (L.nvfp4_abi_version(), ABI_VERSION))
        L.nvfp4_status_str.argtypes, L.nvfp4_status_str.restype = [i32], ctypes.c_char_p
        L.nvfp4_amax.argtypes = [P, i64, i64, i64, P, P]
        L.nvfp4_quantize.argtypes = [P, i64, i64, i32, i32, i32, P, P, P, P]
        L.nvfp4_fakequant.argtypes = [P, i64, i64, i32, i32, i32, P, P, P]
        L.nvfp4_quantize_batched.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P]
        L.nvfp4_fakequant_batched.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P]
        L.nvfp4_quantize_from_amax.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P, P]
        L.nvfp4_fakequant_from_amax.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P]
        L.nvfp4_dequantize.argtypes = [P, P, P, i64, i64, i64, P, P]
        L.nvfp4_quantize_diag.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.nvfp4_quantize_fused.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P, P]
        L.nvfp4_fakequant_fused.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P]
        L.nvfp4_quantize_fused_noalloc.argtypes = [P, i64, i64, i64, i32, i32, i32, P, P, P, P]
        L.nvfp4_fused_single_read.argtypes = [i64, i64, i64, i32, i32, i32]
        L.nvfp4_fused_single_read.restype = i32
        L.nvfp4_fused_set_wait_limit.argtypes = [i64]
        L.nvfp4_fused_set_wait_limit.restype = None
        for name in ("nvfp4_amax", "nvfp4_quantize", "nvfp4_fakequant", "nvfp4_quantize_batched",
                     "nvfp4_fakequant_batched", "nvfp4_quantize_from_amax",
                     "nvfp4_fakequant_from_amax", "nvfp4_dequantize", "nvfp4_quantize_diag",
                     "nvfp4_quantize_fused", "nvfp4_fakequant_fused",
                     "nvfp4_quantize_fused_noalloc"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise NVFP4Error(status, where)


def _mode(m) -> int:
    return MODES[m] if isinstance(m, str) else int(m)


def _rule(r) -> int:
    return RULES[r] if isinstance(r, str) else int(r)


def _dims(x: torch.Tensor):
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16, got %s" % x.dtype)
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1], False
    if x.dim() == 3:
        return x.shape[0], x.shape[1], x.shape[2], True
    raise ValueError("x must be [rows, cols] or [E, rows, cols]")


def _stream(x: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)


def _on(x: torch.Tensor):
    """x's device made current for the call: the library sizes its launches for the current
    device, and the stream passed is x's device's current stream."""
    return torch.cuda.device(x.device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _out(t, shape, dtype, like):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device != like.device:
        raise ValueError("output must be a contiguous %s tensor of shape %s on %s"
                         % (dtype, tuple(shape), like.device))
    return t


def amax(x: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """Per-tensor max |x| (float32 [E], E = 1 for a 2-D x)."""
    E, rows, cols, _ = _dims(x)
    out = _out(out, (E,), torch.float32, x)
    with _on(x):
        _check(lib().nvfp4_amax(_ptr(x), E, rows, cols, _ptr(out), _stream(x)), "nvfp4_amax")
    return out


def _packed_outputs(x, E, rows, cols, batched, codes, scales, alpha):
    lead = (E,) if batched else ()
    codes = _out(codes, lead + (rows, cols // 2), torch.uint8, x)
    scales = _out(scales, lead + (rows, cols // 16), torch.uint8, x)
    alpha = _out(alpha, (E,), torch.float32, x)
    return codes, scales, alpha


def quantize(x: torch.Tensor, mode="four_over_six", rule="mse", *, codes=None, scales=None,
             alpha=None):
    """Packed NVFP4 with a dynamic per-tensor scale -> (codes, scales, alpha)."""
    E, rows, cols, batched = _dims(x)
    codes, scales, alpha = _packed_outputs(x, E, rows, cols, batched, codes, scales, alpha)
    with _on(x):
        if batched:
            st = lib().nvfp4_quantize_batched(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                              _rule(rule), _ptr(codes), _ptr(scales),
                                              _ptr(alpha), _stream(x))
        else:
            st = lib().nvfp4_quantize(_ptr(x), rows, cols, BLOCK, _mode(mode), _rule(rule),
                                      _ptr(codes), _ptr(scales), _ptr(alpha), _stream(x))
    _check(st, "nvfp4_quantize")
    return codes, scales, alpha


def quantize_diag(x: torch.Tensor, mode="four_over_six", rule="mse", *, stats=True,
                  workspace=None):
    """Packed NVFP4 (dynamic scale) plus diagnostics ->
    (codes, scales, alpha, qstar, count4, stats): qstar uint8 [..., rows, cols/16] is 4 or 6
    per block, count4 int32 [E] counts the blocks scaled to 4, and stats float64 [E, 6]
    (columns STATS; None when stats=False) holds per-tensor error statistics.  workspace:
    int32 [diag_ws_words(E)], 128-byte aligned, for the statistics (allocated here if None)."""
    E, rows, cols, batched = _dims(x)
    codes, scales, alpha = _packed_outputs(x, E, rows, cols, batched, None, None, None)
    qstar = torch.empty_like(scales)
    count4 = torch.empty(E, dtype=torch.int32, device=x.device)
    st_out = ws = None
    if stats:
        st_out = torch.empty((E, len(STATS)), dtype=torch.float64, device=x.device)
        ws = _workspace(workspace, diag_ws_words(E), x)
    with _on(x):
        st = lib().nvfp4_quantize_diag(_ptr(x), E, rows, cols, BLOCK, _mode(mode), _rule(rule),
                                       _ptr(codes), _ptr(scales), _ptr(alpha), _ptr(qstar),
                                       _ptr(count4), _ptr(st_out) if stats else None,
                                       _ptr(ws) if stats else None, _stream(x))
    _check(st, "nvfp4_quantize_diag")
    return codes, scales, alpha, qstar, count4, st_out


def fakequant(x: torch.Tensor, mode="four_over_six", rule="mse", *, out=None, alpha=None):
    """bf16 quantize-dequantize with a dynamic per-tensor scale -> (y, alpha).
    out may be x itself (in place)."""
    E, rows, cols, batched = _dims(x)
    out = _out(out, x.shape, torch.bfloat16, x)
    alpha = _out(alpha, (E,), torch.float32, x)
    with _on(x):
        if batched:
            st = lib().nvfp4_fakequant_batched(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                               _rule(rule), _ptr(out), _ptr(alpha), _stream(x))
        else:
            st = lib().nvfp4_fakequant(_ptr(x), rows, cols, BLOCK, _mode(mode), _rule(rule),
                                       _ptr(out), _ptr(alpha), _stream(x))
    _check(st, "nvfp4_fakequant")
    return out, alpha


def quantize_from_amax(x: torch.Tensor, amax_: torch.Tensor, mode="four_over_six", rule="mse",
                       *, codes=None, scales=None, alpha=None):
    """Packed NVFP4 with a caller-supplied amax (float32 [E] on the GPU)."""
    E, rows, cols, batched = _dims(x)
    amax_ = _out(amax_, (E,), torch.float32, x)
    codes, scales, alpha = _packed_outputs(x, E, rows, cols, batched, codes, scales, alpha)
    with _on(x):
        st = lib().nvfp4_quantize_from_amax(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                            _rule(rule), _ptr(amax_), _ptr(codes), _ptr(scales),
                                            _ptr(alpha), _stream(x))
    _check(st, "nvfp4_quantize_from_amax")
    return codes, scales, alpha


def fakequant_from_amax(x: torch.Tensor, amax_: torch.Tensor, mode="four_over_six", rule="mse",
                        *, out=None, alpha=None):
    """bf16 quantize-dequantize with a caller-supplied amax."""
    E, rows, cols, batched = _dims(x)
    amax_ = _out(amax_, (E,), torch.float32, x)
    out = _out(out, x.shape, torch.bfloat16, x)
    alpha = _out(alpha, (E,), torch.float32, x)
    with _on(x):
        st = lib().nvfp4_fakequant_from_amax(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                             _rule(rule), _ptr(amax_), _ptr(out), _ptr(alpha),
                                             _stream(x))
    _check(st, "nvfp4_fakequant_from_amax")
    return out, alpha


def dequantize(codes: torch.Tensor, scales: torch.Tensor, alpha: torch.Tensor, *, out=None):
    """Packed NVFP4 -> bf16: codes uint8 [rows, cols/2] or [E, rows, cols/2], scales uint8
    [..., rows, cols/16], alpha float32 [E]; equal to the fake-quant output."""
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or alpha.dtype != torch.float32:
        raise TypeError("codes and scales must be uint8, alpha float32")
    if not (codes.is_cuda and scales.is_cuda and alpha.is_cuda):
        raise ValueError("codes, scales and alpha must be GPU tensors")
    if not (codes.is_contiguous() and scales.is_contiguous() and alpha.is_contiguous()):
        raise ValueError("codes, scales and alpha must be contiguous")
    if codes.dim() not in (2, 3):
        raise ValueError("codes must be [rows, cols/2] or [E, rows, cols/2]")
    E = codes.shape[0] if codes.dim() == 3 else 1
    rows, cols = codes.shape[-2], codes.shape[-1] * 2
    if tuple(scales.shape) != tuple(codes.shape[:-1]) + (cols // 16,) or alpha.numel() != E:
        raise ValueError("scales must be [..., rows, cols/16] and alpha [E]")
    out = _out(out, tuple(codes.shape[:-1]) + (cols,), torch.bfloat16, codes)
    with _on(codes):
        _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(alpha), E, rows, cols,
                                      _ptr(out), _stream(codes)), "nvfp4_dequantize")
    return out


# ----------------------------------------------------------------------------- single read
def _workspace(workspace, words, x):
    if workspace is None:
        return torch.empty(words, dtype=torch.int32, device=x.device)
    if (workspace.device != x.device or workspace.dtype not in (torch.int32, torch.uint32)
            or workspace.numel() < words or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous int32 tensor of at least %d elements "
                         "on x's device" % words)
    return workspace


def quantize_fused(x: torch.Tensor, mode="four_over_six", rule="mse", *, codes=None,
                   scales=None, alpha=None, workspace=None):
    """Packed NVFP4 with a dynamic scale, reading x once when it fits on chip -> (codes,
    scales, alpha), identical to quantize().  workspace: int32 [FUSED_WS_WORDS * E], 128-byte
    aligned (allocated here if None)."""
    E, rows, cols, batched = _dims(x)
    codes, scales, alpha = _packed_outputs(x, E, rows, cols, batched, codes, scales, alpha)
    ws = _workspace(workspace, FUSED_WS_WORDS * E, x)
    with _on(x):
        st = lib().nvfp4_quantize_fused(_ptr(x), E, rows, cols, BLOCK, _mode(mode), _rule(rule),
                                        _ptr(codes), _ptr(scales), _ptr(alpha), _ptr(ws),
                                        _stream(x))
    _check(st, "nvfp4_quantize_fused")
    return codes, scales, alpha


NOALLOC_MAX_TENSORS = 1024      # NVFP4_NOALLOC_MAX_TENSORS


def quantize_fused_noalloc(x: torch.Tensor, mode="four_over_six", rule="mse", *, codes,
                           scales, alpha):
    """quantize_fused() whose wait counters live in the library's static device array: the
    library allocates nothing (for callers that cannot allocate).  The outputs must be given.
    Calls that may overlap on one GPU race on that array."""
    E, rows, cols, batched = _dims(x)
    codes, scales, alpha = _packed_outputs(x, E, rows, cols, batched, codes, scales, alpha)
    with _on(x):
        st = lib().nvfp4_quantize_fused_noalloc(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                                _rule(rule), _ptr(codes), _ptr(scales),
                                                _ptr(alpha), _stream(x))
    _check(st, "nvfp4_quantize_fused_noalloc")
    return codes, scales, alpha


def fakequant_fused(x: torch.Tensor, mode="four_over_six", rule="mse", *, out=None, alpha=None,
                    workspace=None):
    """bf16 quantize-dequantize with a dynamic scale, reading x once when it fits on chip ->
    (y, alpha), identical to fakequant()."""
    E, rows, cols, batched = _dims(x)
    out = _out(out, x.shape, torch.bfloat16, x)
    alpha = _out(alpha, (E,), torch.float32, x)
    ws = _workspace(workspace, FUSED_WS_WORDS * E, x)
    with _on(x):
        st = lib().nvfp4_fakequant_fused(_ptr(x), E, rows, cols, BLOCK, _mode(mode),
                                         _rule(rule), _ptr(out), _ptr(alpha), _ptr(ws),
                                         _stream(x))
    _check(st, "nvfp4_fakequant_fused")
    return out, alpha


def fused_blocks_per_lane(shape, mode="four_over_six", rule="mse", fakequant=False) -> int:
    """Most blocks a lane holds on chip in a fused call of this shape (1, 4, 10, 12, 14 or 28;
    20 for a batch read by teams of workgroups that take its tensors in turn, 10 when those
    tensors have under 262,144 blocks, 10 or 13 when the output is Four Over Six packed), or 0
    when the call takes the two-pass path (on the current device)."""
    shape = tuple(shape)
    if len(shape) not in (2, 3):
        raise ValueError("shape must be (rows, cols) or (E, rows, cols)")
    E = shape[0] if len(shape) == 3 else 1
    r = lib().nvfp4_fused_single_read(E, shape[-2], shape[-1], _mode(mode), _rule(rule),
                                      int(bool(fakequant)))
    if r < 0:
        raise ValueError("nvfp4_fused_single_read: %s" % lib().nvfp4_status_str(-r).decode())
    return int(r)


def set_fused_wait_limit(polls: int) -> None:
    """Test hook: polls before a fused workgroup stops waiting for the others and computes the
    tensor amax itself (0 = never wait, negative = the default)."""
    lib().nvfp4_fused_set_wait_limit(int(polls))
