"""C-ABI boundary tests that need no GPU.

The library must load on a machine without a GPU, export every entry point that
include/nvfp4_amax.h declares, and reject bad arguments before touching HIP (so
these calls never reach a device).  Python-side checks of the binding are
covered too.
"""
from __future__ import annotations

import ctypes
import os
import re
import sys

import pytest
import torch

import nvfp4_block_scaled_amax_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_amax.h")

OK, ENULL, ESHAPE, EBLOCK, EENUM, EALIGN, EHIP, EALIAS, ESCRATCH = range(9)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_block_scaled_amax_amd import build
        build.build_library()
    return nv.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status|int|void|const char\*)\s+(nvfp4_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(["nvfp4_abi_version", "nvfp4_status_str", "nvfp4_amax",
                            "nvfp4_quantize", "nvfp4_fakequant", "nvfp4_quantize_batched",
                            "nvfp4_fakequant_batched", "nvfp4_quantize_from_amax",
                            "nvfp4_fakequant_from_amax", "nvfp4_dequantize",
                            "nvfp4_quantize_diag", "nvfp4_quantize_fused",
                            "nvfp4_fakequant_fused", "nvfp4_fused_single_read",
                            "nvfp4_fused_set_wait_limit", "nvfp4_quantize_fused_noalloc"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.nvfp4_abi_version() == 5
    for st in range(9):
        assert L.nvfp4_status_str(st) != b"unknown status"
    assert L.nvfp4_status_str(99) == b"unknown status"


# Fake, never dereferenced addresses: every call below fails validation first.
A = 0x100000          # 16-byte aligned
B = 0x900000
C = 0x1100000
D = 0x1900000


def q(L, in_=A, rows=4, cols=32, block=16, mode=1, rule=0, codes=B, scales=C, alpha=D):
    return L.nvfp4_quantize(in_, rows, cols, block, mode, rule, codes, scales, alpha, None)


def test_quantize_rejects_bad_arguments(L):
    assert q(L, in_=None) == ENULL
    assert q(L, codes=None) == ENULL
    assert q(L, scales=None) == ENULL
    assert q(L, alpha=None) == ENULL
    assert q(L, rows=0) == ESHAPE
    assert q(L, rows=-3) == ESHAPE
    assert q(L, cols=0) == ESHAPE
    assert q(L, cols=24) == ESHAPE
    assert q(L, rows=1 << 40, cols=1 << 40) == ESHAPE
    assert q(L, block=32) == EBLOCK
    assert q(L, block=0) == EBLOCK
    assert q(L, mode=2) == EENUM
    assert q(L, mode=-1) == EENUM
    assert q(L, rule=3) == EENUM
    assert q(L, mode=0, rule=7) == EENUM          # validated even though rtn6 ignores it
    assert q(L, in_=A + 8) == EALIGN
    assert q(L, codes=B + 4) == EALIGN
    assert q(L, alpha=D + 2) == EALIGN
    assert q(L, codes=A + 16) == EALIAS            # codes overlap the input
    assert q(L, alpha=A + 64) == EALIAS            # the amax accumulator overlaps the input
    assert q(L, scales=B + 8) == EALIAS            # scales overlap codes
    qb = L.nvfp4_quantize_batched
    assert qb(A, 65536, 1, 16, 16, 1, 0, B, C, D, None) == ESHAPE   # grid y holds 65535 tensors
    assert qb(A, 0, 1, 16, 16, 1, 0, B, C, D, None) == ESHAPE
    assert qb(A, 65535, 1, 16, 16, 1, 0, B, C, A, None) == EALIAS   # shape accepted; alpha in input


def test_fakequant_rejects_bad_arguments_and_partial_overlap(L):
    f = L.nvfp4_fakequant
    assert f(A, 4, 32, 16, 1, 0, None, D, None) == ENULL
    assert f(A, 4, 32, 16, 1, 0, B + 2, D, None) == EALIGN
    assert f(A, 4, 32, 16, 1, 0, A + 32, D, None) == EALIAS   # partial overlap with input
    assert f(A, 4, 32, 16, 1, 0, B, A + 4, None) == EALIAS    # alpha inside the input
    assert f(A, 4, 32, 16, 4, 0, B, D, None) == EENUM


def test_batched_amax_and_fixed_scale_validation(L):
    assert L.nvfp4_quantize_batched(A, 0, 4, 32, 16, 1, 0, B, C, D, None) == ESHAPE
    assert L.nvfp4_quantize_batched(A, 70000, 4, 32, 16, 1, 0, B, C, D, None) == ESHAPE
    assert L.nvfp4_fakequant_batched(A, 2, 4, 33, 16, 1, 0, B, D, None) == ESHAPE
    assert L.nvfp4_amax(None, 1, 4, 32, D, None) == ENULL
    assert L.nvfp4_amax(A, 1, 4, 32, None, None) == ENULL
    assert L.nvfp4_amax(A, 1, 4, 20, D, None) == ESHAPE
    assert L.nvfp4_amax(A, 1, 4, 32, D + 1, None) == EALIGN
    assert L.nvfp4_amax(A, 1, 4, 32, A + 4, None) == EALIAS
    assert L.nvfp4_quantize_from_amax(A, 1, 4, 32, 16, 1, 0, None, B, C, D, None) == ENULL
    assert L.nvfp4_quantize_from_amax(A, 1, 4, 32, 16, 1, 0, D + 2, B, C, D + 64, None) == EALIGN
    assert L.nvfp4_quantize_from_amax(A, 2, 4, 32, 16, 1, 0, D + 4, B, C, D, None) == EALIAS
    assert L.nvfp4_fakequant_from_amax(A, 1, 4, 32, 16, 1, 0, None, B, D, None) == ENULL
    assert L.nvfp4_fakequant_from_amax(A, 1, 4, 32, 16, 1, 9, D, B, D, None) == EENUM


def test_dequantize_validation(L):
    f = L.nvfp4_dequantize
    assert f(None, C, D, 1, 4, 32, A, None) == ENULL
    assert f(B, C, D, 1, 4, 30, A, None) == ESHAPE
    assert f(B + 4, C, D, 1, 4, 32, A, None) == EALIGN
    assert f(B, C, D, 1, 4, 32, A + 8, None) == EALIGN
    assert f(B, C, D, 1, 4, 32, B + 16, None) == EALIAS      # output over the codes


def test_diag_validation(L):
    f = L.nvfp4_quantize_diag
    W = 0x2100000
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, None, D + 64, None, None, None) == ENULL
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, None, None, None, None) == ENULL
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 66, None, None, None) == EALIGN
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C, D + 64, None, None, None) == EALIAS    # qstar over scales
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, A + 8, None, None, None) == EALIAS  # count4 in input
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 132, W, None) == EALIGN  # stats
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 64, W, None) == EALIAS   # over count4
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, A + 64, W, None) == EALIAS   # in input
    # the statistics workspace: required with stats, 128-byte aligned, apart from the rest
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 128, None, None) == ENULL
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 128, W + 64, None) == EALIGN
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 128, A + 128, None) == EALIAS
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 128, D + 128, None) == EALIAS
    assert f(A, 1, 4, 32, 16, 1, 0, B, C, D, C + 1024, D + 64, W, C + 896, None) == EALIAS  # over qstar
    assert f(A, 1, 4, 30, 16, 1, 0, B, C, D, C + 1024, D + 64, D + 128, W, None) == ESHAPE


def test_fused_validation(L):
    fq = L.nvfp4_quantize_fused
    ff = L.nvfp4_fakequant_fused
    W = 0x2100000
    assert fq(A, 1, 4, 32, 16, 1, 0, B, C, D, None, None) == ENULL          # no workspace
    assert fq(A, 1, 4, 32, 16, 1, 0, B, C, D, W + 64, None) == EALIGN       # 128-byte lines
    assert fq(A, 1, 4, 32, 16, 1, 0, B, C, D, A + 128, None) == EALIAS      # in the input
    assert fq(A, 1, 4, 32, 16, 1, 0, B, C, D, D, None) == EALIAS            # over alpha
    assert fq(A, 1, 4, 32, 16, 1, 0, B, C, D, C - 128, None) == EALIAS      # over the scales
    assert fq(A, 1, 4, 30, 16, 1, 0, B, C, D, W, None) == ESHAPE
    assert fq(A, 1, 4, 32, 16, 2, 0, B, C, D, W, None) == EENUM
    assert ff(A, 1, 4, 32, 16, 1, 0, B, D, None, None) == ENULL
    assert ff(A, 1, 4, 32, 16, 1, 0, B, D, B, None) == EALIAS              # over the output
    # the allocation-free variant: the same validation, and at most 1024 tensors
    fn = L.nvfp4_quantize_fused_noalloc
    assert fn(A, 1, 4, 32, 16, 1, 0, B, C, None, None) == ENULL
    assert fn(A, 1, 4, 30, 16, 1, 0, B, C, D, None) == ESHAPE
    assert fn(A, 1, 4, 32, 16, 1, 0, A + 16, C, D, None) == EALIAS
    assert fn(A, 1025, 1, 16, 16, 1, 0, B, C, D, None) == ESCRATCH
    assert fn(A, 1025, 1, 16, 16, 3, 0, B, C, D, None) == EENUM   # argument errors come first
    assert nv.NOALLOC_MAX_TENSORS == 1024
    # the shape query needs no GPU for argument errors
    assert L.nvfp4_fused_single_read(1, 4, 30, 1, 0, 0) == -ESHAPE
    assert L.nvfp4_fused_single_read(1, 4, 32, 3, 0, 0) == -EENUM
    assert L.nvfp4_fused_single_read(0, 4, 32, 1, 0, 0) == -ESHAPE


def test_python_binding_checks_inputs():
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.quantize(x)                                   # not on a GPU
    with pytest.raises(TypeError):
        nv.quantize(torch.zeros(4, 32, dtype=torch.float32))
    with pytest.raises(ValueError):
        nv.fakequant(torch.zeros(2, 2, 4, 32, dtype=torch.bfloat16))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "nvfp4_block_scaled_amax_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), fn
                assert "nvfp4_oracle" not in text, fn


def test_build_rejects_kernels_that_spill():
    from nvfp4_block_scaled_amax_amd import build
    report = "\n".join([
        "k.hip:1:1: remark: Function Name: a_kernel [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:9:1: remark: Function Name: b_kernel [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:9:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]"])
    assert build.scratch_users(report) == [("b_kernel", 24)]
    assert build.scratch_users(report.replace(": 24 ", ": 0 ")) == []


def test_counter_digest_ignores_comments_only(tmp_path):
    """The committed HBM-traffic figure is tied to the kernel source's code: comments and
    layout do not change the digest, code and string literals do."""
    sys.path.insert(0, ROOT)
    import bench
    base = 'int a = 1; // note\n/* block */ const char* s = "x // y"; char q = \'"\';\n'
    variants = {
        "comment": ('int a = 1;   // another note\n/* other */ const char* s = "x // y"; '
                    'char q = \'"\';\n', True),
        "code": ('int a = 2; // note\n/* block */ const char* s = "x // y"; char q = \'"\';\n',
                 False),
        "literal": ('int a = 1; // note\n/* block */ const char* s = "x // z"; char q = \'"\';\n',
                    False),
    }
    p = tmp_path / "k.hip"
    p.write_text(base)
    d0 = bench.source_digest(str(p))
    for name, (text, same) in variants.items():
        p.write_text(text)
        assert (bench.source_digest(str(p)) == d0) == same, name
