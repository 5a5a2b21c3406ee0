"""The allocation-free single-read call against the workspace-taking one (GPU, C ABI).

nvfp4_quantize_fused_noalloc keeps the grid-wide wait's counters in the library's static
device array; its outputs must equal nvfp4_quantize_fused's bit for bit (and the oracle's),
on consecutive calls that reuse the array, the second with a smaller input, across the
single-read tiers, the team tiers and the two-pass route."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_amax_amd as m
    m.lib()
    return m


def _outputs(shape):
    lead, (rows, cols) = tuple(shape[:-2]), shape[-2:]
    E = shape[0] if len(shape) == 3 else 1
    return (torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device="cuda"),
            torch.empty(lead + (rows, cols // 16), dtype=torch.uint8, device="cuda"),
            torch.empty(E, dtype=torch.float32, device="cuda"))


def _call(L, fn, x, E, rows, cols, mode, rule, outs, *extra):
    c, s, a = outs
    st = getattr(L, fn)(x.data_ptr(), E, rows, cols, 16, mode, rule, c.data_ptr(), s.data_ptr(),
                        a.data_ptr(), *extra, torch.cuda.current_stream().cuda_stream)
    assert st == 0, (fn, st)


# (shape, mode, rule): consecutive calls, each smaller than the one before it
SEQUENCES = [
    [((6, 1024, 16384), 1, 0), ((3, 256, 4096), 1, 1)],        # teams of 10, then all at once
    [((4096, 14336), 1, 0), ((256, 256), 0, 0)],               # 10 + 4 per lane, then 1 per lane
    [((600, 256, 256), 1, 2), ((40, 128, 512), 1, 0)],          # teams of 10, then smaller
    [((4096, 16384), 1, 0), ((1024, 4112), 1, 0)],              # two-pass route, then tier 4
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["teams", "tiers", "small-teams", "two-pass"])
def test_no_alloc_equals_workspace_call(nv, orc, seq):
    L = nv.lib()
    for shape, mode, rule in seq:
        E = shape[0] if len(shape) == 3 else 1
        rows, cols = shape[-2:]
        say("[no-alloc] %s mode=%d rule=%d tier=%d" % (
            shape, mode, rule, nv.fused_blocks_per_lane(shape, mode, rule, False)))
        xb = W.bits(W.generate("moe" if len(shape) == 3 else "weight", shape))
        x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda()
        a_out, b_out = _outputs(shape), _outputs(shape)
        for t in a_out + b_out:
            t.fill_(0x5A if t.dtype == torch.uint8 else 3.25)
        _call(L, "nvfp4_quantize_fused_noalloc", x, E, rows, cols, mode, rule, a_out)
        ws = torch.full((nv.FUSED_WS_WORDS * E,), -1, dtype=torch.int32, device="cuda")
        _call(L, "nvfp4_quantize_fused", x, E, rows, cols, mode, rule, b_out, ws.data_ptr())
        torch.cuda.synchronize()
        for p, q in zip(a_out, b_out):
            assert np.array_equal(p.cpu().numpy().view(np.uint8), q.cpu().numpy().view(np.uint8))
        ref = orc.quantize(xb, mode, rule, nthreads=NTHREADS, want_y=False)
        assert np.array_equal(a_out[0].cpu().numpy(), ref["codes"])
        assert np.array_equal(a_out[1].cpu().numpy(), ref["scales"])
        assert np.array_equal(a_out[2].cpu().numpy().view(np.uint32),
                              ref["alpha"][:E].view(np.uint32))


def test_no_alloc_rejects_more_tensors_than_the_scratch_holds(nv):
    x = torch.zeros((1025, 1, 16), dtype=torch.bfloat16, device="cuda")
    c, s, a = _outputs((1025, 1, 16))
    with pytest.raises(nv.NVFP4Error) as e:
        nv.quantize_fused_noalloc(x, codes=c, scales=s, alpha=a)
    assert e.value.status == 8
