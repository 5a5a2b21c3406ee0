"""No entry point writes outside its outputs (GPU, through the C ABI).

Every output array, every workspace and the input of each call sit inside a larger device
buffer whose bytes around them hold a canary pattern (and the outputs themselves start with
it).  After the call the guard bytes must be unchanged, the input must be unchanged, only
the documented part of a workspace may have changed, and the outputs must equal the
oracle's (so the canary inside them was overwritten everywhere).  Covered: the dynamic,
batched and fixed-scale calls, amax, dequantize, the diagnostics call with and without
statistics, and the single-read calls in every tier of blocks per lane and in every team
tier.  Outputs start at odd offsets where their alignment allows (scale bytes, qstar)."""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
CANARY = 0xA5
GUARD = 4096                      # bytes on each side (a multiple of every alignment needed)


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


class Guarded:
    """A device array of `shape` and `dtype` inside GUARD bytes of canary on each side,
    starting `skew` elements after the guard; the array itself starts as canary too."""

    def __init__(self, shape, dtype, skew=0, init=None):
        esz = torch.empty((), dtype=dtype).element_size()
        self.n = math.prod(shape)
        self.lo = GUARD // esz + skew
        total = self.lo + self.n + GUARD // esz
        self.buf = torch.empty(total, dtype=dtype, device="cuda")
        self.buf.view(torch.uint8).fill_(CANARY)
        self.t = self.buf[self.lo:self.lo + self.n].view(shape)
        if init is not None:
            self.t.copy_(init)
        self.esz = esz

    def guards_intact(self) -> bool:
        b = self.buf.view(torch.uint8).cpu().numpy()
        a, z = self.lo * self.esz, (self.lo + self.n) * self.esz
        return bool((b[:a] == CANARY).all() and (b[z:] == CANARY).all())


def bits_gpu(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16)


def u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_packed(orc, x, c, s, a, mode, rule, tag):
    ref = orc.quantize(x, mode, rule, nthreads=NTHREADS, want_y=False)
    E = x.shape[0] if x.ndim == 3 else 1
    assert np.array_equal(a.t.cpu().numpy().view(np.uint32), ref["alpha"][:E].view(np.uint32)), tag
    assert np.array_equal(c.t.cpu().numpy(), ref["codes"]), tag
    assert np.array_equal(s.t.cpu().numpy(), ref["scales"]), tag


def _check_fq(orc, x, y, a, mode, rule, tag):
    ref = orc.quantize(x, mode, rule, nthreads=NTHREADS, want_y=True)
    E = x.shape[0] if x.ndim == 3 else 1
    assert np.array_equal(a.t.cpu().numpy().view(np.uint32), ref["alpha"][:E].view(np.uint32)), tag
    assert np.array_equal(u16(y.t), ref["y"]), tag


def _packed_bufs(shape):
    lead = shape[:-2]
    rows, cols = shape[-2:]
    E = shape[0] if len(shape) == 3 else 1
    return (Guarded(lead + (rows, cols // 2), torch.uint8),
            Guarded(lead + (rows, cols // 16), torch.uint8, skew=3),
            Guarded((E,), torch.float32, skew=1))


def _all_intact(*gs):
    return all(g.guards_intact() for g in gs)


SHAPES = [(33, 240), (3, 17, 96), (1, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=["ragged", "batched", "one-block"])
@pytest.mark.parametrize("mode,rule", [("four_over_six", "mse"), ("rtn6", "mse")])
def test_dynamic_fixed_and_amax_calls(nv, orc, shape, mode, rule):
    x = W.bits(W.generate("large", shape))
    xg = Guarded(shape, torch.bfloat16, init=bits_gpu(x))
    E = shape[0] if len(shape) == 3 else 1
    tag = "%s %s" % (shape, mode)
    # dynamic, packed and fake-quant (batched entry points for 3-D shapes)
    c, s, a = _packed_bufs(shape)
    nv.quantize(xg.t, mode, rule, codes=c.t, scales=s.t, alpha=a.t)
    y, a2 = Guarded(shape, torch.bfloat16), Guarded((E,), torch.float32, skew=1)
    nv.fakequant(xg.t, mode, rule, out=y.t, alpha=a2.t)
    # amax, then the fixed-scale calls from it
    am = Guarded((E,), torch.float32, skew=1)
    nv.amax(xg.t, out=am.t)
    c3, s3, a3 = _packed_bufs(shape)
    nv.quantize_from_amax(xg.t, am.t, mode, rule, codes=c3.t, scales=s3.t, alpha=a3.t)
    y4, a4 = Guarded(shape, torch.bfloat16), Guarded((E,), torch.float32, skew=1)
    nv.fakequant_from_amax(xg.t, am.t, mode, rule, out=y4.t, alpha=a4.t)
    torch.cuda.synchronize()
    assert _all_intact(xg, c, s, a, y, a2, am, c3, s3, a3, y4, a4), tag
    assert np.array_equal(u16(xg.t), x), tag                   # the input is untouched
    assert np.array_equal(am.t.cpu().numpy(), orc.amax(x, E)), tag
    _check_packed(orc, x, c, s, a, mode, rule, tag)
    _check_packed(orc, x, c3, s3, a3, mode, rule, tag)
    _check_fq(orc, x, y, a2, mode, rule, tag)
    _check_fq(orc, x, y4, a4, mode, rule, tag)


@pytest.mark.parametrize("shape", SHAPES, ids=["ragged", "batched", "one-block"])
def test_dequantize(nv, orc, shape):
    x = W.bits(W.generate("weight", shape))
    E = shape[0] if len(shape) == 3 else 1
    ref = orc.quantize(x, "four_over_six", "mae", want_y=True)
    lead, (rows, cols) = shape[:-2], shape[-2:]
    cg = Guarded(lead + (rows, cols // 2), torch.uint8, init=torch.from_numpy(ref["codes"]))
    sg = Guarded(lead + (rows, cols // 16), torch.uint8, skew=5,
                 init=torch.from_numpy(ref["scales"]))
    ag = Guarded((E,), torch.float32, skew=3, init=torch.from_numpy(ref["alpha"][:E]))
    yg = Guarded(shape, torch.bfloat16)
    nv.dequantize(cg.t, sg.t, ag.t, out=yg.t)
    torch.cuda.synchronize()
    assert _all_intact(cg, sg, ag, yg)
    assert np.array_equal(cg.t.cpu().numpy(), ref["codes"])    # inputs untouched
    assert np.array_equal(sg.t.cpu().numpy(), ref["scales"])
    assert np.array_equal(u16(yg.t), ref["y"])


def _diag_ws_words(E):
    return 32 * E + 12 * max(E, 1024)


@pytest.mark.parametrize("shape", SHAPES[:2], ids=["ragged", "batched"])
@pytest.mark.parametrize("with_stats", [False, True], ids=["choice", "stats"])
def test_diagnostics(nv, orc, shape, with_stats):
    x = W.bits(W.generate("weight", shape))
    E = shape[0] if len(shape) == 3 else 1
    xg = Guarded(shape, torch.bfloat16, init=bits_gpu(x))
    c, s, a = _packed_bufs(shape)
    q = Guarded(tuple(s.t.shape), torch.uint8, skew=7)
    n4 = Guarded((E,), torch.int32, skew=1)
    st = Guarded((E, 6), torch.float64, skew=1) if with_stats else None
    ws = Guarded((_diag_ws_words(E),), torch.int32) if with_stats else None
    L = nv.lib()
    status = L.nvfp4_quantize_diag(
        xg.t.data_ptr(), E, shape[-2], shape[-1], 16, 1, 0, c.t.data_ptr(), s.t.data_ptr(),
        a.t.data_ptr(), q.t.data_ptr(), n4.t.data_ptr(),
        st.t.data_ptr() if st else None, ws.t.data_ptr() if ws else None,
        torch.cuda.current_stream().cuda_stream)
    assert status == 0
    torch.cuda.synchronize()
    gs = [xg, c, s, a, q, n4] + ([st, ws] if with_stats else [])
    assert _all_intact(*gs)
    assert np.array_equal(u16(xg.t), x)
    ref = orc.quantize(x, "four_over_six", "mse", want_y=False, want_qstar=True)
    _check_packed(orc, x, c, s, a, "four_over_six", "mse", "diag")
    assert np.array_equal(q.t.cpu().numpy(), ref["qstar"])
    assert np.array_equal(n4.t.cpu().numpy(), (ref["qstar"].reshape(E, -1) == 4).sum(axis=1))
    if with_stats:
        want = orc.quantize_stats(x, "four_over_six", "mse")
        got = st.t.cpu().numpy()
        assert np.array_equal(got[:, [2, 5]], want[:, [2, 5]])     # max |e| and the count: exact
        assert np.allclose(got, want, rtol=1e-12, atol=0)


# Single-read calls: every tier of blocks held per lane, and every team tier.
FUSED = [((256, 256), 1), ((1024, 4112), None), ((4096, 4112), 10), ((8192, 4096), 10),
         ((100, 328, 1024), None), ((4096, 14336), 14),
         ((40, 256, 256), None), ((600, 256, 256), 10), ((6, 1024, 16384), 20),
         ((10, 1024, 8192), 20), ((6, 3072, 4096), None), ((3, 4096, 4096), None)]


@pytest.mark.parametrize("shape,tier", FUSED, ids=[str(s) for s, _ in FUSED])
@pytest.mark.parametrize("mode,rule,fq", [("four_over_six", "mse", False), ("rtn6", "mse", True)],
                         ids=["46mse-packed", "rtn6-fq"])
def test_fused(nv, orc, shape, tier, mode, rule, fq):
    got_tier = nv.fused_blocks_per_lane(shape, mode, rule, fq)
    say("[canary-fused] %s %s fq=%s: %d blocks per lane" % (shape, mode, fq, got_tier))
    if tier == 20 and not fq and mode == "four_over_six":
        tier = 10                           # the wide-workgroup team tiers (1024 / 512 threads)
    if tier is not None:
        assert got_tier == tier
    assert got_tier > 0
    x = W.bits(W.generate("moe" if len(shape) == 3 else "weight", shape))
    E = shape[0] if len(shape) == 3 else 1
    xg = Guarded(shape, torch.bfloat16, init=bits_gpu(x))
    words = E * nv.FUSED_WS_WORDS
    ws = Guarded((words,), torch.int32)
    if fq:
        y, a = Guarded(shape, torch.bfloat16), Guarded((E,), torch.float32, skew=1)
        nv.fakequant_fused(xg.t, mode, rule, out=y.t, alpha=a.t, workspace=ws.t)
        outs = [y, a]
    else:
        c, s, a = _packed_bufs(shape)
        nv.quantize_fused(xg.t, mode, rule, codes=c.t, scales=s.t, alpha=a.t, workspace=ws.t)
        outs = [c, s, a]
    torch.cuda.synchronize()
    assert _all_intact(xg, ws, *outs)
    assert np.array_equal(u16(xg.t), x)
    if fq:
        _check_fq(orc, x, y, a, mode, rule, str(shape))
    else:
        _check_packed(orc, x, c, s, a, mode, rule, str(shape))
