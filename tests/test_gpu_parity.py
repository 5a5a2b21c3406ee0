"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit.

Codes, scale bytes, alpha bits and fake-quant bf16 bits must be identical (the
arithmetic is binary32 round-to-nearest-even in a fixed order on both sides, so
the bar is exact equality).  Small tensors and the five full-size workloads (in the
launch configuration the benchmark times) are compared whole, plus a property that holds
at any size (decoding the packed output gives the fake-quant output)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from helpers import bf16_bits, bf16_to_f32
from nvfp4_block_scaled_amax_amd import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
RUNS = [("rtn6", "mse"), ("four_over_six", "mse"), ("four_over_six", "mae"),
        ("four_over_six", "maxerr")]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_amax_amd as m
    m.lib()          # raises if the HIP library is missing: no fallback
    return m


def to_gpu(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_run(nv, xg, mode, rule, fq):
    if fq:
        y, al = nv.fakequant(xg, mode, rule)
        torch.cuda.synchronize()
        return dict(y=u16(y), alpha=al.cpu().numpy())
    c, s, al = nv.quantize(xg, mode, rule)
    torch.cuda.synchronize()
    return dict(codes=c.cpu().numpy(), scales=s.cpu().numpy(), alpha=al.cpu().numpy())


def assert_same(got, ref, fq, tag):
    assert np.array_equal(got["alpha"].view(np.uint32),
                          np.asarray(ref["alpha"], np.float32).view(np.uint32)), tag
    if fq:
        bad = np.nonzero(got["y"].ravel() != ref["y"].ravel())[0]
        assert bad.size == 0, "%s: %d fake-quant mismatches, first at %s" % (tag, bad.size, bad[:4])
    else:
        bs = np.nonzero(got["scales"].ravel() != ref["scales"].ravel())[0]
        assert bs.size == 0, "%s: %d scale mismatches, first blocks %s" % (tag, bs.size, bs[:4])
        bc = np.nonzero(got["codes"].ravel() != ref["codes"].ravel())[0]
        assert bc.size == 0, "%s: %d code-byte mismatches, first at %s" % (tag, bc.size, bc[:4])


def check_full(nv, orc, xbits, mode, rule, fq, tag):
    say("[parity] %s shape=%s mode=%s rule=%s fq=%s" % (tag, xbits.shape, mode, rule, fq))
    got = gpu_run(nv, to_gpu(xbits), mode, rule, fq)
    ref = orc.quantize(xbits, mode, rule, nthreads=NTHREADS, want_y=fq)
    assert_same(got, ref, fq, tag)


# ----------------------------------------------------------------------------- small, whole
def test_tiny_workload_both_runs(nv, orc):
    x = W.bits(W.generate("tiny"))
    for mode, rule in (("rtn6", "mse"), ("four_over_six", "mse")):
        for fq in (False, True):
            check_full(nv, orc, x, mode, rule, fq, "tiny")


SMALL = [("tiny", (300, 272)), ("weight", (200, 1792)), ("act", (301, 1024)),
         ("large", (97, 3584)), ("moe", (5, 130, 320))]


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
@pytest.mark.parametrize("fq", [False, True], ids=["packed", "fakequant"])
def test_small_workloads_whole(nv, orc, name, shape, mode, rule, fq):
    """Several workgroups per tensor and a ragged last workgroup."""
    check_full(nv, orc, W.bits(W.generate(name, shape)), mode, rule, fq, name)


def test_random_shapes(nv, orc):
    rng = np.random.default_rng(77)
    for k in range(24):
        rows = int(rng.integers(1, 34))
        cols = int(rng.integers(1, 257)) * 16
        E = int(rng.integers(1, 4)) if k % 3 == 0 else None
        shape = (E, rows, cols) if E else (rows, cols)
        x = W.bits(W.normal(shape, seed=1000 + k, sigma=float(np.exp(rng.uniform(-8, 8)))))
        mode, rule = RUNS[k % 4]
        check_full(nv, orc, x, mode, rule, bool(k % 2), "random%d" % k)


# ----------------------------------------------------------------------------- edge cases
def _edge_tensors():
    rng = np.random.default_rng(5)
    out = {}
    z = np.zeros((4, 64), np.uint16)
    z[1, 3] = 0x8000
    z[2, :] = 0x8000
    out["zeros"] = z
    # every bf16 magnitude from subnormal up, so alpha is a binary32 subnormal and the
    # E4M3 clamp and the 1/d-overflow division path are live
    out["subnormal"] = (rng.integers(0, 0x0180, size=(8, 128), dtype=np.uint16) |
                        (rng.integers(0, 2, size=(8, 128), dtype=np.uint16) << 15))
    out["tiny_normal"] = (rng.integers(0x0080, 0x0800, size=(8, 128), dtype=np.uint16) |
                          (rng.integers(0, 2, size=(8, 128), dtype=np.uint16) << 15))
    big = rng.integers(0x7E00, 0x7F80, size=(6, 96), dtype=np.uint16)
    big[0, 0] = 0x7F7F                                   # the largest finite bf16
    out["huge"] = big | (rng.integers(0, 2, size=big.shape, dtype=np.uint16) << 15)
    # dense exact ties: many blocks whose values sit on FP4 midpoints
    t = bf16_bits(np.tile(np.array([6, 5, 3.5, 2.5, 1.75, 1.25, .75, .25, -5, -3.5, -2.5,
                                    -1.75, -1.25, -.75, -.25, 0], np.float32), (16, 4)))
    out["ties"] = t
    # blocks far below the tensor amax (scale byte 0 and subnormal scales)
    w = W.bits(W.normal((16, 256), seed=9, sigma=1e-4))
    w[0, 0] = bf16_bits([28672.0])[0]
    out["dynamic_range"] = w
    out["one_row_one_block"] = W.bits(W.normal((1, 16), seed=10))
    out["one_column_of_blocks"] = W.bits(W.normal((37, 16), seed=11))
    return out


EDGE = _edge_tensors()


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
def test_edge_cases(nv, orc, name, mode, rule):
    for fq in (False, True):
        check_full(nv, orc, EDGE[name], mode, rule, fq, name)


@pytest.mark.parametrize("bad", [0x7FC0, 0x7F80, 0xFF80, 0xFFC1])
def test_non_finite_poisons_only_its_tensor(nv, orc, bad):
    x = W.bits(W.generate("moe", (3, 16, 64))).copy()
    x[1, 5, 17] = bad
    for mode, rule in (("rtn6", "mse"), ("four_over_six", "mae")):
        for fq in (False, True):
            check_full(nv, orc, x, mode, rule, fq, "poison")
    am = nv.amax(to_gpu(x))
    torch.cuda.synchronize()
    a = am.cpu().numpy()
    assert not np.isfinite(a[1]) and np.isfinite(a[0]) and np.isfinite(a[2])


# ----------------------------------------------------------------------------- amax, fixed scale
def test_amax_matches_oracle(nv, orc):
    for name, shape in SMALL:
        x = W.bits(W.generate(name, shape))
        E = x.shape[0] if x.ndim == 3 else 1
        got = nv.amax(to_gpu(x)).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), orc.amax(x, E).view(np.uint32)), name


# Every amax variant: 8 chunks per lane step for tensors that fill their workgroups, read
# coalesced for a single tensor of at most 8 steps per lane (2049x8208: 129 workgroups of 2
# steps, the last span running past the end) and 128 contiguous bytes per lane for longer
# single tensors (8193x16400: 228 workgroups of 9 steps) and batches (3x1001x5648); 1 chunk
# otherwise.  Chunk counts that are not a multiple of 8 (the tail lane of the 128-byte form),
# and the maximum planted first, last and in the middle of each tensor.
AMAX_SHAPES = [(1, 16), (7, 48), (2049, 8208), (8193, 16400), (3, 1000, 5136), (3, 1001, 5648),
               (300, 2, 32)]


@pytest.mark.parametrize("shape", AMAX_SHAPES, ids=["x".join(map(str, s)) for s in AMAX_SHAPES])
def test_amax_variants_and_tails(nv, orc, shape):
    E = shape[0] if len(shape) == 3 else 1
    base = W.bits(W.generate("weight", shape)).reshape(E, -1)
    big = bf16_bits(np.array([3.0, -5.5, 7.25], np.float32))
    for where in ("first", "last", "middle"):
        x = base.copy()
        for t in range(E):
            pos = {"first": 0, "last": x.shape[1] - 1, "middle": x.shape[1] // 2 + 3}[where]
            x[t, pos] = big[t % 3]
        x = x.reshape(shape)
        say("amax %s max %s" % (shape, where))
        got = nv.amax(to_gpu(x)).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), orc.amax(x, E).view(np.uint32)), (shape, where)


@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
def test_fixed_scale_entry(nv, orc, mode, rule):
    x = W.bits(W.generate("moe", (3, 40, 160)))
    xg = to_gpu(x)
    # 1. amax pass + fixed-scale pass == the dynamic call
    am = nv.amax(xg)
    c1, s1, a1 = nv.quantize_from_amax(xg, am, mode, rule)
    c2, s2, a2 = nv.quantize(xg, mode, rule)
    y1, b1 = nv.fakequant_from_amax(xg, am, mode, rule)
    y2, b2 = nv.fakequant(xg, mode, rule)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(y1, y2)
    assert torch.equal(a1, a2) and torch.equal(b1, b2)
    # 2. a static amax below the true one: scales clamp at 448 and values saturate
    true_amax = orc.amax(x, 3)
    static = (true_amax * np.float32(0.3)).astype(np.float32)
    static[1] = -static[1]                                   # the magnitude is used
    sg = torch.from_numpy(static).cuda()
    c, s, a = nv.quantize_from_amax(xg, sg, mode, rule)
    y, _ = nv.fakequant_from_amax(xg, sg, mode, rule)
    torch.cuda.synchronize()
    al = np.array([orc.alpha(abs(float(v)), mode) for v in static], np.float32)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), al.view(np.uint32))
    ids = np.arange(x.size // 16)
    ref = orc.quantize_blocks(x, al, ids, mode, rule)
    assert np.array_equal(c.cpu().numpy().reshape(-1, 8), ref["codes"])
    assert np.array_equal(s.cpu().numpy().ravel(), ref["scales"])
    assert np.array_equal(u16(y).reshape(-1, 16), ref["y"])
    assert (ref["scales"] == 0x7E).any()                      # the clamp was exercised


# A fixed amax anywhere in the binary32 range, on data of every magnitude: alpha from
# FLT_MAX / 1536 down to subnormal and zero, across the bound (alpha = 2^-118) below which every
# block takes the reference path, so the table-driven scales are checked at both ends of the
# range they claim.
EXTREME_AMAX = np.array([3.4028235e38, 2.0 ** 120, 1.0e10, 1.0, 1536 * 2.0 ** -118,
                         np.nextafter(np.float32(1536 * 2.0 ** -118), np.float32(0)),
                         2688 * 2.0 ** -118,
                         np.nextafter(np.float32(2688 * 2.0 ** -118), np.float32(1)), 1.0e-30,
                         1.4e-45, 0.0, -2.0], np.float32)


def _extreme_data():
    rng = np.random.default_rng(21)
    E = EXTREME_AMAX.size
    normal = W.bits(W.normal((E * 8, 256), seed=22)).reshape(E, 8, 256)
    huge = (rng.integers(0x7E00, 0x7F80, size=(E, 8, 256), dtype=np.uint16) |
            (rng.integers(0, 2, size=(E, 8, 256), dtype=np.uint16) << 15))
    tiny = (rng.integers(0x0001, 0x0900, size=(E, 8, 256), dtype=np.uint16) |
            (rng.integers(0, 2, size=(E, 8, 256), dtype=np.uint16) << 15))
    return {"normal": normal, "huge": huge, "tiny": tiny}


@pytest.mark.parametrize("kind", ["normal", "huge", "tiny"])
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
def test_fixed_scale_extreme_amax(nv, orc, kind, mode, rule):
    x = _extreme_data()[kind]
    E = x.shape[0]
    xg, sg = to_gpu(x), torch.from_numpy(EXTREME_AMAX.copy()).cuda()
    say("[parity] extreme amax %s %s/%s" % (kind, mode, rule))
    c, s, a = nv.quantize_from_amax(xg, sg, mode, rule)
    y, b = nv.fakequant_from_amax(xg, sg, mode, rule)
    torch.cuda.synchronize()
    al = np.array([orc.alpha(abs(float(v)), mode) for v in EXTREME_AMAX], np.float32)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), al.view(np.uint32))
    assert np.array_equal(b.cpu().numpy().view(np.uint32), al.view(np.uint32))
    ref = orc.quantize_blocks(x, al, np.arange(x.size // 16), mode, rule)
    got_s = s.cpu().numpy().ravel()
    bad = np.nonzero(got_s != ref["scales"])[0]
    assert bad.size == 0, "scales differ at blocks %s (tensor %s)" % (bad[:4], bad[:4] // (x.size // 16 // E))
    assert np.array_equal(c.cpu().numpy().reshape(-1, 8), ref["codes"])
    assert np.array_equal(u16(y).reshape(-1, 16), ref["y"])


# ----------------------------------------------------------------------------- in place, guards
def test_in_place_fakequant(nv, orc):
    x = W.bits(W.generate("act", (64, 512)))
    xg = to_gpu(x)
    y, al = nv.fakequant(xg, "four_over_six", "mae", out=xg)
    torch.cuda.synchronize()
    assert y.data_ptr() == xg.data_ptr()
    ref = orc.quantize(x, "four_over_six", "mae")
    assert np.array_equal(u16(xg), ref["y"])


def test_no_writes_outside_outputs(nv, orc):
    """Outputs live inside larger buffers filled with a canary; only the output bytes may
    change."""
    x = W.bits(W.generate("large", (33, 240)))           # 495 blocks: ragged
    xg = to_gpu(x)
    G = 4096
    nb = x.size // 16
    for fq in (False, True):
        if fq:
            buf = torch.full((G + x.size + G,), 0x5A5A, dtype=torch.int32, device="cuda") \
                .to(torch.int16)
            out = buf[G:G + x.size].view(torch.bfloat16).view(x.shape)
            abuf = torch.full((64 + 1 + 64,), 7.5, dtype=torch.float32, device="cuda")
            nv.fakequant(xg, "four_over_six", "mse", out=out, alpha=abuf[64:65])
            torch.cuda.synchronize()
            hb = buf.cpu().numpy()
            assert (hb[:G] == 0x5A5A).all() and (hb[G + x.size:] == 0x5A5A).all()
        else:
            cbuf = torch.full((G + nb * 8 + G,), 0xA5, dtype=torch.uint8, device="cuda")
            sbuf = torch.full((G + nb + 3 + G,), 0xA5, dtype=torch.uint8, device="cuda")
            abuf = torch.full((64 + 1 + 64,), 7.5, dtype=torch.float32, device="cuda")
            codes = cbuf[G:G + nb * 8].view(x.shape[0], x.shape[1] // 2)
            scales = sbuf[G + 3:G + 3 + nb].view(x.shape[0], x.shape[1] // 16)
            nv.quantize(xg, "four_over_six", "mse", codes=codes, scales=scales,
                        alpha=abuf[64:65])
            torch.cuda.synchronize()
            hc, hs = cbuf.cpu().numpy(), sbuf.cpu().numpy()
            assert (hc[:G] == 0xA5).all() and (hc[G + nb * 8:] == 0xA5).all()
            assert (hs[:G + 3] == 0xA5).all() and (hs[G + 3 + nb:] == 0xA5).all()
        ha = abuf.cpu().numpy()
        assert (ha[:64] == 7.5).all() and (ha[65:] == 7.5).all()


# ----------------------------------------------------------------------------- full size
_FULL = {}


def full_input(name):
    if name not in _FULL:
        _FULL.clear()
        say("[full] generating %s %s" % (name, W.WORKLOADS[name].shape))
        _FULL[name] = W.generate(name)
    return _FULL[name]


FULL_CASES = [(w.name, mode, rule, out == "fakequant") for w in W.WORKLOADS.values()
              for (mode, rule, out) in w.runs]


def _decode_packed(codes, scales, alpha, shape):
    """Packed NVFP4 -> bf16 with torch ops on the GPU (IEEE binary32 multiplies and the
    round-to-nearest-even bf16 cast): val(code) * RN(dec(scale) * alpha)."""
    fp4 = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6],
                       dtype=torch.float32, device=codes.device)
    c = codes.reshape(-1, 8).to(torch.int32)
    nib = torch.stack([c & 15, c >> 4], dim=-1).reshape(-1, 16)
    dec = scales.reshape(-1).view(torch.float8_e4m3fn).to(torch.float32)
    E = alpha.numel()
    step = dec.view(E, -1) * alpha.view(E, 1)
    xhat = fp4[nib.long()] * step.reshape(-1, 1)
    return xhat.to(torch.bfloat16).view(shape)


@pytest.mark.parametrize("name,mode,rule,fq", FULL_CASES,
                         ids=["%s-%s-%s" % (c[0], c[1], c[2]) for c in FULL_CASES])
def test_full_size_workloads_whole(nv, orc, name, mode, rule, fq):
    """Every workload at its full size, in the launch configuration the benchmark times: the
    whole output (codes and scale bytes, or fake-quant bf16) and alpha against the oracle."""
    xt = full_input(name)
    x = W.bits(xt)
    E = x.shape[0] if x.ndim == 3 else 1
    say("[full] %s %s/%s fq=%s" % (name, mode, rule, fq))
    xg = xt.cuda()
    if fq:
        y, a = nv.fakequant(xg, mode, rule)
        torch.cuda.synchronize()
        got_y, got_a = u16(y), a.cpu().numpy()
    else:
        c, s, a = nv.quantize(xg, mode, rule)
        torch.cuda.synchronize()
        got_c, got_s, got_a = c.cpu().numpy(), s.cpu().numpy(), a.cpu().numpy()
    say("[full] oracle %s %s/%s" % (name, mode, rule))
    ref = orc.quantize(x, mode, rule, nthreads=NTHREADS, want_y=fq)
    assert np.array_equal(got_a.view(np.uint32), ref["alpha"][:E].view(np.uint32))
    if fq:
        assert np.array_equal(got_y, ref["y"])
        del got_y, ref
        # at full size: the packed result decodes to this fake-quant output
        c, s, a2 = nv.quantize(xg, mode, rule)
        dq = _decode_packed(c, s, a2, xg.shape)
        torch.cuda.synchronize()
        assert torch.equal(dq.view(torch.int16), y.view(torch.int16))
    else:
        assert np.array_equal(got_s, ref["scales"])
        assert np.array_equal(got_c, ref["codes"])
        del got_c, got_s, ref
        if name in ("tiny", "weight"):                        # small enough to decode whole
            y, _ = nv.fakequant(xg, mode, rule)
            dq = _decode_packed(c, s, a, xg.shape)
            torch.cuda.synchronize()
            assert torch.equal(dq.view(torch.int16), y.view(torch.int16))
    del xg
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- dequantize
def test_dequantize_random_shapes_and_bytes(nv, orc):
    """Random shapes (ragged last workgroups, batched or not) with arbitrary code bytes, scale
    bytes (NaN and negative scales included) and alphas, against the oracle's dequantization."""
    rng = np.random.default_rng(93)
    for k in range(16):
        rows = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 200)) * 16
        E = int(rng.integers(2, 5)) if k % 2 else 1
        lead = (E,) if k % 2 else ()
        codes = rng.integers(0, 256, size=lead + (rows, cols // 2), dtype=np.uint8)
        scales = rng.integers(0, 256, size=lead + (rows, cols // 16), dtype=np.uint8)
        alpha = np.exp(rng.uniform(-20, 5, size=E)).astype(np.float32)
        y = nv.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                          torch.from_numpy(alpha).cuda())
        torch.cuda.synchronize()
        ref = orc.dequantize(codes.reshape((E, rows, cols // 2)),
                             scales.reshape((E, rows, cols // 16)), alpha)
        assert np.array_equal(u16(y).reshape(-1), ref.reshape(-1)), (k, rows, cols, E)


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
def test_dequantize_equals_fakequant_and_oracle(nv, orc, name, shape):
    x = W.bits(W.generate(name, shape))
    xg = to_gpu(x)
    for mode, rule in (("rtn6", "mse"), ("four_over_six", "mae")):
        c, s, a = nv.quantize(xg, mode, rule)
        y = nv.dequantize(c, s, a)
        yf, _ = nv.fakequant(xg, mode, rule)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), yf.view(torch.int16))
        ref = orc.dequantize(c.cpu().numpy(), s.cpu().numpy(), a.cpu().numpy())
        assert np.array_equal(u16(y), ref)


def test_dequantize_arbitrary_bytes(nv, orc):
    """Every code and every scale byte (NaN 0x7F/0xFF and negative scales included), a
    NaN alpha in one tensor of a batch."""
    rng = np.random.default_rng(8)
    E, rows, cols = 3, 20, 512
    codes = rng.integers(0, 256, size=(E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(E, rows, cols // 16), dtype=np.uint8)
    scales[0, 0, :] = np.arange(cols // 16, dtype=np.uint8)
    alpha = np.array([2.0 ** -8, np.nan, 3.1e-5], np.float32)
    y = nv.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                      torch.from_numpy(alpha).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(u16(y), orc.dequantize(codes, scales, alpha))


def test_dequantize_full_size_weight(nv, orc):
    xt = full_input("weight")
    xg = xt.cuda()
    c, s, a = nv.quantize(xg, "four_over_six", "mse")
    y = nv.dequantize(c, s, a)
    yf, _ = nv.fakequant(xg, "four_over_six", "mse")
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yf.view(torch.int16))


# ----------------------------------------------------------------------------- diagnostics
MAXERR_COL, NEAR_COL = 2, 5


def check_stats(got, ref, n, tag):
    """Per-tensor statistics: NaN rows match, max |e| and the near-band count exactly, the
    sums within their rounding bound.  The terms are non-negative and exact in binary64, so
    the GPU's binary64 sums in any order are within (n-1)*2^-53 of the exact sum relative to
    it, and the oracle's long-double sums within (n-1)*2^-64 plus one rounding to binary64."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    tol = (n - 1) * 2.0 ** -53 + (n - 1) * 2.0 ** -64 + 2.0 ** -53
    for t in range(ref.shape[0]):
        if np.isnan(ref[t]).any():
            assert np.isnan(got[t]).all(), (tag, t)
            continue
        assert got[t, MAXERR_COL] == ref[t, MAXERR_COL], (tag, t)
        assert got[t, NEAR_COL] == ref[t, NEAR_COL], (tag, t)
        for k in (0, 1, 3, 4):
            assert abs(got[t, k] - ref[t, k]) <= tol * ref[t, k], (tag, t, k, got[t, k], ref[t, k])


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
def test_diag_choice_and_count(nv, orc, name, shape, mode, rule):
    x = W.bits(W.generate(name, shape))
    c, s, a, q, n4, st = nv.quantize_diag(to_gpu(x), mode, rule)
    torch.cuda.synchronize()
    ref = orc.quantize(x, mode, rule, want_y=False, want_qstar=True)
    assert np.array_equal(c.cpu().numpy(), ref["codes"])
    assert np.array_equal(s.cpu().numpy(), ref["scales"])
    assert np.array_equal(q.cpu().numpy(), ref["qstar"])
    E = x.shape[0] if x.ndim == 3 else 1
    want = (ref["qstar"].reshape(E, -1) == 4).sum(axis=1)
    assert np.array_equal(n4.cpu().numpy(), want)
    if mode == "four_over_six":
        assert want.sum() > 0
    check_stats(st.cpu().numpy(), orc.quantize_stats(x, mode, rule, nthreads=NTHREADS),
                x.size // E, name)
    # without statistics the other outputs are the same
    c2, s2, a2, q2, n42, st2 = nv.quantize_diag(to_gpu(x), mode, rule, stats=False)
    torch.cuda.synchronize()
    assert st2 is None and torch.equal(c2, c) and torch.equal(q2, q) and torch.equal(n42, n4)


def test_diag_poison_and_edges(nv, orc):
    x = W.bits(W.generate("moe", (3, 16, 64))).copy()
    x[2, 3, 5] = 0x7FC0
    for name, xb in (("poison", x), ("subnormal", EDGE["subnormal"]), ("zeros", EDGE["zeros"])):
        c, s, a, q, n4, st = nv.quantize_diag(to_gpu(xb), "four_over_six", "mse")
        torch.cuda.synchronize()
        ref = orc.quantize(xb, "four_over_six", "mse", want_y=False, want_qstar=True)
        assert np.array_equal(q.cpu().numpy(), ref["qstar"]), name
        E = xb.shape[0] if xb.ndim == 3 else 1
        assert np.array_equal(n4.cpu().numpy(), (ref["qstar"].reshape(E, -1) == 4).sum(axis=1)), name
        check_stats(st.cpu().numpy(), orc.quantize_stats(xb, "four_over_six", "mse"),
                    xb.size // E, name)
    assert np.isnan(st.cpu().numpy()).sum() == 0


@pytest.mark.parametrize("shape", [(2, 1, 16), (5, 3, 112), (7, 40, 176), (3000, 48)],
                         ids=["one-block-tensors", "21-blocks", "440-blocks", "one-tensor"])
def test_diag_count_from_choice_bytes(nv, orc, shape):
    """Without statistics the count of blocks scaled to 4 comes from the per-block choice bytes
    after the pass: tensors whose byte ranges start and end off 16-byte boundaries, and a
    poisoned tensor (choice bytes 0, count 0)."""
    x = W.bits(W.generate("moe", shape) if len(shape) == 3 else W.weight(shape, seed=43)).copy()
    if x.ndim == 3:
        x[1, 0, 3] = 0x7FC0
    c, s, a, q, n4, st = nv.quantize_diag(to_gpu(x), "four_over_six", "mse", stats=False)
    torch.cuda.synchronize()
    ref = orc.quantize(x, "four_over_six", "mse", want_y=False, want_qstar=True)
    E = x.shape[0] if x.ndim == 3 else 1
    assert np.array_equal(q.cpu().numpy(), ref["qstar"])
    assert np.array_equal(n4.cpu().numpy(), (ref["qstar"].reshape(E, -1) == 4).sum(axis=1))
    assert np.array_equal(c.cpu().numpy(), ref["codes"])
    if x.ndim == 3:
        assert n4.cpu().numpy()[1] == 0 and (q.cpu().numpy()[1] == 0).all()


def test_diag_count_long_call(nv, orc):
    """A plain diagnostics call of 2^23 blocks or more takes the block pass's grid and counts
    the choice bytes after the pass: five tensors of 1,678,677 blocks (an odd count, so every
    tensor's byte range starts and ends off a 16-byte boundary), one of them poisoned."""
    shape = (5, 1001, 26832)
    x = W.bits(W.generate("moe", shape)).copy()
    x[2, 500, 7] = 0xFF80            # -inf
    assert x.size // 16 >= 2 ** 23 and (x.size // 16 // 5) % 16 != 0
    c, s, a, q, n4, _ = nv.quantize_diag(to_gpu(x), "four_over_six", "mse", stats=False)
    torch.cuda.synchronize()
    ref = orc.quantize(x, "four_over_six", "mse", nthreads=NTHREADS, want_y=False,
                       want_qstar=True)
    assert np.array_equal(q.cpu().numpy(), ref["qstar"])
    want = (ref["qstar"].reshape(5, -1) == 4).sum(axis=1)
    assert np.array_equal(n4.cpu().numpy(), want) and want[2] == 0 and want.sum() > 0
    assert np.array_equal(c.cpu().numpy(), ref["codes"])
    assert np.array_equal(s.cpu().numpy(), ref["scales"])


@pytest.mark.parametrize("shape", [(1024, 8208), (4, 300, 640), (1100, 2, 32)],
                         ids=["one-tensor", "batched", "more-tensors-than-slots"])
def test_diag_stats_repeatable_with_any_workspace(nv, orc, shape):
    """The statistics are summed in an order fixed by the shape: repeated calls give the same
    bits, whatever the workspace held before (here all ones, then random words)."""
    x = W.bits(W.weight(shape, seed=41))
    E = shape[0] if len(shape) == 3 else 1
    xg = to_gpu(x)
    ws = torch.full((nv.diag_ws_words(E),), -1, dtype=torch.int32, device="cuda")
    first = nv.quantize_diag(xg, "four_over_six", "mse", workspace=ws)[5].cpu().numpy()
    ws.copy_(torch.randint(-2**31, 2**31 - 1, ws.shape, dtype=torch.int32))
    again = nv.quantize_diag(xg, "four_over_six", "mse", workspace=ws)[5].cpu().numpy()
    third = nv.quantize_diag(xg, "four_over_six", "mse")[5].cpu().numpy()
    assert np.array_equal(first.view(np.uint64), again.view(np.uint64))
    assert np.array_equal(first.view(np.uint64), third.view(np.uint64))
    check_stats(first, orc.quantize_stats(x, "four_over_six", "mse", nthreads=NTHREADS),
                x.size // E, str(shape))


DIAG_FULL = [(w.name, mode, rule) for w in W.WORKLOADS.values()
             for (mode, rule, _) in w.runs[:1]]


@pytest.mark.parametrize("name,mode,rule", DIAG_FULL, ids=[c[0] for c in DIAG_FULL])
def test_diag_stats_full_size(nv, orc, name, mode, rule):
    """The diagnostics at full size: qstar on sampled blocks, the count of blocks scaled
    to 4 and the error statistics of every tensor against the oracle."""
    xt = full_input(name)
    x = W.bits(xt)
    E = x.shape[0] if x.ndim == 3 else 1
    say("[diag-full] %s %s/%s" % (name, mode, rule))
    c, s, a, q, n4, st = nv.quantize_diag(xt.cuda(), mode, rule)
    torch.cuda.synchronize()
    ref = orc.quantize_stats(x, mode, rule, nthreads=NTHREADS)
    check_stats(st.cpu().numpy(), ref, x.size // E, name)
    rng = np.random.default_rng(7)
    ids = rng.integers(0, x.size // 16, size=4000)
    amax = orc.amax(x, E)
    al = np.array([orc.alpha(float(v), mode) for v in amax], np.float32)
    rb = orc.quantize_blocks(x, al, ids, mode, rule)
    assert np.array_equal(q.cpu().numpy().reshape(-1)[ids], rb["qstar"])
    if mode == "four_over_six":
        assert int(n4.sum()) > 0
    t = st.cpu().numpy().sum(axis=0)
    say("[diag-full] %s: near-band share of sum e^2 %.3f, scale-rounding share %.3f, "
        "blocks scaled to 4 %.3f" % (name, t[3] / t[0], (t[0] - t[4]) / t[0],
                                     int(n4.sum()) / (x.size // 16)))
