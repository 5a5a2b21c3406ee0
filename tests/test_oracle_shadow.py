"""Pins of the oracle's exact-quotient shadow (CPU only).

The shadow reads the encoding of the Four Over Six explainer ("Adaptive block
scaling algorithm": quantize each block with its max mapped to 6 and to 4, take
both errors against the original high-precision values, keep the smaller;
"Implementation details": the per-tensor scale with 256 instead of 448) with exact
arithmetic everywhere after the per-tensor scale, instead of one binary32
rounding per step.  It is a diagnostic of the binary32 reading, so it is pinned
here to an exact-rational brute force written from the same definition (nearest
grid values by exact distance over every candidate), to closed forms and to the
hand-derived worked examples.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

from helpers import bf16_bits, bf16_to_f32, read_examples
from nvfp4_block_scaled_amax_amd import workloads as W

GRID = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]     # FP4 magnitudes, "Problem definition"


def _e4m3(b: int) -> Fraction:
    """E4M3FN value of byte b (sign bit clear): 4 exponent bits (bias 7), 3 mantissa bits."""
    e, m = (b >> 3) & 15, b & 7
    return Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _bf16(p: int) -> Fraction:
    """bfloat16 value of a non-negative pattern; the all-ones exponent stands for 2^128."""
    e, m = (p >> 7) & 0xFF, p & 0x7F
    return Fraction(m) * Fraction(2) ** -133 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def _nearest(target: Fraction, values, ties_even=True) -> int:
    """Index of the value nearest to target by exact distance; a tie goes to the even index."""
    best, bd = 0, abs(target - values[0])
    for i in range(1, len(values)):
        d = abs(target - values[i])
        if d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


E4M3 = [_e4m3(b) for b in range(0x7F)]                          # 0x00 .. 0x7E (448)


def _bf16_nearest(a: Fraction) -> int:
    """Pattern of the bfloat16 nearest to a >= 0 (ties to the even pattern)."""
    t = int(np.float32(float(a)).view(np.uint32)) >> 16
    cands = [p for p in (t - 1, t, t + 1) if 0 <= p <= 0x7F80]
    return min(cands, key=lambda p: (abs(a - _bf16(p)), p % 2))


def brute_block(xbits, A: Fraction, mode: str, rule: str):
    """The exact reading of one block from its definition, in exact rationals: every scale
    byte and every FP4 code is the nearest by exact distance (ties to the even code), the
    errors are exact, the smaller error wins and ties keep 6."""
    x = [Fraction(float(v)) for v in bf16_to_f32(xbits)]
    neg = [bool(int(b) & 0x8000) for b in xbits]
    bmax = max(abs(v) for v in x)
    out = {}
    for Q in ((6, 4) if mode == "four_over_six" else (6,)):
        s = 0 if A == 0 else _nearest(bmax / (Q * A), E4M3)
        D = E4M3[s] * A
        cap = 6 if Q == 4 else 7
        mags, xh = [], []
        for v in x:
            m = 0 if D == 0 else min(_nearest(abs(v) / D, GRID), cap)
            mags.append(m)
            xh.append(GRID[m] * D)
        sx = [-h if n else h for h, n in zip(xh, neg)]
        errs = [v - h for v, h in zip(x, sx)]
        err = (sum(e * e for e in errs) if rule == "mse" else
               sum(abs(e) for e in errs) if rule == "mae" else max(abs(e) for e in errs))
        out[Q] = (s, mags, sx, err)
    Qs = 4 if mode == "four_over_six" and out[4][3] < out[6][3] else 6
    s, mags, sx, _ = out[Qs]
    codes = np.zeros(8, np.uint8)
    for i in range(16):
        codes[i // 2] |= ((8 if neg[i] else 0) | mags[i]) << (4 * (i & 1))
    y = np.array([_bf16_nearest(abs(h)) | (0x8000 if neg[i] else 0) for i, h in enumerate(sx)],
                 np.uint16)
    return codes, s, y, Qs


def _blocks():
    """Blocks of the five workload distributions plus blocks built on exact FP4 ties: values
    that are the block max times 2^-k times 3/4, 5/8, 5/12 and the like."""
    out = []
    for name, shape in (("tiny", (8, 64)), ("weight", (8, 64)), ("act", (8, 64)),
                        ("large", (8, 64)), ("moe", (2, 4, 64))):
        xb = W.bits(W.generate(name, shape)).reshape(-1, 16)
        out.extend(xb[:24])
    rng = np.random.default_rng(7)
    for _ in range(60):
        top = float(bf16_to_f32(np.array([rng.integers(0x3C00, 0x4300)], np.uint16))[0])
        fr = rng.choice([0.75, 0.625, 5 / 12, 0.125, 0.25, 0.375, 1.0, 0.5, 7 / 12, 0.0], 15)
        v = np.concatenate([[top], top * fr * 2.0 ** -rng.integers(0, 4, 15)]).astype(np.float32)
        v *= rng.choice([-1, 1], 16)
        out.append(torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    return out


@pytest.mark.parametrize("mode,rule", [("rtn6", "mse"), ("four_over_six", "mse"),
                                       ("four_over_six", "mae"), ("four_over_six", "maxerr")])
def test_shadow_equals_exact_rational_brute_force(orc, mode, rule):
    blocks = _blocks()
    C = 1536 if mode == "four_over_six" else 2688
    # the tensor amax is the block's own max, larger (up to 2^18 times: the block scales fall
    # into the E4M3 subnormals or to zero), or smaller, as a fixed amax may be (the scales
    # saturate at 448 and the cap at 4 decides between the candidates)
    amaxes = [float(np.abs(bf16_to_f32(b)).max()) * f for b, f in
              zip(blocks, np.resize([1.0, 1.0, 2.0, 5.5, 700.0, 2.0 ** 16 * 1.3, 2.0 ** 17 * 1.1,
                                     2.0 ** 18, 0.6, 0.3, 0.45], len(blocks)))]
    n_diff_b32 = 0
    for b, am in zip(blocks, amaxes):
        am = float(np.float32(am))
        for exact_alpha in (False, True):
            if exact_alpha:
                a, A = am, Fraction(am) / C
            else:
                a = float(orc.alpha(am, mode))
                A = Fraction(a)
            codes, s, y, q = orc.shadow_block(b, a, mode, rule, exact_alpha)
            wc, ws, wy, wq = brute_block(b, A, mode, rule)
            assert np.array_equal(codes, wc) and s == ws and q == wq, (b, am, exact_alpha)
            assert np.array_equal(y, wy), (b, am, exact_alpha)
            c32, s32, _, _ = orc.quantize_block(b, orc.alpha(am, mode), mode, rule)
            n_diff_b32 += not (np.array_equal(c32, codes) and s32 == s)
    assert orc.shadow_inexact() == 0
    if mode == "rtn6":
        assert n_diff_b32 > 0          # the tie-built blocks separate the two readings


def test_shadow_worked_examples(orc):
    """The hand-derived worked examples involve no rounding that the two readings treat
    differently (every quotient is exact), so the shadow reproduces their printed codes,
    scale bytes and fake-quant values in both of its forms."""
    for ex in read_examples():
        x = bf16_bits(np.array(ex["input"], np.float32))
        nblk = x.size // 16
        for rule in ex["rules"]:
            mode = ex["mode"]
            al = float(np.uint32(ex["alpha_bits"]).view(np.float32))
            amax = float(np.abs(bf16_to_f32(x)).max())
            for exact_alpha in (False, True):
                a = amax if exact_alpha else al
                if exact_alpha and (amax == 0 or float(orc.alpha(amax, mode)) != al):
                    continue                   # the example fixes alpha by other means
                for k in range(nblk):
                    codes, s, y, q = orc.shadow_block(x[16 * k:16 * k + 16], a, mode, rule,
                                                      exact_alpha)
                    assert s == ex["scales"][k], (ex["name"], rule, k)
                    assert list(codes) == ex["codes"][8 * k:8 * k + 8], (ex["name"], rule, k)
                    if "y" in ex:
                        want = bf16_bits(np.array(ex["y"][16 * k:16 * k + 16], np.float32))
                        assert np.array_equal(y, want), (ex["name"], rule, k)


def test_shadow_resolves_exact_ties_to_the_even_code(orc):
    """rtn6 block [A, A/8, 0 x 14] with the tensor amax A: sigma = A / (6 * A/2688) = 448
    exactly, so D = 448 * A/2688 = A/6 and A/8 divided by D is 0.75, the midpoint of FP4
    values 0.5 (code 1) and 1 (code 2): the even code 2 wins.  The fully exact reading gives
    code 2 for every A; the binary32 reading rounds alpha, d, 1/d and the product, and lands
    on either side."""
    seen_b32 = set()
    for p in range(0x3C00, 0x4300, 7):               # A over [1, 128)
        A = float(bf16_to_f32(np.array([p], np.uint16))[0])
        x = bf16_bits(np.array([A, A / 8] + [0.0] * 14, np.float32))
        codes, s, y, q = orc.shadow_block(x, A, "rtn6", "mse", True)
        assert s == 0x7E and codes[0] == 0x27, (A, hex(codes[0]))
        c32, s32, _, _ = orc.quantize_block(x, orc.alpha(A, "rtn6"), "rtn6", "mse")
        assert s32 == 0x7E and c32[0] & 0x0F == 0x7
        seen_b32.add(int(c32[0]) >> 4)
    assert seen_b32 == {1, 2}          # both sides occur over this range of A


def test_shadow_invariants_and_counts(orc):
    """Scaling a tensor by 2^k changes no byte of the exact reading; negation flips the sign
    bits; the whole-tensor comparison counts what a block-by-block comparison finds."""
    x = W.bits(W.generate("weight", (16, 448)))
    amax = float(orc.amax(x)[0])
    for mode, rule in (("four_over_six", "mse"), ("rtn6", "mse"), ("four_over_six", "maxerr")):
        for exact_alpha in (False, True):
            tot = dict(blocks=0, scale_diff=0, choice_diff=0, block_diff=0, code_diff=0,
                       y_diff=0)
            al = float(orc.alpha(amax, mode))
            for b in x.reshape(-1, 16):
                a = amax if exact_alpha else al
                codes, s, y, q = orc.shadow_block(b, a, mode, rule, exact_alpha)
                for k in (-7, 5):
                    bk = bf16_bits(bf16_to_f32(b) * np.float32(2.0 ** k))
                    ak = float(np.float32(a) * np.float32(2.0 ** k))
                    ck, sk, yk, qk = orc.shadow_block(bk, ak, mode, rule, exact_alpha)
                    assert np.array_equal(ck, codes) and sk == s and qk == q
                cn, sn, yn, qn = orc.shadow_block(b ^ np.uint16(0x8000), a, mode, rule,
                                                  exact_alpha)
                assert np.array_equal(cn, codes ^ np.uint8(0x88)) and sn == s and qn == q
                assert np.array_equal(yn, y ^ np.uint16(0x8000))
                c32, s32, y32, d = orc.quantize_block(b, al, mode, rule)
                dc = sum(((c32[i // 2] >> (4 * (i & 1))) & 15) != ((codes[i // 2] >> (4 * (i & 1))) & 15)
                         for i in range(16))
                tot["blocks"] += 1
                tot["scale_diff"] += s32 != s
                tot["choice_diff"] += d["qstar"] != q
                tot["block_diff"] += dc > 0 or s32 != s
                tot["code_diff"] += dc
                tot["y_diff"] += int((y32 != y).sum())
            got = orc.shadow_compare(x, mode, rule, exact_alpha, nthreads=3)
            assert got["inexact"] == 0
            for k, v in tot.items():
                assert got[k] == v, (mode, rule, exact_alpha, k)


def test_shadow_resolves_exact_scale_ties_to_the_even_byte(orc):
    """rtn6 tensor of two blocks [A, 0 x 15] and [B, 0 x 15], B < A, with alpha = A/2688 taken
    exactly: sigma of the second block is B / (6 * A/2688) = 448 * B/A.  For A = 28 and every
    bf16 B that makes 16 * B the midpoint of two consecutive E4M3 values (e.g. B = 25:
    sigma = 400, halfway between 384 = 0x7C and 416 = 0x7D), the even byte wins."""
    A = 28.0
    mids = {}
    for lo in range(0x08, 0x7E):                   # consecutive normal E4M3 pairs (lo, lo + 1)
        mids[(_e4m3(lo) + _e4m3(lo + 1)) / 2] = lo if lo % 2 == 0 else lo + 1
    hits = 0
    for p in range(0x3F00, 0x41E0):                # bf16 B over [0.5, 28)
        B = float(bf16_to_f32(np.array([p], np.uint16))[0])
        sigma = Fraction(448) * Fraction(B) / Fraction(A)
        if sigma not in mids:
            continue
        x = bf16_bits(np.array([A] + [0.0] * 15 + [B] + [0.0] * 15, np.float32))
        _, s0, _, _ = orc.shadow_block(x[:16], A, "rtn6", "mse", True)
        _, s1, _, _ = orc.shadow_block(x[16:], A, "rtn6", "mse", True)
        assert s0 == 0x7E and s1 == mids[sigma], (B, float(sigma), hex(s1))
        hits += 1
    assert hits >= 20
