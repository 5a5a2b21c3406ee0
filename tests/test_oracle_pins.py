"""Pins of the CPU oracle to what the pages and the mathematics fix (CPU only).

Sources: "Four Over Six: More Accurate NVFP4 Quantization with Adaptive Block
Scaling" (gist.science explainer) -- sections "Problem definition", "Method /
core mechanism", "Adaptive block scaling algorithm", "Implementation details";
"Quantization-Aware Distillation for NVFP4 Inference Accuracy Recovery"
(gist.science explainer), key findings item 3 (block size 16).

Every pin compares the oracle with something other than itself: values the
pages print, hand-derived worked examples, library routines (torch's float8 and
bfloat16 casts), exact rational arithmetic, or invariants of the method.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from helpers import GOLDEN, bf16_bits, bf16_to_f32, f32_bits, read_examples
from nvfp4_block_scaled_amax_amd import workloads as W

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _neigh(values, k):
    """All positive float32 within +-k ulps (bit patterns) of each value."""
    out = []
    for v in values:
        b = int(np.float32(v).view(np.uint32))
        lo, hi = max(0, b - k), min(0x7F7FFFFF, b + k)
        out.append(np.arange(lo, hi + 1, dtype=np.uint32))
    return np.concatenate(out).view(np.float32)


# ----------------------------------------------------------------------------- E2M1
def test_e2m1_grid_is_the_printed_value_set(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 8
    for code, val in rows:
        code, val = int(code), float(val)
        assert orc.e2m1_decode(code) == val
        neg = orc.e2m1_decode(code | 8)
        assert neg == -val and math.copysign(1.0, neg) == -1.0
    mags = [orc.e2m1_decode(c) for c in range(8)]
    # steps of 0.5 on [0,2], 1 on [2,4], 2 on [4,6]; range [-6, 6]
    assert list(np.diff(mags)) == [0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0]
    assert max(mags) == 6.0
    assert list(orc.e2m1_round_mag(mags)) == list(range(8))  # round trip


def _e2m1_by_midpoints(a: np.ndarray) -> np.ndarray:
    """Independent formulation: count the midpoints below a; at a midpoint take the even code."""
    grid = np.array(GRID)
    mids = (grid[:-1] + grid[1:]) / 2
    a64 = a.astype(np.float64)
    idx = np.searchsorted(mids, a64, side="left")
    at_mid = np.zeros(a.shape, bool)
    inb = idx < len(mids)
    at_mid[inb] = mids[idx[inb]] == a64[inb]
    code = np.where(at_mid & (idx % 2 == 1), idx + 1, idx)
    return np.where(a64 >= 6.0, 7, code).astype(np.uint8)


def test_e2m1_rounding_near_every_threshold(orc):
    grid = np.array(GRID)
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(11)
    a = np.concatenate([
        _neigh(list(grid) + list(mids), 1 << 14),
        rng.integers(0, 0x41000000, size=1 << 21, dtype=np.uint32).view(np.float32),
        np.array([6.0, 7.0, 5.0000005, 1e30, 3.4028235e38, np.inf], np.float32)])
    got = orc.e2m1_round_mag(a)
    want = _e2m1_by_midpoints(a)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (a[bad[:5]], got[bad[:5]], want[bad[:5]])
    # the seven ties resolve to the even code
    assert list(orc.e2m1_round_mag(mids)) == [0, 2, 2, 4, 4, 6, 6]


# ----------------------------------------------------------------------------- E4M3
def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch(orc):
    b = np.array([v for v in range(256) if v not in (0x7F, 0xFF)], np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_decode(int(v)) for v in b])
    assert np.array_equal(got, want)
    assert orc.e4m3_decode(0x7E) == 448.0 and orc.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range(orc):
    vals = np.array([orc.e4m3_decode(b) for b in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(12)
    s = np.concatenate([
        _neigh(list(vals[1:]) + list(mids) + [2.0 ** -10, 464.0], 1 << 11),
        np.arange(0, 1 << 12, dtype=np.uint32).view(np.float32),       # tiny and subnormal
        rng.uniform(0, 464.0, size=1 << 20).astype(np.float32)])
    s = s[(s >= 0) & (s <= 464.0)]
    got = orc.e4m3_encode(s)
    want = _torch_e4m3(s)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (s[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_saturates_instead_of_nan(orc):
    s = np.array([448.0, 464.0, 464.00003, 500.0, 1e10, 3.4028235e38, np.inf], np.float32)
    assert list(orc.e4m3_encode(s)) == [0x7E] * len(s)
    # below half of the smallest subnormal (2^-9) and at exactly half: zero (tie to even)
    assert list(orc.e4m3_encode(np.array([0.0, 2.0 ** -11, 2.0 ** -10], np.float32))) == [0, 0, 0]


# ----------------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(13)
    u = rng.integers(0, 0x7F800000, size=1 << 20, dtype=np.uint32)
    ties = (u & 0xFFFF0000) | 0x8000
    sub = rng.integers(0, 0x00800000, size=1 << 16, dtype=np.uint32)
    top = np.arange(0x7F7F0000, 0x7F800000, 7, dtype=np.uint32)       # rounds to inf at the top
    allu = np.concatenate([u, ties, sub, top])
    allu = np.concatenate([allu, allu | 0x80000000])
    f = allu.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_rne(f), want)


# ----------------------------------------------------------------------------- alpha
def test_alpha_closed_forms(orc):
    # alpha uses 6 * 448 for standard NVFP4 and 6 * 256 for Four Over Six
    assert orc.alpha(6.0, "four_over_six") == 2.0 ** -8
    assert orc.alpha(5.25, "rtn6") == 2.0 ** -9
    assert orc.alpha(2688.0, "rtn6") == 1.0 and orc.alpha(1536.0, "four_over_six") == 1.0
    assert orc.alpha(0.0, "rtn6") == 0.0 and orc.alpha(0.0, "four_over_six") == 0.0
    assert orc.alpha(448.0 * 6, "four_over_six") == np.float32(1.75)


def test_alpha_is_the_correctly_rounded_quotient(orc):
    rng = np.random.default_rng(14)
    amax = bf16_to_f32(rng.integers(1, 0x7F80, size=400, dtype=np.uint16))
    for a in amax:
        for mode, C in (("rtn6", 2688), ("four_over_six", 1536)):
            al = orc.alpha(float(a), mode)
            q = Fraction(float(a)) / C
            # nearest binary32 to q: no binary32 neighbour of al is closer
            up = np.nextafter(al, np.float32(np.inf))
            dn = np.nextafter(al, np.float32(0))
            d0 = abs(Fraction(float(al)) - q)
            assert d0 <= abs(Fraction(float(up)) - q) and d0 <= abs(Fraction(float(dn)) - q)


# ----------------------------------------------------------------------------- worked examples
@pytest.mark.parametrize("ex", read_examples(), ids=lambda e: e["name"])
def test_worked_example(orc, ex):
    x = bf16_bits(ex["input"]).reshape(1, -1)
    for rule in ex["rules"]:
        r = orc.quantize(x, ex["mode"], rule)
        assert int(r["alpha"].view(np.uint32)[0]) == ex["alpha_bits"], rule
        assert list(r["scales"].ravel()) == ex["scales"], rule
        assert list(r["codes"].ravel()) == ex["codes"], rule
        assert np.array_equal(r["y"].ravel(), bf16_bits(ex["y"])), rule
        q = orc.quantize(x, ex["mode"], rule, want_qstar=True)["qstar"]
        assert list(q.ravel()) == ex["qstar"], rule
        assert list(orc.quantize_stats(x, ex["mode"], rule)[0]) == ex["stats"], rule


def test_page_fact_four_is_two_thirds_of_the_max_under_scale_six(orc):
    # rtn6 block with exact step d = 0.875 (amax 5.25): 3.5 is 66.6 % of the max and is
    # FP4 "4" exactly; values between 66.6 % and 100 % of the max are not representable.
    x = bf16_bits([5.25, 3.5, 4.375, 5.0] + [0.0] * 12)
    mag, s, xh, _ = orc.candidate(x, orc.alpha(5.25, "rtn6"), 6, "mse")
    assert s == 0x7E and orc.e4m3_decode(s) * 2.0 ** -9 == 0.875
    assert mag[0] == 7 and xh[0] == 5.25
    assert mag[1] == 6 and xh[1] == 3.5 and xh[1] / 5.25 == pytest.approx(2 / 3)
    assert xh[2] != 4.375 and xh[3] != 5.0


def test_page_fact_75_percent_is_three_under_scale_four(orc):
    x = bf16_bits([6.0, 4.5] + [0.0] * 14)   # 4.5 = 75 % of the block max
    al = orc.alpha(6.0, "four_over_six")
    mag4, s4, xh4, _ = orc.candidate(x, al, 4, "mse")
    mag6, s6, xh6, _ = orc.candidate(x, al, 6, "mse")
    assert mag4[1] == 5 and orc.e2m1_decode(5) == 3.0 and xh4[1] == 4.5   # exactly "3"
    assert mag6[1] == 6 and xh6[1] == 4.0                                 # in the 4..6 gap
    assert orc.e4m3_decode(s4) / orc.e4m3_decode(s6) == 1.5               # 1.5x larger scale
    for rule in ("mse", "mae", "maxerr"):
        _, _, _, dbg = orc.quantize_block(x, al, "four_over_six", rule)
        assert dbg["qstar"] == 4


def _random_blocks(n, seed):
    """n blocks of 16 bf16 values with widely varying magnitudes and shapes."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 16)).astype(np.float32)
    x *= np.exp(rng.uniform(-6, 6, size=(n, 1))).astype(np.float32)
    x[rng.random((n, 16)) < 0.05] = 0.0
    spikes = rng.random(n) < 0.3
    x[spikes, rng.integers(0, 16, size=spikes.sum())] *= 8
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_scale_four_blocks_stay_in_four_and_scale_ratio(orc):
    blocks = _random_blocks(3000, 21)
    x = blocks.reshape(1, -1)
    for rule in ("mse", "mae", "maxerr"):
        r = orc.quantize(x, "four_over_six", rule, want_qstar=True)
        al = float(r["alpha"][0])
        q = r["qstar"].ravel()
        codes = r["codes"].reshape(-1, 8)
        lo, hi = codes & 7, (codes >> 4) & 7
        four = q == 4
        assert four.any() and (q == 6).any()
        assert lo[four].max() <= 6 and hi[four].max() <= 6         # blocks scaled to 4: [-4, 4]
        assert r["scales"].max() <= 0x7C                             # 256 * 1.5 = 384 at most
        for b in np.nonzero(four)[0][:200]:
            _, s6, _, _ = orc.candidate(blocks[b], al, 6, rule)
            _, s4, _, _ = orc.candidate(blocks[b], al, 4, rule)
            if s6 >= 0x08:                                             # normal E4M3 range
                ratio = orc.e4m3_decode(s4) / orc.e4m3_decode(s6)
                assert 1.5 * (15 / 16) / (17 / 16) <= ratio <= 1.5 * (17 / 16) / (15 / 16)
    r6 = orc.quantize(x, "rtn6", "mse")
    amax_block = np.argmax(np.abs(bf16_to_f32(blocks)).max(axis=1))
    assert r6["scales"].ravel()[amax_block] == 0x7E                  # the amax block maps to 448


def test_selection_keeps_the_smaller_error_ties_to_six(orc):
    blocks = _random_blocks(2000, 22)
    al = orc.alpha(float(np.abs(bf16_to_f32(blocks)).max()), "four_over_six")
    for rule in ("mse", "mae", "maxerr"):
        for b in blocks:
            _, _, _, d = orc.quantize_block(b, al, "four_over_six", rule)
            want = 4 if d["err4"] < d["err6"] else 6
            assert d["qstar"] == want


def _nearest_code_exact(x: Fraction, d: Fraction, cap: int):
    """Brute force over the FP4 magnitudes allowed by the cap; ties to the even code."""
    best, bestd = None, None
    for m in range(cap + 1):
        dist = abs(abs(x) - Fraction(GRID[m]) * d)
        if bestd is None or dist < bestd or (dist == bestd and m % 2 == 0):
            best, bestd = m, dist
    return best


def test_brute_force_nearest_codes_scales_and_choice(orc):
    """Exact-arithmetic brute force on tiny inputs: per candidate the scale is the nearest
    E4M3 value to bmax / (Q*alpha), each value takes the nearest allowed FP4 code of x/d,
    and the chosen candidate has the smaller exact error.  Binary32 rounding of the
    intermediate steps may flip a decision only within a relative 2^-18 of a tie."""
    blocks = _random_blocks(300, 23)
    e4 = [Fraction(orc.e4m3_decode(b)) for b in range(0x7F)]
    tol = Fraction(1, 1 << 18)
    for rule in ("mse", "mae", "maxerr"):
        for blk in blocks:
            xf = [Fraction(float(v)) for v in bf16_to_f32(blk)]
            bmax = max(abs(v) for v in xf)
            amax = float(bmax) * 1.3
            al = orc.alpha(amax, "four_over_six")
            errs = {}
            for Q in (6, 4):
                mag, s, xh, err = orc.candidate(blk, al, Q, rule)
                sigma = bmax / (Q * Fraction(float(al)))
                dist = [abs(sigma - v) for v in e4]
                best = min(dist)
                near = [b for b, dd in enumerate(dist) if dd - best <= tol * max(sigma, Fraction(1, 1 << 9))]
                assert s in near
                d = e4[s] * Fraction(float(al))
                cap = 6 if Q == 4 else 7
                for i, xv in enumerate(xf):
                    m = _nearest_code_exact(xv, d, cap)
                    if m != mag[i]:
                        # allowed only next to a rounding threshold of x/d
                        t = abs(xv) / d
                        mids = [Fraction(GRID[k] + GRID[k + 1]) / 2 for k in range(7)]
                        assert min(abs(t - mm) for mm in mids) <= tol * max(t, 1), (xv, d)
                ex = [xv - Fraction(float(h)) for xv, h in zip(xf, xh)]
                if rule == "mse":
                    exact = sum(e * e for e in ex)
                elif rule == "mae":
                    exact = sum(abs(e) for e in ex)
                else:
                    exact = max(abs(e) for e in ex)
                assert abs(Fraction(float(err)) - exact) <= tol * max(exact, Fraction(1, 10 ** 30))
                errs[Q] = exact
            _, _, _, dbg = orc.quantize_block(blk, al, "four_over_six", rule)
            gap = abs(errs[4] - errs[6])
            if gap > tol * max(errs[4], errs[6]):
                assert dbg["qstar"] == (4 if errs[4] < errs[6] else 6)


# ----------------------------------------------------------------------------- invariants
SMALL = [("tiny", (64, 256)), ("weight", (48, 448)), ("act", (96, 128)),
         ("large", (40, 224)), ("moe", (3, 24, 80))]


def _small(name, shape):
    return W.bits(W.generate(name, shape))


@pytest.mark.parametrize("name,shape", SMALL)
@pytest.mark.parametrize("mode,rule", [("rtn6", "mse"), ("four_over_six", "mse"),
                                       ("four_over_six", "mae"), ("four_over_six", "maxerr")])
def test_invariants_scaling_sign_decode(orc, name, shape, mode, rule):
    x = _small(name, shape)
    base = orc.quantize(x, mode, rule)
    # 1. scaling the tensor by 2^k scales alpha and y by 2^k and leaves every byte alone
    for k in (-5, 3):
        xs = bf16_bits(bf16_to_f32(x) * np.float32(2.0 ** k))
        r = orc.quantize(xs, mode, rule)
        assert np.array_equal(r["alpha"], base["alpha"] * np.float32(2.0 ** k))
        assert np.array_equal(r["codes"], base["codes"])
        assert np.array_equal(r["scales"], base["scales"])
        assert np.array_equal(bf16_to_f32(r["y"]), bf16_to_f32(base["y"]) * np.float32(2.0 ** k))
    # 2. x -> -x flips exactly the sign bits
    r = orc.quantize(x ^ np.uint16(0x8000), mode, rule)
    assert np.array_equal(r["codes"], base["codes"] ^ np.uint8(0x88))
    assert np.array_equal(r["scales"], base["scales"])
    assert np.array_equal(r["y"], base["y"] ^ np.uint16(0x8000))
    # 3. decoding the packed output gives the fake-quant output bit for bit
    codes = base["codes"].reshape(-1, 8)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(-1, 16)
    val = np.array([orc.e2m1_decode(c) for c in range(16)], np.float32)[nib]
    E = x.shape[0] if x.ndim == 3 else 1
    al = np.repeat(base["alpha"], nib.shape[0] // E).astype(np.float32)
    dec = np.array([orc.e4m3_decode(b) for b in range(256)], np.float64).astype(np.float32)
    step = dec[base["scales"].ravel()] * al
    xhat = val * step[:, None]
    y = torch.from_numpy(xhat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y.reshape(x.shape), base["y"])
    assert orc.inexact_subtractions() == 0


def test_permutation_locality_threads_and_batching(orc):
    x = _small("large", (40, 224))
    base = orc.quantize(x, "four_over_six", "mae")
    perm = np.random.default_rng(5).permutation(x.shape[0])
    r = orc.quantize(x[perm], "four_over_six", "mae")
    assert np.array_equal(r["codes"], base["codes"][perm])
    assert np.array_equal(r["scales"], base["scales"][perm])
    # changing one block without moving the amax changes only that block
    x2 = x.copy()
    x2[7, 32:48] = bf16_bits(np.arange(-8, 8, dtype=np.float32) / 8)
    r2 = orc.quantize(x2, "four_over_six", "mae")
    diff = np.nonzero((r2["scales"] != base["scales"]).ravel())[0]
    assert set(diff) <= {7 * 14 + 2}
    cd = np.nonzero((r2["codes"].reshape(-1, 8) != base["codes"].reshape(-1, 8)).any(1))[0]
    assert set(cd) <= {7 * 14 + 2}
    # threads do not change the result
    r3 = orc.quantize(x, "four_over_six", "mae", nthreads=3)
    for k in ("codes", "scales", "alpha", "y"):
        assert np.array_equal(r3[k], base[k])
    # batched tensors = each tensor alone, one alpha per tensor
    xb = _small("moe", (3, 24, 80))
    rb = orc.quantize(xb, "four_over_six", "mse")
    for e in range(3):
        re = orc.quantize(xb[e], "four_over_six", "mse")
        assert np.array_equal(rb["codes"][e], re["codes"])
        assert np.array_equal(rb["scales"][e], re["scales"])
        assert rb["alpha"][e] == re["alpha"][0]


@pytest.mark.parametrize("bad", [0x7FC0, 0x7F80, 0xFF80, 0xFFC1])
def test_non_finite_input_poisons_only_its_tensor(orc, bad):
    xb = _small("moe", (3, 16, 64)).copy()
    xb[1, 5, 17] = bad
    r = orc.quantize(xb, "four_over_six", "mse")
    assert np.isnan(r["alpha"][1]) and int(r["alpha"].view(np.uint32)[1]) == 0x7FC00000
    assert (r["scales"][1] == 0x7F).all() and (r["codes"][1] == 0).all()
    assert (r["y"][1] == 0x7FC0).all()
    ok = orc.quantize(xb[0], "four_over_six", "mse")
    assert np.array_equal(r["codes"][0], ok["codes"]) and not np.isnan(r["alpha"][0])


def test_tiny_and_subnormal_tensors_are_consistent(orc):
    """alpha subnormal (amax < 1536 * 2^-126): the scale clamp and the division fallback
    are live.  Packed decode must still equal the fake-quant output."""
    rng = np.random.default_rng(31)
    for lo_exp in (-133, -128, -120, -110):
        mags = rng.integers(0, 0x0100 + (lo_exp + 133) * 0x80, size=(8, 64), dtype=np.uint16)
        x = mags | (rng.integers(0, 2, size=mags.shape, dtype=np.uint16) << 15)
        for mode in ("rtn6", "four_over_six"):
            r = orc.quantize(x, mode, "mse")
            codes = r["codes"].reshape(-1, 8)
            nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(-1, 16)
            val = np.array([orc.e2m1_decode(c) for c in range(16)], np.float32)[nib]
            dec = np.array([orc.e4m3_decode(b) for b in range(256)]).astype(np.float32)
            step = dec[r["scales"].ravel()] * r["alpha"][0]
            xhat = val * step[:, None]
            y = torch.from_numpy(xhat).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(y.reshape(x.shape), r["y"])
    assert orc.inexact_subtractions() == 0


def _rn32(q: Fraction) -> Fraction:
    """IEEE binary32 round-to-nearest-even of an exact rational (with subnormals)."""
    if q == 0:
        return Fraction(0)
    sgn = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    qe = max(e - 23, -149)
    scaled = q / Fraction(2) ** qe
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * n * Fraction(2) ** qe


def test_error_sums_follow_the_sequential_binary32_definition(orc):
    """The reading fixes the error reduction: i = 0..15 in order, MSE by fused
    multiply-add (one rounding per step), MAE by one rounded add per step, max exact.
    Recomputed here from the IEEE definition with exact rationals."""
    blocks = _random_blocks(400, 41)
    al = orc.alpha(float(np.abs(bf16_to_f32(blocks)).max()), "four_over_six")
    fused_differs = 0
    for blk in blocks:
        xf = [Fraction(float(v)) for v in bf16_to_f32(blk)]
        for Q in (6, 4):
            for rule in ("mse", "mae", "maxerr"):
                _, _, xh, err = orc.candidate(blk, al, Q, rule)
                acc = Fraction(0)
                unfused = Fraction(0)
                for xv, h in zip(xf, xh):
                    e = xv - Fraction(float(h))
                    if rule == "mse":
                        acc = _rn32(e * e + acc)
                        unfused = _rn32(_rn32(e * e) + unfused)
                    elif rule == "mae":
                        acc = _rn32(acc + abs(e))
                    else:
                        acc = max(acc, abs(e))
                assert Fraction(float(err)) == acc, (rule, Q)
                fused_differs += rule == "mse" and unfused != acc
    assert fused_differs > 0          # the data does tell fused from unfused sums


def test_scale_four_candidate_is_capped_at_four_with_subnormal_scales(orc):
    """Blocks scaled to 4 give up the FP4 values 5 and 6 and live in [-4, 4]; with a
    subnormal E4M3 scale the scaled values can exceed 5, and they must stop at 4."""
    rng = np.random.default_rng(42)
    al = orc.alpha(6.0, "four_over_six")
    bit = 0
    for _ in range(300):
        mags = np.exp(rng.uniform(np.log(2.0 ** -20), np.log(2.0 ** -14))) * \
            rng.uniform(0.2, 1.0, size=16)
        blk = bf16_bits(torch.from_numpy(mags.astype(np.float32)).to(torch.bfloat16)
                        .to(torch.float32).numpy())
        mag, s, xh, _ = orc.candidate(blk, al, 4, "mse")
        assert mag.max() <= 6 and s < 0x08
        d = Fraction(orc.e4m3_decode(s)) * Fraction(float(al))
        xf = [Fraction(float(v)) for v in bf16_to_f32(blk)]
        bit += sum(1 for v in xf if d > 0 and v / d > 5)
        assert all(Fraction(float(h)) <= 4 * d * (1 + Fraction(1, 1 << 20)) for h in xh)
    assert bit > 0                    # the cap was exercised


@pytest.mark.parametrize("name,shape", SMALL)
@pytest.mark.parametrize("mode,rule", [("rtn6", "mse"), ("four_over_six", "mae")])
def test_dequantize_of_packed_equals_fakequant(orc, name, shape, mode, rule):
    """Decoding the packed output reproduces the simulated-quantization output."""
    x = _small(name, shape)
    r = orc.quantize(x, mode, rule)
    assert np.array_equal(orc.dequantize(r["codes"], r["scales"], r["alpha"]), r["y"])


def test_dequantize_closed_forms(orc):
    # scale 0x38 = 1.0, alpha 2^-8: code 0x7 = 6 -> 6/256, code 0xE = -4 -> -4/256, 0x8 -> -0
    codes = np.array([[0x87, 0x0E, 0, 0, 0, 0, 0, 0]], np.uint8)
    y = orc.dequantize(codes, np.array([[0x38]], np.uint8), np.array([2.0 ** -8], np.float32))
    want = bf16_bits([6 / 256, -0.0, -4 / 256, 0.0] + [0.0] * 12)
    assert np.array_equal(y.ravel(), want)
    # NaN scale byte and NaN alpha give NaN blocks
    y = orc.dequantize(codes, np.array([[0x7F]], np.uint8), np.array([1.0], np.float32))
    assert (y == 0x7FC0).all()
    y = orc.dequantize(codes, np.array([[0x38]], np.uint8), np.array([np.nan], np.float32))
    assert (y == 0x7FC0).all()


# ----------------------------------------------------------------------------- error statistics
# Columns: sum e^2, sum |e|, max |e|, sum e^2 over |x| > 2/3 bmax, sum e^2 with binary32
# block scales, count of |x| > 2/3 bmax.
SSE, SAE, MAXERR, SSE_NEAR, SSE_F32, NEAR = range(6)


def test_stats_near_max_band_is_strictly_above_two_thirds(orc):
    # [6, 4, 3, 5, 0...] under rtn6 with amax 6: 4 is exactly 2/3 of the block max, so only
    # 6 and 5 are in the band the pages single out (66.6 % to 100 % of the block max).
    x = bf16_bits([6.0, 4.0, 3.0, 5.0] + [0.0] * 12).reshape(1, 16)
    st = orc.quantize_stats(x, "rtn6", "mse")[0]
    assert st[NEAR] == 2
    # alpha = 6/2688, sigma = RN32(6 / RN32(6 alpha)) rounds to 448; the 5 is the only
    # value that the step cannot hit, so it carries the near-band error alone
    r = orc.quantize(x, "rtn6", "mse")
    xhat = bf16_to_f32(r["y"]).ravel()
    assert st[SSE_NEAR] > 0 and st[SSE_NEAR] <= st[SSE]
    assert xhat[1] == 4.0 and xhat[2] == 3.0


def _exact_stats(orc, x_bits, mode, rule):
    """Brute force in exact rationals from the encoded output: xhat from the codes and
    scale bytes, e = x - xhat exactly, the near band by an exact comparison, and the
    binary32-scale trial recomputed from the IEEE definition with a brute-force nearest
    FP4 value (ties to the even code, capped at 4 for blocks scaled to 4)."""
    r = orc.quantize(x_bits, mode, rule, want_qstar=True)
    al = Fraction(float(r["alpha"][0]))
    xs = bf16_to_f32(x_bits).reshape(-1, 16)
    codes = r["codes"].reshape(-1, 8)
    sse = sae = near_sse = f32_sse = Fraction(0)
    mx, near = Fraction(0), 0
    for b in range(xs.shape[0]):
        xf = [Fraction(float(v)) for v in xs[b]]
        bmax = max(abs(v) for v in xf)
        d = _rn32(Fraction(orc.e4m3_decode(int(r["scales"].ravel()[b]))) * al)
        Q = int(r["qstar"].ravel()[b])
        cq = _rn32(Q * al)
        sig = _rn32(bmax / cq) if al != 0 else Fraction(0)
        du = _rn32(sig * al)
        ru = _rn32(1 / du) if du != 0 else Fraction(0)
        for i, xv in enumerate(xf):
            c = (int(codes[b, i // 2]) >> (4 * (i % 2))) & 15
            xh = _rn32(Fraction(GRID[c & 7]) * d)
            e = abs(xv) - xh                      # xhat carries the sign of x
            sse += e * e
            sae += abs(e)
            mx = max(mx, abs(e))
            if 3 * abs(xv) > 2 * bmax:
                near_sse += e * e
                near += 1
            m = 0
            if du != 0:
                v = abs(_rn32(xv * ru))
                m = _nearest_code_exact(v, Fraction(1), 6 if Q == 4 else 7)
            eu = _rn32(abs(xv) - _rn32(Fraction(GRID[m]) * du))
            f32_sse += eu * eu
    return [sse, sae, mx, near_sse, f32_sse, Fraction(near)]


def test_stats_equal_exact_sums_on_tiny_tensors(orc):
    """Every statistic against exact rational arithmetic: the maximum and the count
    exactly, the sums within one rounding to binary64 plus the long-double accumulation
    (relative 2^-51 at these sizes)."""
    tol = Fraction(1, 1 << 51)
    for seed, (mode, rule) in enumerate([("rtn6", "mse"), ("four_over_six", "mse"),
                                         ("four_over_six", "mae"), ("four_over_six", "maxerr")]):
        blocks = _random_blocks(48, 60 + seed)
        x = blocks.reshape(1, -1)
        got = orc.quantize_stats(x, mode, rule)[0]
        exact = _exact_stats(orc, x, mode, rule)
        for k in (SSE, SAE, SSE_NEAR, SSE_F32):
            assert abs(Fraction(float(got[k])) - exact[k]) <= tol * exact[k], (mode, rule, k)
        assert Fraction(float(got[MAXERR])) == exact[MAXERR]
        assert got[NEAR] == exact[NEAR]
        assert exact[SSE_F32] != exact[SSE]       # the scale rounding shows in the data


@pytest.mark.parametrize("name,shape", SMALL)
@pytest.mark.parametrize("mode,rule", [("rtn6", "mse"), ("four_over_six", "mse"),
                                       ("four_over_six", "mae")])
def test_stats_invariants(orc, name, shape, mode, rule):
    x = _small(name, shape)
    E = x.shape[0] if x.ndim == 3 else 1
    st = orc.quantize_stats(x, mode, rule)
    n = x.size // E
    xb = np.abs(bf16_to_f32(x)).reshape(E, -1, 16)
    nonzero_blocks = (xb.max(axis=2) > 0).sum(axis=1)
    for t in range(E):
        s_ = st[t]
        assert 0 <= s_[SSE_NEAR] <= s_[SSE]
        assert s_[MAXERR] ** 2 <= s_[SSE] * (1 + 1e-12) and s_[SSE] <= n * s_[MAXERR] ** 2
        assert s_[SAE] ** 2 <= n * s_[SSE] * (1 + 1e-12) and s_[SAE] <= n * s_[MAXERR]
        assert nonzero_blocks[t] <= s_[NEAR] <= n        # every block max is in its band
        assert s_[SSE_F32] > 0
    # scaling by 2^k scales the sums exactly (no rounding depends on the exponent here)
    for k in (-4, 3):
        xs = bf16_bits(bf16_to_f32(x) * np.float32(2.0 ** k))
        sk = orc.quantize_stats(xs, mode, rule)
        f = np.array([4.0 ** k, 2.0 ** k, 2.0 ** k, 4.0 ** k, 4.0 ** k, 1.0])
        assert np.array_equal(sk, st * f)
    # the sign of the input does not matter; the thread split changes only rounding
    assert np.array_equal(orc.quantize_stats(x ^ np.uint16(0x8000), mode, rule), st)
    s8 = orc.quantize_stats(x, mode, rule, nthreads=8)
    assert np.allclose(s8, st, rtol=n * 2.0 ** -60, atol=0)
    assert np.array_equal(s8[:, [MAXERR, NEAR]], st[:, [MAXERR, NEAR]])


def test_stats_poisoned_tensor_is_nan(orc):
    x = _small("moe", (3, 24, 80)).copy()
    x[1, 3, 7] = 0x7F80                               # +inf
    st = orc.quantize_stats(x, "four_over_six", "mse")
    assert np.isnan(st[1]).all() and np.isfinite(st[[0, 2]]).all()


# ----------------------------------------------------------------------------- amax, sampled blocks
def _amax_by_numpy(x_bits: np.ndarray, E: int) -> np.ndarray:
    """Per-tensor max |x| of E equal tensors computed with numpy from the bf16 bit patterns
    (bf16 -> binary32 is a 16-bit shift); NaN for a tensor holding a NaN or an infinity."""
    v = bf16_to_f32(np.asarray(x_bits, np.uint16).reshape(E, -1))
    out = np.abs(v).max(axis=1).astype(np.float32)
    out[~np.isfinite(v).all(axis=1)] = np.nan
    return out


def test_amax_of_batches_with_special_values(orc):
    """The per-tensor amax alpha is computed from [4/6, "Implementation details"], pinned to
    an independent numpy reduction: batches with -0, subnormals, +-Inf and NaN, tensors whose
    max sits at their first or last element, and one-element tensors."""
    rng = np.random.default_rng(41)
    E, n = 7, 48
    v = (rng.standard_normal((E, n)).astype(np.float32)
         * np.float32(2.0) ** rng.integers(-20, 20, size=(E, 1)).astype(np.float32))
    x = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    x[0] = 0x8000                                      # all -0: amax 0
    x[1] = rng.integers(1, 0x80, size=n) | (rng.integers(0, 2, size=n) << 15)   # subnormals
    x[2, -1] = 0xF149                                  # max at the last element, negative
    x[3, 0] = 0x7A00                                   # max at the first element
    x[4, 11] = 0xFF80                                  # -Inf
    x[5, 30] = 0x7FC1                                  # NaN
    x[6, 3] = 0x7F80                                   # +Inf
    got = orc.amax(x, E)
    want = _amax_by_numpy(x, E)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))
    assert got[0] == 0.0 and not np.signbit(got[0])
    # each tensor alone gives its own value: no tensor's amax leaks into another's
    for e in range(E):
        one = orc.amax(x[e], 1)
        assert np.array_equal(np.isnan(one), np.isnan(want[e:e + 1]))
        if ok[e]:
            assert one[0] == want[e]
    # one-element tensors (n = 1): the max is the magnitude of the element itself
    single = np.array([0xC020, 0x3F40, 0x8000, 0x000B], np.uint16)   # -2.5, 0.75, -0, 2^-130*11
    assert np.array_equal(orc.amax(single, 4), np.abs(bf16_to_f32(single)))


def test_sampled_blocks_equal_the_whole_tensor_result(orc):
    """orc.quantize_blocks (the checker of sampled blocks at full size) gives, for every block
    id of a batch with one alpha per tensor (from orc.amax and orc.alpha), exactly what
    orc.quantize gives for the whole batch, and the same on shuffled subsets of ids."""
    x = _small("moe", (5, 24, 96))                     # 5 tensors, sigma from 0.005 to 0.05
    E = x.shape[0]
    for mode, rule in (("four_over_six", "mse"), ("four_over_six", "maxerr"), ("rtn6", "mse")):
        whole = orc.quantize(x, mode, rule, want_qstar=True)
        al = np.array([orc.alpha(a, mode) for a in orc.amax(x, E)], np.float32)
        assert np.array_equal(al.view(np.uint32), whole["alpha"].view(np.uint32))
        assert len(set(al.tolist())) == E              # every tensor has its own alpha
        nb = x.size // 16
        ids = np.arange(nb)
        r = orc.quantize_blocks(x, al, ids, mode, rule)
        assert np.array_equal(r["codes"], whole["codes"].reshape(-1, 8))
        assert np.array_equal(r["scales"], whole["scales"].ravel())
        assert np.array_equal(r["y"], whole["y"].reshape(-1, 16))
        assert np.array_equal(r["qstar"], whole["qstar"].ravel())
        rng = np.random.default_rng(42)
        for k in (1, 17, nb // 3):
            sel = rng.permutation(nb)[:k]
            rs = orc.quantize_blocks(x, al, sel, mode, rule)
            assert np.array_equal(rs["codes"], whole["codes"].reshape(-1, 8)[sel])
            assert np.array_equal(rs["scales"], whole["scales"].ravel()[sel])
            assert np.array_equal(rs["y"], whole["y"].reshape(-1, 16)[sel])
    # a poisoned tensor (alpha NaN) poisons only its own sampled blocks
    al = np.array([orc.alpha(a, "four_over_six") for a in orc.amax(x, E)], np.float32)
    al[2] = np.nan
    nb1 = x[0].size // 16
    sel = np.array([2 * nb1 + 3, 1 * nb1 + 3, 3 * nb1 + 3])
    rs = orc.quantize_blocks(x, al, sel, "four_over_six", "mse")
    assert rs["scales"][0] == 0x7F and (rs["codes"][0] == 0).all()
    assert rs["scales"][1] != 0x7F and rs["scales"][2] != 0x7F
