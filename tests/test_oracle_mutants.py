"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case below copies the oracle's C++ source, changes one thing in it (a wrong
tensor offset, a tie sent the wrong way, a constant swapped, a term dropped),
builds the copy, routes the oracle module to it, and runs the pins that claim to
cover that part: at least one of them must fail.  A pin that passes on a mutant
would not have caught that mistake in the oracle itself.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import test_oracle_pins as P
import test_oracle_shadow as S
from helpers import read_examples

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _examples(orc):
    for ex in read_examples():
        P.test_worked_example(orc, ex)


def _invariants(orc):
    for name, shape in P.SMALL[:3]:
        for mode, rule in (("rtn6", "mse"), ("four_over_six", "mse")):
            P.test_invariants_scaling_sign_decode(orc, name, shape, mode, rule)


def _shadow_brute(orc):
    for mode, rule in (("rtn6", "mse"), ("four_over_six", "mse"), ("four_over_six", "maxerr")):
        S.test_shadow_equals_exact_rational_brute_force(orc, mode, rule)


# (name, text to replace, replacement, which occurrence, occurrences expected, pins)
MUTANTS = [
    ("amax: tensor offset t instead of t*n", "tensor_amax(in + t * n, n)",
     "tensor_amax(in + t, n)", 0, 1, [P.test_amax_of_batches_with_special_values]),
    ("amax: only NaN poisons, not Inf", "if (!std::isfinite(x)) return NAN;",
     "if (std::isnan(x)) return NAN;", 0, 1, [P.test_amax_of_batches_with_special_values]),
    ("amax: signed max", "amax = std::max(amax, std::fabs(x));", "amax = std::max(amax, x);",
     0, 1, [P.test_amax_of_batches_with_special_values]),
    ("sampled blocks: alpha of the first tensor", "alpha[b / nb]", "alpha[0]", 0, 1,
     [P.test_sampled_blocks_equal_the_whole_tensor_result]),
    ("sampled blocks: alpha indexed by position in the selection", "alpha[b / nb]",
     "alpha[k / nb]", 0, 1, [P.test_sampled_blocks_equal_the_whole_tensor_result]),
    ("sampled blocks: input at the selection index", "in[b * 16 + i]", "in[k * 16 + i]", 0, 1,
     [P.test_sampled_blocks_equal_the_whole_tensor_result]),
    ("E2M1 ties to the odd code", "(dist == bestd && (c & 1) == 0)",
     "(dist == bestd && (c & 1) == 1)", 0, 2,
     [P.test_e2m1_rounding_near_every_threshold, _examples]),
    ("no cap at 4 for blocks scaled to 4", "const int cap = Q == 4 ? 6 : 7;",
     "const int cap = 7;", 0, 2, [P.test_scale_four_candidate_is_capped_at_four_with_subnormal_scales]),
    ("448 and 256 swapped in alpha", "1536.0f : 2688.0f", "2688.0f : 1536.0f", 0, 1,
     [P.test_alpha_closed_forms, _examples]),
    ("candidate tie goes to 4", "if (c4.err < c6.err) win = &c4;",
     "if (c4.err <= c6.err) win = &c4;", 0, 1, [_examples]),
    ("nibbles swapped", "codes8[j] = uint8_t(lo | (hi << 4));",
     "codes8[j] = uint8_t(hi | (lo << 4));", 0, 2, [_examples]),
    ("unfused squared error", "acc = std::fma(e, e, acc);", "acc = acc + e * e;", 0, 1,
     [P.test_error_sums_follow_the_sequential_binary32_definition]),
    ("block scale bmax * c instead of bmax / c", "bmax / cq", "bmax * cq", 0, 1,
     [_examples]),
    ("E4M3 ties to the odd byte", "(dist == bestd && (b & 1) == 0)",
     "(dist == bestd && (b & 1) == 1)", 0, 2, [P.test_e4m3_encode_matches_torch_in_range]),
    ("last element left out of the block max",
     "for (int i = 0; i < 16; ++i) bmax = std::max(bmax, std::fabs(x[i]));",
     "for (int i = 0; i < 15; ++i) bmax = std::max(bmax, std::fabs(x[i]));", 0, 2,
     [P.test_brute_force_nearest_codes_scales_and_choice, _invariants]),
    ("sign bit from x < 0 (loses -0)", "std::signbit(x[2 * j])", "(x[2 * j] < 0)", 0, 1,
     [_examples, _invariants]),
    # the exact-quotient shadow
    ("shadow: E2M1 ties to the odd code", "(dist == bestd && (c & 1) == 0)",
     "(dist == bestd && (c & 1) == 1)", 1, 2,
     [S.test_shadow_resolves_exact_ties_to_the_even_code, _shadow_brute]),
    ("shadow: E4M3 ties to the odd byte", "(dist == bestd && (b & 1) == 0)",
     "(dist == bestd && (b & 1) == 1)", 1, 2,
     [S.test_shadow_resolves_exact_scale_ties_to_the_even_byte, _shadow_brute]),
    ("shadow: no cap at 4", "const int cap = Q == 4 ? 6 : 7;", "const int cap = 7;", 1, 2,
     [_shadow_brute]),
    ("shadow: candidate tie goes to 4", "if (cmp < 0) win = &c4;", "if (cmp <= 0) win = &c4;",
     0, 1, [S.test_shadow_worked_examples, _shadow_brute]),
    ("shadow: |e| summed instead of e^2", "c->sum.add((unsigned __int128)mm * mm, 2 * kk);",
     "c->sum.add(mm, kk);", 0, 1, [_shadow_brute]),
    ("shadow: 448 and 256 swapped in the exact alpha", "1536 : 2688", "2688 : 1536", 0, 1,
     [_shadow_brute]),
    ("shadow: bf16 output not divided back", "a - c * xf(bf16_pattern_value(t))",
     "a - xf(bf16_pattern_value(t))", 0, 1, [_shadow_brute]),
    ("shadow: nibbles swapped", "codes8[j] = uint8_t(lo | (hi << 4));",
     "codes8[j] = uint8_t(hi | (lo << 4));", 1, 2, [S.test_shadow_worked_examples]),
]


def _mutate(src: str, old: str, new: str, occ: int, count: int) -> str:
    assert src.count(old) == count, "mutation site moved: %r" % old
    i = -1
    for _ in range(occ + 1):
        i = src.index(old, i + 1)
    return src[:i] + new + src[i + len(old):]


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(os.path.join(ORACLE, "nvfp4_oracle.cpp")).read()
    root = tmp_path_factory.mktemp("mutants")

    def build(k):
        name, old, new, occ, count, _ = MUTANTS[k]
        d = root / ("m%02d" % k)
        d.mkdir()
        shutil.copy(os.path.join(ORACLE, "nvfp4_oracle.h"), d)
        (d / "nvfp4_oracle.cpp").write_text(_mutate(src, old, new, occ, count))
        lib = str(d / "libm.so")
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", "-o", lib, str(d / "nvfp4_oracle.cpp")])
        return lib

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return list(ex.map(build, range(len(MUTANTS))))


@pytest.mark.parametrize("k", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(orc, mutant_libs, k):
    name, _, _, _, _, pins = MUTANTS[k]
    caught = []
    with orc.using(mutant_libs[k]):
        for pin in pins:
            try:
                pin(orc)
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, "no pin caught the planted mistake: %s" % name
