"""Single-read (fused) dynamic quantization on the GPU, through the C ABI, against the oracle.

The fused entry points must give the dynamic entry points' results bit for bit: codes, scale
bytes, alpha bits and fake-quant bf16 bits equal to the oracle's.  Covered here: every tier of
blocks held per lane (1, 4 and 12 in 256-thread workgroups, 10 and 10 + 4 in 1024-thread ones, 28,
confirmed through the shape query), the batched form,
batches run in teams (10 or 20 per lane, in workgroups of 256, 512 or 1024 threads; the 64-expert
MoE batch whole),
the edge tensors, poisoning, the bounded grid-wide wait forced from the host (every workgroup
or some of them computing the tensor amax alone), the two-pass route for tensors that do not
fit on chip and for in-place fake-quant, and a workspace that starts with arbitrary content."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W
from test_gpu_parity import EDGE, RUNS, SMALL, to_gpu, u16

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
    yield m
    m.set_fused_wait_limit(-1)


def run_fused(nv, x_bits, mode, rule, fq, workspace=None):
    xg = to_gpu(x_bits)
    if fq:
        y, al = nv.fakequant_fused(xg, mode, rule, workspace=workspace)
        torch.cuda.synchronize()
        return dict(y=u16(y), alpha=al.cpu().numpy())
    c, s, al = nv.quantize_fused(xg, mode, rule, workspace=workspace)
    torch.cuda.synchronize()
    return dict(codes=c.cpu().numpy(), scales=s.cpu().numpy(), alpha=al.cpu().numpy())


def assert_matches_oracle(orc, x_bits, got, mode, rule, fq, tag):
    ref = orc.quantize(x_bits, mode, rule, nthreads=NTHREADS, want_y=fq)
    E = x_bits.shape[0] if x_bits.ndim == 3 else 1
    assert np.array_equal(got["alpha"].view(np.uint32), ref["alpha"][:E].view(np.uint32)), tag
    if fq:
        assert np.array_equal(got["y"], ref["y"]), tag
    else:
        assert np.array_equal(got["codes"], ref["codes"]), tag
        assert np.array_equal(got["scales"], ref["scales"]), tag


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
@pytest.mark.parametrize("fq", [False, True], ids=["packed", "fakequant"])
def test_fused_small_whole(nv, orc, name, shape, mode, rule, fq):
    x = W.bits(W.generate(name, shape))
    assert nv.fused_blocks_per_lane(shape, mode, rule, fq) >= 1
    assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq), mode, rule, fq, name)


def test_fused_random_shapes(nv, orc):
    """Random shapes with ragged last workgroups, batched or not, every mode and rule, both
    outputs, values spread over 2^-8 to 2^8 in scale."""
    rng = np.random.default_rng(91)
    for k in range(24):
        rows = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 200)) * 16
        E = int(rng.integers(2, 6)) if k % 3 == 0 else None
        shape = (E, rows, cols) if E else (rows, cols)
        x = W.bits(W.normal(shape, seed=2000 + k, sigma=float(np.exp(rng.uniform(-8, 8)))))
        mode, rule = RUNS[k % 4]
        fq = bool((k // 4) % 2)
        assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq), mode, rule, fq,
                              "random%d %s" % (k, shape))


# Shapes that select each tier on a 256-CU MI355X (the test checks the tier it gets).
TIERS = [(1, (256, 256)), (4, (1024, 4112)), (10, (4096, 4112)), (10, (8192, 4096)),
         (12, (100, 328, 1024)), (14, (4096, 14336))]


@pytest.mark.parametrize("tier,shape", TIERS, ids=["tier%d-%s" % (t, "x".join(map(str, s)))
                                                    for t, s in TIERS])
@pytest.mark.parametrize("mode,rule,fq", [("four_over_six", "mse", False),
                                          ("rtn6", "mse", True),
                                          ("four_over_six", "mae", True)],
                         ids=["46mse-packed", "rtn6-fq", "46mae-fq"])
def test_fused_tiers_whole_tensor(nv, orc, tier, shape, mode, rule, fq):
    got_tier = nv.fused_blocks_per_lane(shape, mode, rule, fq)
    say("[fused] %s %s/%s fq=%s: %d blocks per lane" % (shape, mode, rule, fq, got_tier))
    want = 28 if (tier == 14 and mode == "four_over_six" and fq) else tier   # 4/6 fq: (20,8)
    if tier == 14 and got_tier == 0:
        pytest.fail("the weight-sized tensor does not fit on chip on this device")
    assert got_tier >= 1
    if tier in (1, 10, 14) or (tier == 12 and not fq):
        assert got_tier == want, got_tier
    x = W.bits(W.weight(shape, seed=300 + tier))
    assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq), mode, rule, fq,
                          "tier%d" % tier)


def test_fused_tiers_are_all_exercised(nv):
    seen = {nv.fused_blocks_per_lane(s, m, r, f) for _, s in TIERS
            for (m, r, f) in (("four_over_six", "mse", False), ("rtn6", "mse", True),
                              ("four_over_six", "mae", True))}
    assert {1, 4, 10, 12, 14, 28} <= seen, seen


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("mode,rule", RUNS, ids=["-".join(r) for r in RUNS])
def test_fused_edge_cases(nv, orc, name, mode, rule):
    for fq in (False, True):
        assert_matches_oracle(orc, EDGE[name], run_fused(nv, EDGE[name], mode, rule, fq),
                              mode, rule, fq, name)


def test_fused_poison_only_its_tensor(nv, orc):
    x = W.bits(W.generate("moe", (4, 40, 160))).copy()
    x[2, 7, 33] = 0x7FC0             # NaN
    x[0, 0, 0] = 0xFF80              # -inf
    for mode, rule in RUNS:
        for fq in (False, True):
            got = run_fused(nv, x, mode, rule, fq)
            assert_matches_oracle(orc, x, got, mode, rule, fq, "poison")
            assert np.isnan(got["alpha"][[0, 2]]).all() and np.isfinite(got["alpha"][[1, 3]]).all()


@pytest.mark.parametrize("limit", [0, 1], ids=["never-wait", "one-poll"])
@pytest.mark.parametrize("shape", [(5, 130, 320), (1024, 4112), (4096, 4112)],
                         ids=["batched", "tier4", "tier12"])
def test_fused_bounded_wait_fallback(nv, orc, limit, shape):
    """The wait for the other workgroups is cut short from the host: workgroups that stop
    waiting compute the tensor amax alone, and the result does not change."""
    x = W.bits(W.weight(shape, seed=400))
    nv.set_fused_wait_limit(limit)
    try:
        say("[fused] wait limit %d %s" % (limit, shape))
        for mode, rule, fq in (("four_over_six", "mse", False), ("rtn6", "mse", True)):
            assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq), mode, rule, fq,
                                  "limit%d" % limit)
    finally:
        nv.set_fused_wait_limit(-1)


# Batches that no tier holds at once but whose single tensors fit: teams of workgroups take the
# tensors in turn (odd teams start half a cycle late); team_tier gives the blocks per lane.
TEAMS = [((6, 1024, 16384), "four_over_six", "mse", False),     # 2 teams of 1024 threads
         ((10, 1024, 8192), "four_over_six", "mse", False),     # 4 teams of 512 threads
         ((6, 3072, 4096), "four_over_six", "mae", False),      # 4 teams of 512, 9 + 4 per lane
         ((5, 1000, 14336), "four_over_six", "mae", True),
         ((12, 512, 14336), "rtn6", "mse", False),
         ((3, 2048, 14336), "four_over_six", "maxerr", False),
         ((600, 256, 256), "four_over_six", "mse", False),     # one-workgroup teams
         ((700, 128, 512), "four_over_six", "mae", True),
         ((16, 1024, 4096), "rtn6", "mse", False),              # teams of 52 rounded to 64
         ((16, 1024, 4096), "four_over_six", "mae", True)]


def team_tier(shape, mode, fq):
    """Blocks per lane of the team tier a batch gets on a 256-CU MI355X: 10 for tensors under
    262,144 blocks; for Four Over Six into packed output, 10 or 9 + 4 in 512-thread workgroups
    when that makes at least four teams of a power-of-two size (512 resident workgroups), else
    10 in 1024-thread ones; 20 otherwise."""
    E, nblk = shape[0], shape[1] * shape[2] // 16
    if nblk < 2 ** 18:
        return 10
    if mode != "four_over_six" or fq:
        return 20
    for per_lane in (10, 13):
        g = -(-nblk // (per_lane * 512))
        gp = 1 << (g - 1).bit_length()
        if 4 * gp <= 512 and E >= 4:
            return per_lane
    return 10


@pytest.mark.parametrize("shape,mode,rule,fq", TEAMS, ids=["t%d" % i for i in range(len(TEAMS))])
def test_fused_teams_whole_batch(nv, orc, shape, mode, rule, fq):
    tier = nv.fused_blocks_per_lane(shape, mode, rule, fq)
    say("[fused-teams] %s %s/%s fq=%s: %d blocks per lane" % (shape, mode, rule, fq, tier))
    assert tier == team_tier(shape, mode, fq), tier
    x = W.bits(W.generate("moe", shape))
    assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq), mode, rule, fq, str(shape))


def check_limits(nv, orc, x, mode, rule, fq, tag):
    """The call with the wait cut short from the host (no poll, then one poll), against one
    oracle result: workgroups that stop waiting compute the tensor amax alone."""
    ref = orc.quantize(x, mode, rule, nthreads=NTHREADS, want_y=fq)
    E = x.shape[0] if x.ndim == 3 else 1
    for limit in (0, 1):
        nv.set_fused_wait_limit(limit)
        try:
            say("[fused] %s wait limit %d" % (tag, limit))
            got = run_fused(nv, x, mode, rule, fq)
        finally:
            nv.set_fused_wait_limit(-1)
        assert np.array_equal(got["alpha"].view(np.uint32), ref["alpha"][:E].view(np.uint32)), (tag, limit)
        if fq:
            assert np.array_equal(got["y"], ref["y"]), (tag, limit)
        else:
            assert np.array_equal(got["codes"], ref["codes"]), (tag, limit)
            assert np.array_equal(got["scales"], ref["scales"]), (tag, limit)


# Team launches of each kind with the wait cut short: 1024-thread teams, 512-thread teams (the
# Four Over Six loading phase at raised issue priority), teams of the small-tensor tier.
TEAM_LIMITS = [((6, 1024, 16384), "four_over_six", "mse", False, 10),
               ((16, 1024, 4096), "four_over_six", "mse", False, 10),
               ((600, 256, 256), "four_over_six", "mae", True, 10)]


@pytest.mark.parametrize("shape,mode,rule,fq,tier", TEAM_LIMITS,
                         ids=["teams1024", "teams512", "small-teams"])
def test_fused_teams_bounded_wait(nv, orc, shape, mode, rule, fq, tier):
    assert nv.fused_blocks_per_lane(shape, mode, rule, fq) == tier
    x = W.bits(W.generate("moe", shape))
    check_limits(nv, orc, x, mode, rule, fq, "teams %s" % (shape,))


def test_fused_group_wait_bounded(nv, orc):
    """The 28-block fake-quant tier meets at the two-level counter (the other instances use one
    collector workgroup); its bounded wait falls back the same way."""
    shape = (4096, 14336)
    assert nv.fused_blocks_per_lane(shape, "four_over_six", "mae", True) == 28
    x = W.bits(W.weight(shape, seed=401))
    check_limits(nv, orc, x, "four_over_six", "mae", True, "group-form")


def test_fused_teams_moe_full_size(nv, orc):
    """The 64-expert MoE tensor (2048 x 5120 per expert), read once, whole against the oracle."""
    shape = W.WORKLOADS["moe"].shape
    assert nv.fused_blocks_per_lane(shape, "four_over_six", "mse", False) == 10
    xt = W.generate("moe")
    say("[fused-teams] moe %s" % (shape,))
    c, s, a = nv.quantize_fused(xt.cuda(), "four_over_six", "mse")
    torch.cuda.synchronize()
    got = dict(codes=c.cpu().numpy(), scales=s.cpu().numpy(), alpha=a.cpu().numpy())
    del c, s
    assert_matches_oracle(orc, W.bits(xt), got, "four_over_six", "mse", False, "moe")


def test_fused_two_pass_route(nv, orc):
    """A tensor too large to hold on chip and in-place fake-quant take the two-pass path; every
    tensor up to 3,670,016 blocks is read once, in every mode (a single Four Over Six tensor
    into packed output too, in the 1024-thread tiers)."""
    shape = (4096, 16384)                                  # 4.2 M blocks
    assert nv.fused_blocks_per_lane(shape, "four_over_six", "mse", False) == 0
    assert nv.fused_blocks_per_lane(shape, "rtn6", "mse", False) == 0
    assert nv.fused_blocks_per_lane((8192, 4096), "four_over_six", "mae", False) == 10
    assert nv.fused_blocks_per_lane((4096, 14336), "four_over_six", "mae", False) == 14
    for shp in ((4096, 14336), (8192, 4096)):
        assert nv.fused_blocks_per_lane(shp, "rtn6", "mse", False) > 0
        assert nv.fused_blocks_per_lane(shp, "four_over_six", "mae", True) > 0
        assert nv.fused_blocks_per_lane((2,) + shp[:1] + (shp[1] // 2,), "four_over_six",
                                        "mse", False) > 0    # batches read once
    xr = W.bits(W.weight((4096, 14336), seed=501))
    got = run_fused(nv, xr, "four_over_six", "maxerr", False)
    assert_matches_oracle(orc, xr, got, "four_over_six", "maxerr", False, "weight-read-once")
    x = W.bits(W.weight(shape, seed=500))
    got = run_fused(nv, x, "four_over_six", "mse", False)
    assert_matches_oracle(orc, x, got, "four_over_six", "mse", False, "too-large")
    xs = W.bits(W.generate("act", (64, 512)))
    xg = to_gpu(xs)
    y, al = nv.fakequant_fused(xg, "four_over_six", "mae", out=xg)
    torch.cuda.synchronize()
    ref = orc.quantize(xs, "four_over_six", "mae", want_y=True)
    assert np.array_equal(u16(y), ref["y"])


def test_fused_two_streams_at_once(nv, orc):
    """Two single-read calls enqueued together on two streams (default priority), each sized
    to fill the chip: one may find the CUs held by the other, and the bounded wait keeps every
    workgroup moving (a workgroup that gives up computes the tensor amax itself).  Three rounds;
    every result equals the oracle's."""
    xa = W.bits(W.weight((8192, 4096), seed=610))             # 1024-thread tier, whole chip
    xb = W.bits(W.generate("moe", (10, 1024, 8192)))          # 4 teams of 512-thread workgroups
    ga, gb = to_gpu(xa), to_gpu(xb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(3):
        say("[fused] two streams, round %d" % rnd)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            ca, sca, aa = nv.quantize_fused(ga, "four_over_six", "mse")
        with torch.cuda.stream(sb):
            yb, ab = nv.fakequant_fused(gb, "four_over_six", "mae") if rnd % 2 else (None, None)
            if yb is None:
                cb, scb, ab = nv.quantize_fused(gb, "four_over_six", "mse")
        torch.cuda.synchronize()
        assert_matches_oracle(orc, xa, dict(codes=ca.cpu().numpy(), scales=sca.cpu().numpy(),
                                            alpha=aa.cpu().numpy()),
                              "four_over_six", "mse", False, "stream a %d" % rnd)
        if rnd % 2:
            assert_matches_oracle(orc, xb, dict(y=u16(yb), alpha=ab.cpu().numpy()),
                                  "four_over_six", "mae", True, "stream b %d" % rnd)
        else:
            assert_matches_oracle(orc, xb, dict(codes=cb.cpu().numpy(), scales=scb.cpu().numpy(),
                                                alpha=ab.cpu().numpy()),
                                  "four_over_six", "mse", False, "stream b %d" % rnd)


def test_fused_workspace_content_and_reuse(nv, orc):
    """The workspace may hold anything before a call; one workspace serves consecutive calls
    on a stream, and a larger one than needed is fine."""
    ws = torch.full((8 * nv.FUSED_WS_WORDS,), -1, dtype=torch.int32, device="cuda")
    for k, (name, shape) in enumerate(SMALL):
        x = W.bits(W.generate(name, shape))
        mode, rule = RUNS[k % 4]
        for fq in (False, True):
            assert_matches_oracle(orc, x, run_fused(nv, x, mode, rule, fq, workspace=ws),
                                  mode, rule, fq, name)
