"""HIP graph capture of the library's launches (GPU).

The library launches only kernels (its accumulator clear is a kernel, not a memset), so a
call can be captured into a HIP graph and replayed.  Each graph here is replayed several
times with other eager work and synchronizations between the replays, and every replay
is compared with the eager result."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_amax_amd as m
    m.lib()
    return m


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("shape", [(96, 448), (3, 40, 160)], ids=["2d", "batched"])
@pytest.mark.parametrize("mode,rule", [("rtn6", "mse"), ("four_over_six", "mae")])
def test_graph_replays_match_eager(nv, orc, shape, mode, rule):
    x = W.generate("large", shape).cuda()
    other = W.generate("weight", shape).cuda()
    E = shape[0] if len(shape) == 3 else 1
    lead = shape[:-2]
    codes = torch.empty(lead + (shape[-2], shape[-1] // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty(lead + (shape[-2], shape[-1] // 16), dtype=torch.uint8, device="cuda")
    alpha = torch.empty(E, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    alpha_y = torch.empty(E, dtype=torch.float32, device="cuda")
    am = torch.empty(E, dtype=torch.float32, device="cuda")
    codes2, scales2, alpha2 = torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(alpha)
    codes3, scales3, alpha3 = torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(alpha)
    y3, alpha_y3 = torch.empty_like(x), torch.empty_like(alpha)
    ws = torch.empty(nv.FUSED_WS_WORDS * E, dtype=torch.int32, device="cuda")
    dws = torch.empty(nv.diag_ws_words(E), dtype=torch.int32, device="cuda")
    codes4, scales4, alpha4 = torch.empty_like(codes), torch.empty_like(scales), torch.empty_like(alpha)
    qstar = torch.empty_like(scales)
    count4 = torch.empty(E, dtype=torch.int32, device="cuda")
    stats = torch.empty((E, len(nv.STATS)), dtype=torch.float64, device="cuda")

    def diag():
        st = nv.lib().nvfp4_quantize_diag(
            x.data_ptr(), E, shape[-2], shape[-1], 16, nv.MODES[mode], nv.RULES[rule],
            codes4.data_ptr(), scales4.data_ptr(), alpha4.data_ptr(), qstar.data_ptr(),
            count4.data_ptr(), stats.data_ptr(), dws.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    def work():
        nv.quantize(x, mode, rule, codes=codes, scales=scales, alpha=alpha)
        nv.fakequant(x, mode, rule, out=y, alpha=alpha_y)
        nv.amax(x, out=am)
        nv.quantize_from_amax(x, am, mode, rule, codes=codes2, scales=scales2, alpha=alpha2)
        nv.quantize_fused(x, mode, rule, codes=codes3, scales=scales3, alpha=alpha3, workspace=ws)
        nv.fakequant_fused(x, mode, rule, out=y3, alpha=alpha_y3, workspace=ws)
        diag()                                    # statistics: counters reset by the call

    work()
    torch.cuda.synchronize()
    outs = (codes, scales, alpha, y, alpha_y, am, codes2, scales2, alpha2, codes3, scales3,
            alpha3, y3, alpha_y3, codes4, scales4, alpha4, qstar, count4, stats)
    ref = [t.clone() for t in outs]
    g = _capture(work)
    for r in range(4):
        for t in outs:
            t.zero_()
        nv.quantize(other, mode, rule)            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (t, e) in enumerate(zip(outs, ref)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), (r, k)
    # the eager result itself is the oracle's
    xb = W.bits(x.cpu())
    o = orc.quantize(xb, mode, rule)
    assert np.array_equal(codes.cpu().numpy(), o["codes"])
    assert np.array_equal(W.bits(y.cpu()), o["y"])
    assert torch.equal(codes3, codes) and torch.equal(y3, y) and torch.equal(alpha3, alpha)
    assert torch.equal(codes4, codes) and torch.equal(scales4, scales)


@pytest.mark.parametrize("shape,fq", [((600, 256, 256), False), ((4096, 4112), True),
                                      ((6, 1024, 16384), False)],
                         ids=["teams-small", "tier12-fq", "teams-large"])
def test_graph_replays_of_fused_tiers_and_teams(nv, shape, fq):
    """The single-read call in its spread tiers and in team mode, captured and replayed: every
    replay equals the eager two-pass result."""
    x = W.generate("moe" if len(shape) == 3 else "weight", shape).cuda()
    E = shape[0] if len(shape) == 3 else 1
    lead = shape[:-2]
    ws = torch.empty(nv.FUSED_WS_WORDS * E, dtype=torch.int32, device="cuda")
    if fq:
        out, al = torch.empty_like(x), torch.empty(E, dtype=torch.float32, device="cuda")
        ref = nv.fakequant(x, "four_over_six", "mse")
        outs = (out, al)
        work = lambda: nv.fakequant_fused(x, "four_over_six", "mse", out=out, alpha=al, workspace=ws)
    else:
        c = torch.empty(lead + (shape[-2], shape[-1] // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty(lead + (shape[-2], shape[-1] // 16), dtype=torch.uint8, device="cuda")
        al = torch.empty(E, dtype=torch.float32, device="cuda")
        ref = nv.quantize(x, "four_over_six", "mse")
        outs = (c, s, al)
        work = lambda: nv.quantize_fused(x, "four_over_six", "mse", codes=c, scales=s, alpha=al,
                                         workspace=ws)
    torch.cuda.synchronize()
    print("[graph] fused %s fq=%s: %d blocks per lane" % (
        shape, fq, nv.fused_blocks_per_lane(shape, "four_over_six", "mse", fq)), flush=True)
    assert nv.fused_blocks_per_lane(shape, "four_over_six", "mse", fq) > 0
    g = _capture(work)
    for r in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (t, e) in enumerate(zip(outs, ref)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), (r, k)
