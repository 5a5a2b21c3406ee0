"""A tensor of more than 2^27 blocks on the GPU, against the oracle.

Block indices inside a kernel are 32-bit, so the host splits the block pass of a tensor with
2^27 blocks or more into launches over consecutive block ranges (offset pointers, one tensor
per launch).  This runs the dynamic packed, fake-quant and diagnostics calls (with and
without statistics) on a
131080 x 16384 bf16 tensor (2^27 + 8192 blocks, 4.3 GB) and compares the whole packed output,
alpha, the count of blocks scaled to 4, the error statistics (summed over both launches), and
sampled fake-quant and dequantized blocks around the launch boundary with the oracle
(dequantize splits its launches the same way)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_amax_amd import workloads as W
from test_gpu_parity import check_stats

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
ROWS, COLS = 131080, 16384
NBLK = ROWS * COLS // 16
SPLIT = 1 << 27


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


def test_tensor_over_2pow27_blocks(nv, orc):
    assert NBLK > SPLIT
    say("[huge] generating %dx%d (%d blocks)" % (ROWS, COLS, NBLK))
    xt = W.normal((ROWS, COLS), seed=77, sigma=0.5)
    x = W.bits(xt)
    xg = xt.cuda()

    say("[huge] packed, four_over_six/mse")
    c, s, a = nv.quantize(xg, "four_over_six", "mse")
    cq, sq, aq, q, n4, stg = nv.quantize_diag(xg, "four_over_six", "mse")
    torch.cuda.synchronize()
    assert torch.equal(cq, c) and torch.equal(sq, s) and torch.equal(aq, a)
    say("[huge] diagnostics without statistics (counted from the choice bytes after the pass)")
    cp, sp, ap, qp, n4p, _ = nv.quantize_diag(xg, "four_over_six", "mse", stats=False)
    torch.cuda.synchronize()
    assert torch.equal(cp, c) and torch.equal(sp, s) and torch.equal(qp, q) and torch.equal(n4p, n4)
    del cp, sp, qp
    codes, scales = c.cpu().numpy(), s.cpu().numpy()
    qstar_gpu, n4_gpu, stats_gpu = q.cpu().numpy(), int(n4.cpu()[0]), stg.cpu().numpy()
    del cq, sq, q

    say("[huge] dequantize, sampled around the launch boundary")
    rng = np.random.default_rng(78)
    ids = np.unique(np.concatenate([rng.integers(0, NBLK, size=20000),
                                    np.arange(SPLIT - 512, SPLIT + 512),
                                    np.arange(NBLK - 256, NBLK), np.arange(256)]))
    ydq = nv.dequantize(c, s, a)
    torch.cuda.synchronize()
    got = ydq.view(-1, 16)[torch.from_numpy(ids).cuda()].cpu().view(torch.int16).numpy()
    want = orc.dequantize(codes.reshape(-1, 8)[ids].reshape(1, -1, 8),
                          scales.reshape(-1)[ids].reshape(1, -1, 1), a.cpu().numpy())
    assert np.array_equal(got.view(np.uint16).reshape(-1), want.reshape(-1))
    del c, s, ydq

    say("[huge] oracle, whole tensor")
    ref = orc.quantize(x, "four_over_six", "mse", nthreads=NTHREADS, want_y=False,
                       want_qstar=True)
    assert int(a.cpu().numpy().view(np.uint32)[0]) == int(ref["alpha"].view(np.uint32)[0])
    assert np.array_equal(scales, ref["scales"])
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(qstar_gpu, ref["qstar"])
    assert n4_gpu == int((ref["qstar"] == 4).sum()) > 0
    del codes, scales, ref, qstar_gpu

    say("[huge] oracle statistics, whole tensor")
    check_stats(stats_gpu, orc.quantize_stats(x, "four_over_six", "mse", nthreads=NTHREADS),
                x.size, "huge")

    say("[huge] fake-quant, rtn6, sampled around the launch boundary")
    y, a2 = nv.fakequant(xg, "rtn6", "mse")
    torch.cuda.synchronize()
    yb = y.view(-1, 16)[torch.from_numpy(ids).cuda()].cpu().view(torch.int16).numpy()
    al = np.array([orc.alpha(float(orc.amax(x, 1)[0]), "rtn6")], np.float32)
    assert np.array_equal(a2.cpu().numpy().view(np.uint32), al.view(np.uint32))
    refb = orc.quantize_blocks(x, al, ids, "rtn6", "mse")
    assert np.array_equal(yb.view(np.uint16), refb["y"])
    say("[huge] done")
