"""q4_0_gemm_smallm (M <= 16): against the oracle, and row m against the M=1
GEMV of X[m] (the batched verify pass agrees with plain decode)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED

SHAPES = [(1, 64), (37, 128), (100, 5120), (64, 1088), (31, 17408), (7, 96), (513, 2048)]


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("n,k", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_parity(m, n, k):
    q4 = lib()
    w = synth.q4_0(SEED, 7000 + n + k, n, k)
    x = synth.f16_normal(SEED, 8000 + n + k + m, m * k).reshape(m, k)
    wd, xd = dev_u8(w), dev_f16(x)
    y = q4.q4_0_gemm_smallm(wd, xd)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    assert_parity(y, y_ref, a_ref, "smallm m=%d %dx%d" % (m, n, k))
    for i in range(m):
        yi = q4.q4_0_gemv(wd, xd[i].contiguous()).cpu().numpy()
        assert_parity(yi, y_ref[i], a_ref[i])


def test_layer_shapes_sampled():
    """M = 16 against one full layer of the sweep shapes (q, gate, down)."""
    q4 = lib()
    rng = np.random.default_rng(9)
    for proj in (0, 4, 6):
        _, n, k = synth.PROJ[proj]
        sw = synth.stream_id(3, 0, proj, synth.T_W)
        w = synth.q4_0(SEED, sw, n, k)
        x = synth.f16_normal(SEED, synth.stream_id(3, 0, proj, synth.T_X), 16 * k).reshape(16, k)
        say("smallm layer shape", n, k)
        y = q4.q4_0_gemm_smallm(dev_u8(w), dev_f16(x))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 30)]))
        y_ref, a_ref = oracle.gemm_rows(w[rows], k, x)
        assert_parity(y.cpu().numpy()[:, rows], y_ref, a_ref)
