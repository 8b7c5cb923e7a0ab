"""q4_0_gemm_prefill: against the oracle on full small shapes and on sampled
rows of the prompt sizes 169 and 512."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED

CASES = [(1, 64, 64), (17, 100, 1024), (33, 257, 2048), (64, 128, 5120), (5, 31, 96), (169, 200, 1088)]


@pytest.mark.parametrize("m,n,k", CASES, ids=["%dx%dx%d" % c for c in CASES])
def test_parity(m, n, k):
    q4 = lib()
    w = synth.q4_0(SEED, 9000 + n + k, n, k)
    x = synth.f16_normal(SEED, 9500 + m + k, m * k).reshape(m, k)
    y = q4.q4_0_gemm_prefill(dev_u8(w), dev_f16(x))
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    assert_parity(y.cpu().numpy(), y_ref, a_ref, "prefill %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m", [169, 512])
def test_prompt_sizes_sampled(m):
    q4 = lib()
    rng = np.random.default_rng(m)
    for proj in (0, 4, 6):
        _, n, k = synth.PROJ[proj]
        sw = synth.stream_id(4, 0, proj, synth.T_W)
        w = synth.q4_0(SEED, sw, n, k)
        x = synth.f16_normal(SEED, synth.stream_id(4, m, proj, synth.T_X), m * k).reshape(m, k)
        say("prefill", m, n, k)
        y = q4.q4_0_gemm_prefill(dev_u8(w), dev_f16(x))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 14)]))
        y_ref, a_ref = oracle.gemm_rows(w[rows], k, x)
        assert_parity(y.cpu().numpy()[:, rows], y_ref, a_ref, "prefill m=%d %dx%d" % (m, n, k))
