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


@pytest.mark.parametrize("m", [37, 169])
def test_batch_parity_and_single_calls(m):
    """A mixed prefill list in one launch: every GEMM within the bound of the
    oracle and equal to its own q4_0_gemm_prefill call, with ragged M, N
    (rows past a tile) and K (1088: 17 pairs)."""
    q4 = lib()
    shapes = [(300, 1024), (64, 2048), (257, 1088), (31, 4096), (512, 64)]
    host, items = [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.q4_0(SEED, 9600 + i, n, k)
        x = synth.f16_normal(SEED, 9700 + 13 * i + m, m * k).reshape(m, k)
        host.append((w, x))
        items.append((dev_u8(w), dev_f16(x), torch.full((m, n), float("nan"), device="cuda")))
    say("prefill batch m=%d of %d GEMMs" % (m, len(items)))
    batch = q4.PrefillBatch(items)
    batch()
    torch.cuda.synchronize()
    for (w, x), (wd, xd, yd), (n, k) in zip(host, items, shapes):
        y = yd.cpu().numpy()
        y_ref, a_ref = oracle.gemm_rows(w, k, x)
        assert_parity(y, y_ref, a_ref, "prefill batch m=%d %dx%d" % (m, n, k))
        single = q4.q4_0_gemm_prefill(wd, xd).cpu().numpy()
        assert_parity(single, y_ref, a_ref)
        assert np.array_equal(y, single), (m, n, k)
    before = [it[2].clone() for it in items]
    batch()
    torch.cuda.synchronize()
    for b, it in zip(before, items):
        assert torch.equal(b, it[2])


def test_batch_layer_sampled():
    """One layer's seven projections at M = 169 as one batch, sampled rows
    against the oracle."""
    q4 = lib()
    m = 169
    rng = np.random.default_rng(1690)
    items, checks = [], []
    for proj in range(7):
        _, n, k = synth.PROJ[proj]
        sw = synth.stream_id(4, 1, proj, synth.T_W)
        x = synth.f16_normal(SEED, synth.stream_id(4, 1000 + m, proj, synth.T_X), m * k).reshape(m, k)
        w = synth.q4_0(SEED, sw, n, k)
        items.append((dev_u8(w), dev_f16(x), torch.empty((m, n), dtype=torch.float32, device="cuda")))
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 6)]))
        checks.append((w[rows], x, k, rows))
        del w
    batch = q4.PrefillBatch(items)
    batch()
    torch.cuda.synchronize()
    for (wr, x, k, rows), it in zip(checks, items):
        y_ref, a_ref = oracle.gemm_rows(wr, k, x)
        assert_parity(it[2].cpu().numpy()[:, rows], y_ref, a_ref, "prefill layer batch")
