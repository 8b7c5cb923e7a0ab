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

CASES = [(1, 64, 64), (17, 100, 1024), (33, 257, 2048), (64, 128, 5120), (5, 31, 96), (169, 200, 1088),
         (37, 100, 32768), (70, 90, 20544)]  # the largest k on both kernels (k % 256 == 0 and not)


@pytest.mark.parametrize("m,n,k", CASES, ids=["%dx%dx%d" % c for c in CASES])
def test_parity(m, n, k):
    q4 = lib()
    w = synth.q4_0(SEED, 9000 + n + k, n, k)
    x = synth.f16_normal(SEED, 9500 + m + k, m * k).reshape(m, k)
    y = q4.q4_0_gemm_prefill(dev_u8(w), dev_f16(x))
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    assert_parity(y.cpu().numpy(), y_ref, a_ref, "prefill %dx%dx%d" % (m, n, k))


def sampled_rows(rng, n, count=1024):
    """`count` distinct rows of n (all of them when n <= count), first and last included."""
    if n <= count:
        return np.arange(n)
    inner = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, n - 1], inner]))


@pytest.mark.parametrize("m", [169, 512])
def test_prompt_sizes_sampled(m):
    """Single q4_0_gemm_prefill calls at the prompt sizes on three projection
    shapes, 1,024 sampled output rows each (first and last included), every
    one of the m activation rows."""
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
        rows = sampled_rows(rng, n)
        assert len(rows) == min(n, 1024) and rows[0] == 0 and rows[-1] == n - 1
        y_ref, a_ref = oracle.gemm_rows(w[rows], k, x)
        assert_parity(y.cpu().numpy()[:, rows], y_ref, a_ref, "prefill m=%d %dx%d" % (m, n, k))


TILE_M = {37: 64, 96: 96, 100: 128, 169: 96, 512: 128}


@pytest.mark.parametrize("m", [37, 96, 100, 169, 512])
def test_batch_parity_and_single_calls(m):
    """A mixed prefill list in one launch: every GEMM within the bound of the
    oracle and equal to its own q4_0_gemm_prefill call, with ragged M, N
    (rows past a tile) and K (1088: 17 pairs).  M = 37 runs on 64-row tiles,
    M = 96 and 169 (ragged) on 96-row tiles (the k % 256 != 0 GEMMs on 64-row
    ones), M = 100 (ragged) and 512 on 128-row tiles, on both batch kernels
    (k % 256 == 0 and the others)."""
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
    assert batch.plan.tile_m == TILE_M[m], batch.plan.tile_m
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


@pytest.mark.parametrize("m", [169, 512])
def test_batch_full_layers(m):
    """Layers 0 and 63 of the prefill workload the benchmark times (the
    sweep's weights, the prefill activations, the same batch kernel and tile
    shape: 96-row tiles at M = 169, 128-row tiles at M = 512) as one batch of
    14 GEMMs: every output of every GEMM against the oracle, and each GEMM bit
    for bit equal to its own q4_0_gemm_prefill call."""
    q4 = lib()
    items, host = [], []
    for layer in (0, 63):
        for proj in range(7):
            _, n, k = synth.PROJ[proj]
            w = synth.q4_0(SEED, synth.stream_id(1, layer, proj, synth.T_W), n, k)
            x = synth.f16_normal(SEED, synth.stream_id(4, layer, proj, synth.T_X), m * k).reshape(m, k)
            items.append((dev_u8(w), dev_f16(x), torch.full((m, n), float("nan"), device="cuda")))
            host.append((layer, proj, w, x))
    batch = q4.PrefillBatch(items)
    assert batch.plan.tile_m == TILE_M[m]
    say("prefill full layers 0 and 63, m=%d, tile_m=%d" % (m, batch.plan.tile_m))
    batch()
    torch.cuda.synchronize()
    worst = 0.0
    for (layer, proj, w, x), (wd, xd, yd) in zip(host, items):
        _, n, k = synth.PROJ[proj]
        y = yd.cpu().numpy()
        single = q4.q4_0_gemm_prefill(wd, xd).cpu().numpy()
        assert np.array_equal(y, single), (m, layer, proj)
        y_ref, a_ref = oracle.gemm_rows(w, k, x)
        worst = max(worst, assert_parity(y, y_ref, a_ref, "prefill m=%d layer %d proj %d" % (m, layer, proj)))
    say("prefill full layers m=%d: worst err/a %.3g" % (m, worst))


@pytest.mark.parametrize("k", [1024, 1088])
def test_single_call_96_row_tiles(k):
    """A single q4_0_gemm_prefill call wide enough to run 96-row tiles (M =
    169, N = 33,000: 258 tiles of 96 x 256, more than the CUs), on both
    kernels (k % 256 == 0 and not): 1,024 sampled rows against the oracle,
    and bit-equal to the same GEMM in a batch (whose k % 256 != 0 part runs
    64-row tiles: the tile shape does not change any output's summation
    order)."""
    q4 = lib()
    m, n = 169, 33000
    w = synth.q4_0(SEED, 9900 + k, n, k)
    x = synth.f16_normal(SEED, 9950 + k, m * k).reshape(m, k)
    wd, xd = dev_u8(w), dev_f16(x)
    say("prefill single 96-row tiles", m, n, k)
    y = q4.q4_0_gemm_prefill(wd, xd)
    yb = torch.full((m, n), float("nan"), device="cuda")
    batch = q4.PrefillBatch([(wd, xd, yb)])
    assert batch.plan.tile_m == 96
    batch()
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.array_equal(y, yb.cpu().numpy())
    rows = sampled_rows(np.random.default_rng(k), n)
    y_ref, a_ref = oracle.gemm_rows(w[rows], k, x)
    assert_parity(y[:, rows], y_ref, a_ref, "prefill 96-row single m=%d n=%d k=%d" % (m, n, k))
