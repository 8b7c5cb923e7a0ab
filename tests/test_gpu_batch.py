"""q4_0_gemv_batch: a list of GEMVs in one launch, against single GEMVs and the
oracle; the full 64-layer decode weight sweep on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, device, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def test_mixed_list_matches_single_gemv_and_oracle():
    q4 = lib()
    shapes = [(5, 64), (100, 5120), (33, 1088), (1, 17408), (257, 2048), (64, 1024), (31, 17408), (2000, 320)]
    items, host = [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.q4_0(SEED, 5000 + i, n, k)
        x = synth.f16_normal(SEED, 6000 + i, k)
        host.append((w, x))
        items.append((dev_u8(w), dev_f16(x), torch.full((n,), float("nan"), device=device())))
    say("batch of", len(items))
    batch = q4.GemvBatch(items)
    batch()
    torch.cuda.synchronize()
    for (w, x), (wd, xd, yd), (n, k) in zip(host, items, shapes):
        y = yd.cpu().numpy()
        single = q4.q4_0_gemv(wd, xd).cpu().numpy()
        assert np.array_equal(y, single), (n, k)
        y_ref, a_ref = oracle.gemm_rows(w, k, x)
        assert_parity(y, y_ref, a_ref, "batch %dx%d" % (n, k))
    # a second run gives identical results
    before = [it[2].clone() for it in items]
    batch()
    torch.cuda.synchronize()
    for b, it in zip(before, items):
        assert torch.equal(b, it[2])


def test_full_decode_sweep_sampled():
    """All 448 GEMVs of the 64-layer sweep (13.4 GB of weights) in one launch;
    every GEMV checked on 6 sampled rows against the oracle."""
    q4 = lib()
    rng = np.random.default_rng(2024)
    items, checks = [], []
    say("generating the 64-layer sweep")
    for (layer, proj, n, k) in synth.decode_sweep():
        sw = synth.stream_id(1, layer, proj, synth.T_W)
        sx = synth.stream_id(1, layer, proj, synth.T_X)
        w = synth.q4_0(SEED, sw, n, k)
        x = synth.f16_normal(SEED, sx, k)
        items.append((dev_u8(w), dev_f16(x), torch.empty(n, dtype=torch.float32, device=device())))
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 4)]))
        checks.append((sw, x, k, rows))
        del w
    say("running the sweep")
    batch = q4.GemvBatch(items)
    batch()
    torch.cuda.synchronize()
    worst = 0.0
    for (sw, x, k, rows), (_, _, yd) in zip(checks, items):
        y = yd.cpu().numpy()[rows]
        w_rows = synth.q4_0_row_list(SEED, sw, k, rows)
        y_ref, a_ref = oracle.gemm_rows(w_rows, k, x)
        worst = max(worst, assert_parity(y, y_ref, a_ref, "sweep stream %d" % sw))
    say("sweep worst err/a", worst)
