"""q4_0_gemm_smallm (M <= 16): against the oracle, and row m against the M=1
GEMV of X[m] (the batched verify pass agrees with plain decode).  M <= 7 runs
the LDS-ring engine, larger M the register-load one; both are covered, each
with a K split into ranges (M = 4, 7, 16 at K = 17,408)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED

SHAPES = [(1, 64), (37, 128), (100, 5120), (64, 1088), (31, 17408), (7, 96), (513, 2048), (50, 32768)]


@pytest.mark.parametrize("m", [1, 2, 3, 4, 7, 8, 16])
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


@pytest.mark.parametrize("m", [4, 16])
def test_layer_shapes_sampled(m):
    """M = 4 (LDS ring) and 16 (register loads) against one full layer of the
    sweep shapes (q, gate, down)."""
    q4 = lib()
    rng = np.random.default_rng(9)
    for proj in (0, 4, 6):
        _, n, k = synth.PROJ[proj]
        sw = synth.stream_id(3, 0, proj, synth.T_W)
        w = synth.q4_0(SEED, sw, n, k)
        x = synth.f16_normal(SEED, synth.stream_id(3, 0, proj, synth.T_X), m * k).reshape(m, k)
        say("smallm layer shape", n, k)
        y = q4.q4_0_gemm_smallm(dev_u8(w), dev_f16(x))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 30)]))
        y_ref, a_ref = oracle.gemm_rows(w[rows], k, x)
        assert_parity(y.cpu().numpy()[:, rows], y_ref, a_ref)


@pytest.mark.parametrize("m", [2, 5, 7, 16])
def test_batch_matches_single_calls_and_oracle(m):
    """A mixed small-M list in one launch: every GEMM bit-identical to its own
    q4_0_gemm_smallm call and within the bound of the oracle, including GEMMs
    whose K is split into ranges (m = 16, k = 17408 and 9216), ragged row tiles
    and a ragged last segment (k = 1088)."""
    q4 = lib()
    shapes = [(100, 5120), (31, 17408), (513, 2048), (64, 1088), (1, 64), (257, 4096), (40, 9216)]
    host, items = [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.q4_0(SEED, 9100 + i, n, k)
        x = synth.f16_normal(SEED, 9200 + 17 * i + m, m * k).reshape(m, k)
        host.append((w, x))
        items.append((dev_u8(w), dev_f16(x), torch.full((m, n), float("nan"), device="cuda")))
    say("smallm batch m=%d of %d GEMMs" % (m, len(items)))
    batch = q4.SmallMBatch(items)
    batch()
    torch.cuda.synchronize()
    for (w, x), (wd, xd, yd), (n, k) in zip(host, items, shapes):
        single = q4.q4_0_gemm_smallm(wd, xd).cpu().numpy()
        y = yd.cpu().numpy()
        assert np.array_equal(y, single), (m, n, k)
        y_ref, a_ref = oracle.gemm_rows(w, k, x)
        assert_parity(y, y_ref, a_ref, "smallm batch m=%d %dx%d" % (m, n, k))
    before = [it[2].clone() for it in items]
    batch()
    torch.cuda.synchronize()
    for b, it in zip(before, items):
        assert torch.equal(b, it[2])


def test_batch_graph_replay():
    """The small-M batch captured in a HIP graph: every replay, with eager work
    between them, equals the eager result."""
    q4 = lib()
    m = 16
    shapes = [(300, 5120), (70, 17408), (129, 1024)]
    items = []
    for i, (n, k) in enumerate(shapes):
        items.append((dev_u8(synth.q4_0(SEED, 9300 + i, n, k)),
                      dev_f16(synth.f16_normal(SEED, 9400 + i, m * k).reshape(m, k)),
                      torch.empty((m, n), dtype=torch.float32, device="cuda")))
    batch = q4.SmallMBatch(items)
    batch()
    torch.cuda.synchronize()
    ref = [it[2].clone() for it in items]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        batch(stream)  # warm up on the capture stream
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            batch(stream)
    for rep in range(3):
        for it in items:
            it[2].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for r, it in zip(ref, items):
            assert torch.equal(r, it[2]), rep
