"""q8_0_gemv: the Q8_0 GEMV against the oracle, element by element within the
bound, over shapes that cover odd block counts per row (rows that start 2 bytes
into a dword), a single block, the largest K, ragged row counts, the matrix's
last block on a dword boundary, and the Qwen3-4B-shaped projections."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def run(w_np, x_np):
    q4 = lib()
    y = q4.q8_0_gemv(dev_u8(w_np), dev_f16(x_np))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("n,k", [(1, 32), (7, 32), (65, 96), (300, 160), (1000, 1024), (513, 2080),
                                 (4096, 2560), (2560, 9728), (200, 32768), (9728, 2560)])
def test_q8_parity(n, k):
    w = synth.q8_0(SEED, 9300 + k % 1000, n, k)
    x = synth.f16_normal(SEED, 9400 + n % 1000, k)
    y = run(w, x)
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    r = assert_parity(y, y_ref, a_ref, "q8 n=%d k=%d" % (n, k))
    say("q8 n=%d k=%d max err/a %.3g" % (n, k, r))


def test_q8_last_block_ends_the_allocation():
    """The matrix copied to the end of a larger buffer's exact length: the last
    block starts on a dword, so its 36-byte window would pass the end."""
    n, k = 33, 96  # 99 blocks: the last one starts at 98 * 34, a multiple of 4
    w = synth.q8_0(SEED, 9501, n, k)
    assert ((n * (k // 32) - 1) * 34) % 4 == 0
    x = synth.f16_normal(SEED, 9502, k)
    buf = torch.empty(w.size, dtype=torch.uint8, device="cuda")
    buf.copy_(torch.from_numpy(w.ravel()))
    q4 = lib()
    y = q4.q8_0_gemv(buf.view(n, -1), dev_f16(x))
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    assert_parity(y.cpu().numpy(), y_ref, a_ref, "q8 tail")


def test_q8_rows_are_position_independent():
    """A row's output does not depend on where it sits: the same rows shuffled give the same bits."""
    n, k = 777, 2560
    w = synth.q8_0(SEED, 9601, n, k)
    x = synth.f16_normal(SEED, 9602, k)
    perm = np.random.default_rng(5).permutation(n)
    y1 = run(w, x)
    y2 = run(np.ascontiguousarray(w[perm]), x)
    assert np.array_equal(y1[perm], y2)


def test_q8_extreme_codes_and_scales():
    """Every code -128 or +127 with large scales: the f16 decode of the codes stays exact."""
    n, k = 64, 512
    rng = np.random.default_rng(7)
    codes = rng.choice([-128, 127], size=(n, k))
    d = rng.choice([-8.0, 4.0, 0.5], size=(n, k // 32)).astype(np.float16)
    import q4_encode
    w = q4_encode.encode_q8(codes, d.view(np.uint16))
    x = synth.f16_normal(SEED, 9701, k)
    y = run(w, x)
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    assert_parity(y, y_ref, a_ref, "q8 extremes")


def test_q8_graph_replay_matches_eager():
    """Three Q8_0 GEMVs captured in a HIP graph: every replay (with eager work
    and synchronisations between them) gives the eager bits."""
    q4 = lib()
    shapes = [(1024, 2560), (2560, 4096), (333, 96)]
    ws = [dev_u8(synth.q8_0(SEED, 9800 + i, n, k)) for i, (n, k) in enumerate(shapes)]
    xs = [dev_f16(synth.f16_normal(SEED, 9900 + i, k)) for i, (n, k) in enumerate(shapes)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for n, _ in shapes]
    eager = [q4.q8_0_gemv(w, x).clone() for w, x in zip(ws, xs)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for w, x, y in zip(ws, xs, ys):
            q4.q8_0_gemv(w, x, y)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w, x, y in zip(ws, xs, ys):
            q4.q8_0_gemv(w, x, y)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y, e), rep
        q4.q8_0_gemv(ws[0], xs[1][:2560].contiguous())  # eager work between replays
        torch.cuda.synchronize()


def _batch_items(shapes, base):
    ws = [synth.q8_0(SEED, base + i, n, k) for i, (n, k) in enumerate(shapes)]
    xs = [synth.f16_normal(SEED, base + 500 + i, k) for i, (n, k) in enumerate(shapes)]
    items = [(dev_u8(w), dev_f16(x), torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"))
             for w, x, (n, k) in zip(ws, xs, shapes)]
    return ws, xs, items


def test_q8_batch_equals_single_calls():
    """A mixed list in one launch: every row bit-equal to q8_0_gemv's, every row within the bound."""
    q4 = lib()
    shapes = [(1, 32), (15, 96), (16, 160), (17, 2080), (300, 2560), (1024, 2560), (33, 32768), (2560, 9728),
              (5, 64), (4096, 2560), (3, 2048), (1, 4096), (9, 28672)]
    ws, xs, items = _batch_items(shapes, 10100)
    batch = q4.Q8Batch(items)
    # on the slab engine: (300, 2560), (1024, 2560), (2560, 9728), (4096, 2560), and the groups of
    # fewer than 8 rows (3, 2048), (1, 4096) and (9, 28672)
    assert batch.plan.n_slab == 7
    batch()
    torch.cuda.synchronize()
    for i, ((w_d, x_d, y), w, x, (n, k)) in enumerate(zip(items, ws, xs, shapes)):
        single = q4.q8_0_gemv(w_d, x_d)
        torch.cuda.synchronize()
        assert torch.equal(y, single), (i, n, k)
        y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
        assert_parity(y.cpu().numpy(), y_ref, a_ref, "q8 batch %d" % i)


def test_q8_batch_model_layers():
    """Two layers of the Qwen3-4B-shaped projections (14 GEMVs) as one launch, against the oracle."""
    q4 = lib()
    shapes = [(n, k) for _ in range(2) for (_, n, k) in synth.Q8_PROJ]
    ws, xs, items = _batch_items(shapes, 10300)
    batch = q4.Q8Batch(items)
    say("q8 batch grid %d over %d GEMVs" % (batch.plan.grid, len(items)))
    batch()
    torch.cuda.synchronize()
    for i, ((_, _, y), w, x, (n, k)) in enumerate(zip(items, ws, xs, shapes)):
        y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
        assert_parity(y.cpu().numpy(), y_ref, a_ref, "q8 layers %d" % i)


def test_q8_batch_graph_replay():
    """The batch launch captured in a HIP graph: every replay gives the eager bits."""
    q4 = lib()
    shapes = [(1024, 2560), (2560, 4096), (97, 1056)]
    _, _, items = _batch_items(shapes, 10500)
    batch = q4.Q8Batch(items)
    batch()
    torch.cuda.synchronize()
    eager = [y.clone() for _, _, y in items]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        batch()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        batch()
    for rep in range(3):
        for _, _, y in items:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for (_, _, y), e in zip(items, eager):
            assert torch.equal(y, e), rep
        batch()  # eager work between replays
        torch.cuda.synchronize()


def test_q8_vocabulary_sized_rows_sampled():
    """151,936 rows x 2,560 (a Q8_0 LM head of the small dense model's width):
    sampled rows, the first and the last included, against the oracle."""
    n, k = synth.VOCAB, 2560
    q4 = lib()
    w = synth.q8_0(SEED, 10701, n, k)
    x = synth.f16_normal(SEED, 10702, k)
    y = q4.q8_0_gemv(dev_u8(w), dev_f16(x))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], np.random.default_rng(11).integers(0, n, 3000)]))
    y_ref, a_ref = oracle.q8_gemm_rows(np.ascontiguousarray(w[rows]), k, x)
    assert_parity(y[rows], y_ref, a_ref, "q8 vocabulary rows")


# Shapes of the slab kernel (k % 512 == 0, 2048 <= k <= 28672, w 16-byte
# aligned): fewer rows than one 8-row group, ragged row counts, slabs that
# hold pairs of three rows (k = 2048: 32 pairs per row), rows that span many
# slabs, the largest k; and the first k above it, which takes the per-block
# kernel.  Single calls with fewer than 32,768 rows run on the rows kernel
# (the slab engine's association), larger ones (50000 x 2048) on the slab engine.
SLAB_SHAPES = [(1, 2048), (7, 2048), (9, 3072), (95, 2560), (97, 4096), (1000, 2048), (333, 9728),
               (100, 28672), (50000, 2048), (64, 29184)]


@pytest.mark.parametrize("n,k", SLAB_SHAPES, ids=["%dx%d" % s for s in SLAB_SHAPES])
def test_q8_slab_shapes(n, k):
    w = synth.q8_0(SEED, 11000 + k % 997, n, k)
    x = synth.f16_normal(SEED, 11100 + n % 997, k)
    say("q8 slab n=%d k=%d" % (n, k))
    y = run(w, x)
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    r = assert_parity(y, y_ref, a_ref, "q8 slab n=%d k=%d" % (n, k))
    say("q8 slab n=%d k=%d max err/a %.3g" % (n, k, r))


def test_q8_slab_rows_position_independent_long_rows():
    """Rows of 152 pairs (k = 9728) span two or three slabs and start at every
    multiple of 8 lanes: a shuffle of the rows gives the same bits."""
    n, k = 515, 9728
    w = synth.q8_0(SEED, 11201, n, k)
    x = synth.f16_normal(SEED, 11202, k)
    perm = np.random.default_rng(9).permutation(n)
    y1 = run(w, x)
    y2 = run(np.ascontiguousarray(w[perm]), x)
    assert np.array_equal(y1[perm], y2)


def test_q8_rows_kernel_equals_slab_engine():
    """The same rows through the slab engine (a 49,200-row single call) and
    through the rows kernel (single calls on slices of it): equal bits."""
    n, k = 49200, 2560
    q4 = lib()
    w = synth.q8_0(SEED, 11401, n, k)
    x = dev_f16(synth.f16_normal(SEED, 11402, k))
    wd = dev_u8(w)
    y = q4.q8_0_gemv(wd, x)
    for lo, hi in [(0, 1000), (48001, 49200), (20000, 20037)]:
        ys = q4.q8_0_gemv(wd[lo:hi], x)
        torch.cuda.synchronize()
        assert torch.equal(y[lo:hi], ys), (lo, hi)
    y_ref, a_ref = oracle.q8_gemm_rows(np.ascontiguousarray(w[:2000]), k, x.cpu().numpy())
    assert_parity(y[:2000].cpu().numpy(), y_ref, a_ref, "q8 slab engine rows")


def test_q8_misaligned_weights_take_the_block_kernel():
    """w 4- but not 16-byte aligned at a slab shape: the per-block kernel runs,
    within the bound, and a list holding the same descriptor gives its bits."""
    n, k = 300, 2560
    w = synth.q8_0(SEED, 11301, n, k)
    x = synth.f16_normal(SEED, 11302, k)
    buf = torch.empty(w.size + 4, dtype=torch.uint8, device="cuda")
    wd = buf[4:].view(n, -1)
    wd.copy_(torch.from_numpy(w))
    assert wd.data_ptr() % 16 == 4
    q4 = lib()
    xd = dev_f16(x)
    y = q4.q8_0_gemv(wd, xd)
    yb = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    batch = q4.Q8Batch([(wd, xd, yb)])
    assert batch.plan.n_slab == 0
    batch()
    torch.cuda.synchronize()
    assert torch.equal(y, yb)
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    assert_parity(y.cpu().numpy(), y_ref, a_ref, "q8 misaligned")


@pytest.mark.parametrize("n,k", [(1, 32768), (1, 32), (2, 33 * 32)])
def test_q8_single_rows(n, k):
    """One or two rows: the largest K, a single block, an odd block count."""
    w = synth.q8_0(SEED, 10800 + n, n, k)
    x = synth.f16_normal(SEED, 10801, k)
    y = run(w, x)
    y_ref, a_ref = oracle.q8_gemm_rows(w, k, x)
    assert_parity(y, y_ref, a_ref, "q8 n=%d k=%d" % (n, k))
