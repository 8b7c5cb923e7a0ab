"""q4_0_gemv_batch: a list of GEMVs in one launch, against single GEMVs and the
oracle; the full 64-layer decode weight sweep on sampled rows."""
import ctypes

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
    # single calls of these run on the rows kernel; (40, 32768) and (70, 20544) stage x past the fixed stride
    shapes = [(5, 64), (100, 5120), (33, 1088), (1, 17408), (257, 2048), (64, 1024), (31, 17408), (2000, 320),
              (40, 32768), (70, 20544)]
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


def _read_plan(batch):
    """Head, descriptors and chunk schedule of a plan, read back from the device."""
    raw = batch.buffer.cpu().numpy()
    nxt, done, nchunks, grid = np.frombuffer(raw[:16].tobytes(), dtype=np.int32)
    count = batch.plan.count
    desc_t = np.dtype([("w", "<u8"), ("x", "<u8"), ("y", "<u8"), ("n", "<i8"), ("k", "<i4"), ("npl", "<i4"),
                       ("steps", "<i8"), ("cost_begin", "<i8"), ("residual", "<u8"), ("h16", "<i4"),
                       ("reserved", "<i4")])
    chunk_t = np.dtype([("d0", "<i4"), ("s0", "<i4"), ("c_end", "<i8")])
    descs = np.frombuffer(raw[16:16 + count * desc_t.itemsize].tobytes(), dtype=desc_t)
    off = 16 + count * desc_t.itemsize
    chunks = np.frombuffer(raw[off:off + nchunks * chunk_t.itemsize].tobytes(), dtype=chunk_t)
    return int(nxt), int(done), int(nchunks), int(grid), descs, chunks


def test_schedule_partitions_the_row_steps():
    """The plan's chunks cover every row step once, in list order; every chunk
    but the last holds at least two units (pairs-per-lane steps); the counters
    are zero after planning and again after every launch."""
    q4 = lib()
    shapes = [(5, 64), (100, 5120), (33, 1088), (1, 17408), (257, 2048), (64, 1024), (31, 17408), (2000, 320),
              (64, 64), (70, 1024), (1, 64)]
    items = []
    for i, (n, k) in enumerate(shapes):
        items.append((dev_u8(synth.q4_0(SEED, 7000 + i, n, k)), dev_f16(synth.f16_normal(SEED, 7100 + i, k)),
                      torch.empty(n, dtype=torch.float32, device=device())))
    batch = q4.GemvBatch(items)
    nxt, done, nchunks, grid, descs, chunks = _read_plan(batch)
    # the plan holds the list ordered by row-step size, largest first (stable)
    shapes = [shapes[i] for i in sorted(range(len(shapes)), key=lambda i: (-(shapes[i][1] // 64)) // 16)]
    assert [int(d["k"]) for d in descs] == [k for _, k in shapes]
    assert (nxt, done) == (0, 0)
    assert nchunks == batch.plan.nchunks and grid == batch.plan.grid and 1 <= grid <= nchunks
    # the plan's row steps: every descriptor's step count fits one rows-per-step value
    fits = [r for r in range(1, 2049)
            if all(int(d["steps"]) == -(-n // r) for (n, _), d in zip(shapes, descs))]
    assert fits, "no common rows-per-step"
    starts, units = [], []
    cost = 0
    for (n, k), d in zip(shapes, descs):
        npl = -(-(k // 64) // 16)
        assert int(d["npl"]) == npl and int(d["cost_begin"]) == cost
        for st in range(int(d["steps"])):
            starts.append(cost + st * npl)
            units.append(npl)
        cost += int(d["steps"]) * npl
    starts = np.array(starts)
    units = np.array(units)
    begin = [int(descs["cost_begin"][c["d0"]]) + int(c["s0"]) * int(descs["npl"][c["d0"]]) for c in chunks]
    assert begin[0] == 0
    ends = [int(c["c_end"]) for c in chunks]
    assert ends[-1] == cost
    for i in range(nchunks):
        assert begin[i] < ends[i]
        if i + 1 < nchunks:
            assert ends[i] == begin[i + 1]
        assert begin[i] in set(starts.tolist())
        u = int(units[(starts >= begin[i]) & (starts < ends[i])].sum())
        assert u >= 2 or i == nchunks - 1, (i, u)
    for _ in range(3):
        batch()
    torch.cuda.synchronize()
    nxt, done, *_ = _read_plan(batch)
    assert (nxt, done) == (0, 0)
    for (wd, xd, yd) in items:
        assert torch.equal(yd, q4.q4_0_gemv(wd, xd))


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


def test_stage_handoff_in_the_batch():
    """One layer of the sweep shapes as a stage whose last GEMV (the down
    projection) is the hand-off: the other outputs equal the plain batch's bit
    for bit, the hand-off writes binary16(y + residual) of the plain batch's y
    (numpy's float32 add and float16 rounding) and leaves its old y alone; the
    plain GEMV of a second plan is unaffected."""
    q4 = lib()
    seed = synth.DEFAULT_SEED
    shapes = [(n, k) for (_, n, k) in synth.PROJ]
    ws = [dev_u8(synth.q4_0(seed, 11000 + i, n, k)) for i, (n, k) in enumerate(shapes)]
    xs = [dev_f16(synth.f16_normal(seed, 11100 + i, k)) for i, (n, k) in enumerate(shapes)]
    ys_plain = [torch.empty(n, dtype=torch.float32, device="cuda") for n, _ in shapes]
    ys_stage = [torch.empty(n, dtype=torch.float32, device="cuda") for n, _ in shapes]
    last = len(shapes) - 1
    n_last = shapes[last][0]
    r = torch.from_numpy(4.0 * synth.f16_normal(seed, 11200, n_last).astype(np.float32)).cuda()
    h16 = torch.full((n_last,), float("nan"), dtype=torch.float16, device="cuda")
    plain = q4.GemvBatch(list(zip(ws, xs, ys_plain)))
    stage = q4.GemvBatch(list(zip(ws, xs, ys_stage)))
    ys_stage[last].fill_(float("nan"))
    stage.set_handoff(last, h16, r)
    say("stage hand-off: %d GEMVs, hand-off n=%d" % (len(shapes), n_last))
    for _ in range(2):  # a second launch of each: the plans stay as they are
        plain()
        stage()
    torch.cuda.synchronize()
    for i in range(last):
        assert torch.equal(ys_plain[i], ys_stage[i]), i
    assert torch.isnan(ys_stage[last]).all()
    want = (ys_plain[last].cpu().numpy() + r.cpu().numpy()).astype(np.float16)
    assert np.array_equal(h16.cpu().numpy().view(np.uint16), want.view(np.uint16))
    # the same as the single hand-off call
    single = q4.q4_0_gemv_handoff(ws[last], xs[last], r)
    torch.cuda.synchronize()
    assert torch.equal(single.view(torch.int16), h16.view(torch.int16))


def test_batch_handoff_refuses_an_h16_over_the_plan():
    """h16 may not overlap any part of the plan the kernel reads during a
    launch: the head, the descriptors, or the chunk table at the plan's end
    (an h16 lying wholly inside the chunk table is refused).  A refused call
    leaves the plan as it was."""
    q4 = lib()
    shapes = [(5120, 5120), (17408, 5120), (512, 5120)]
    ws = [dev_u8(synth.q4_0(SEED, 11300 + i, n, k)) for i, (n, k) in enumerate(shapes)]
    xs = [dev_f16(synth.f16_normal(SEED, 11400 + i, k)) for i, (n, k) in enumerate(shapes)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for n, _ in shapes]
    batch = q4.GemvBatch(list(zip(ws, xs, ys)))
    batch()
    torch.cuda.synchronize()
    want = [y.clone() for y in ys]
    lb = q4.load_library()
    base, nbytes = batch.buffer.data_ptr(), batch.buffer.numel()
    n_last = shapes[-1][0]
    chunk_table = nbytes - 16 * batch.plan.nchunks
    assert chunk_table > 0 and 16 * batch.plan.nchunks >= 2 * n_last + 16
    for off in (0, 16, chunk_table, chunk_table + 16, nbytes - 2 * n_last):
        st = lb.q4_0_gemv_batch_handoff(ctypes.byref(batch.plan), ys[-1].data_ptr(), None, base + off, None)
        assert st == q4.Q4_ERR_INVALID_ARG, (off, st)
    # the plan is intact
    for y in ys:
        y.fill_(float("nan"))
    batch()
    torch.cuda.synchronize()
    for a, b in zip(ys, want):
        assert torch.equal(a, b)


def test_widest_k_runs_on_eight_wave_workgroups():
    """k above 24,576 stages more activations than leave room for 12 waves'
    rings: a quad-engine list (k % 1024 == 0) and a wide single call run with
    8-wave workgroups.  Every output equals the single call's (rows kernel for
    the slices) bit for bit and lies within the bound on sampled rows."""
    q4 = lib()
    shapes = [(300, 32768), (100, 28672), (2, 25600)]
    items, host = [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.q4_0(SEED, 7600 + i, n, k)
        x = synth.f16_normal(SEED, 7700 + i, k)
        host.append((w, x))
        items.append((dev_u8(w), dev_f16(x), torch.full((n,), float("nan"), device=device())))
    batch = q4.GemvBatch(items)
    assert batch.plan.flags == 3  # quad engine, 8-wave workgroups
    batch()
    torch.cuda.synchronize()
    for (w, x), (wd, xd, yd), (n, k) in zip(host, items, shapes):
        assert torch.equal(yd, q4.q4_0_gemv(wd, xd)), (n, k)
        y_ref, a_ref = oracle.gemm_rows(w, k, x)
        assert_parity(yd.cpu().numpy(), y_ref, a_ref, "8-wave list %dx%d" % (n, k))
    # a single call wide enough for the wide shape: 40,000 rows x 32,768 (737 MB)
    n, k = 40000, 32768
    w = synth.q4_0(SEED, 7800, n, k)
    x = synth.f16_normal(SEED, 7801, k)
    wd, xd = dev_u8(w), dev_f16(x)
    say("wide single 40000 x 32768")
    y = q4.q4_0_gemv(wd, xd)
    for lo, hi in [(0, 64), (39936, 40000), (20011, 20100)]:
        assert torch.equal(y[lo:hi], q4.q4_0_gemv(wd[lo:hi], xd)), (lo, hi)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(3).integers(0, n, 254)]))
    y_ref, a_ref = oracle.gemm_rows(np.ascontiguousarray(w[rows]), k, x)
    assert_parity(y[rows].cpu().numpy(), y_ref, a_ref, "wide single k = 32768")
