"""Benchmark of the Q4_0 dequantize-and-multiply path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload sweep|gemv|lmhead|lmhead_norm|handoff|q8|verify|smallm|prefill|copy|stream]
                    [--m M] [--pattern P --wg-per-cu W]

Default workload ("sweep"): the 27B-shaped decode weight sweep, 64 layers x
(q, k, v, o 5120x5120; gate, up 17408x5120; down 5120x17408) = 448 Q4_0 GEMVs
and 13,400,801,280 bytes of packed weights, each GEMV with its own f16 input
(synthetic, seeded).  One step = one sweep = one launch of the batch kernel
(q4_0_gemv_batch).  Inputs are resident in HBM before timing starts; K steps
are bracketed by HIP events on the launch stream.

Prints ONE JSON line: metric/value/unit (algorithmic GB/s of the sweep), the
roofline of the dominant kernel and a CPU baseline (the binary64 oracle timed
on a bounded sample of the same workload on this host's cores).

Other workloads print the same kind of line for the single 5120x5120 GEMV
(rotating weight copies so the 256 MB last-level cache does not serve them),
the LM head with argmax (with the final norm fused: lmhead_norm), the stage
hand-off (a 22-layer range ending in the binary16 hidden state: handoff), the Q8_0 GEMV over a
small dense model's layers (q8), the greedy
verify of an M-row draft, small-M (--m) and prefill (--m) over the sweep.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_0 GEMV HBM GB/s (% of 8 TB/s) and 27B-shape decode weight-sweeps/sec"
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Kernel source of each workload's dominant kernel (besides the shared device
# and launch headers, the host-side C ABI and the build script).
KERNEL_SOURCE = {"sweep": ["gemv.hip"], "gemv": ["gemv.hip"], "lmhead": ["gemv.hip"], "lmhead_norm": ["gemv.hip"],
                 "handoff": ["gemv.hip"], "q8": ["gemv.hip", "q8.hip"],
                 "smallm": ["smallm.hip"],
                 "prefill": ["prefill.hip"], "verify": ["smallm.hip", "gemv.hip", "verify.hip"]}


def kernel_source_hash(workload: str) -> str:
    """Hash of the sources that build `workload`'s kernel and of the build
    flags, comments and blank space left out (so an edited comment, or a
    change to another workload's kernel, does not invalidate a measurement)."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "q4_dequant_gemv_block_amd", "csrc")
    names = KERNEL_SOURCE[workload.split("_m")[0]] + ["q4_device.h", "q4_launch.h", "api.cpp"]
    files = [os.path.join(csrc, n) for n in sorted(names)]
    files.append(os.path.join(ROOT, "q4_dequant_gemv_block_amd", "build.py"))
    for path in files:
        with open(path) as f:
            text = f.read()
        if not path.endswith(".py"):
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(os.path.basename(path).encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from committed
    rocprofv3 counter runs (profiles/traffic.json), or None when there are none
    or the kernel sources changed since they were taken."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    e = table.get(workload)
    if not e or e.get("source_hash") != kernel_source_hash(workload):
        return None
    return e.get("bytes_per_launch")


def load_q4():
    import q4_dequant_gemv_block_amd as q4
    if not os.path.exists(q4.LIB_PATH):
        from q4_dequant_gemv_block_amd import build
        build.build()
    q4.load_library()
    return q4


def cpu_cores() -> int:
    """Threads the oracle runs with: OMP_NUM_THREADS when set, else the CPUs
    this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(items, budget_s: float):
    """Run the oracle over the sweep's GEMVs in order until about budget_s of
    wall time; returns (algorithmic bytes, GEMVs, seconds)."""
    import oracle
    import synth
    done_bytes, done, t_total = 0, 0, 0.0
    for (sw, sx, n, k) in items:
        w = synth.q4_0(SEED, sw, n, k)
        x = synth.f16_normal(SEED, sx, k)
        t0 = time.perf_counter()
        oracle.gemm_rows(w, k, x)
        t_total += time.perf_counter() - t0
        done_bytes += w.nbytes + k * 2 + n * 4
        done += 1
        if t_total >= budget_s:
            break
    return done_bytes, done, t_total


def cpu_baseline(items, budget_s: float = 12.0, one_core_s: float = 4.0) -> dict:
    """Time the oracle over the sweep's GEMVs in order until about budget_s of
    CPU work with the thread count set explicitly (cpu_cores), then about
    one_core_s on one thread; report algorithmic GB/s (and the sweeps/s it
    implies)."""
    import oracle
    o = oracle.default()
    threads = o.set_threads(cpu_cores())
    done_bytes, done, t_total = _oracle_rate(items, budget_s)
    o.set_threads(1)
    b1, d1, t1 = _oracle_rate(items, one_core_s)
    o.set_threads(threads)
    gbs = done_bytes / t_total / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of the sweep's GEMVs (%.2f GB of weights), binary64, %.1f s, %d threads" % (
                done, done_bytes / 1e9, t_total, threads),
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "one_core_gbps": round(b1 / t1 / 1e9, 4), "one_core_sample": "first %d GEMVs, %.1f s" % (d1, t1),
            "sweeps_per_s": round(gbs * 1e9 / SWEEP_BYTES, 6)}


SEED = 0x51A40000
SWEEP_BYTES = 13_422_428_160  # weights 13,400,801,280 + x 6,160,384 + y 15,466,496


# After an idle period the GPU's power management lets the first launch of a
# memory-bound kernel run at full speed, slows the next ones by up to 45 % and
# recovers over about 50 ms (measured on the 448-GEMV sweep: 2.25, 3.13, 2.78,
# 2.61, ... 2.15 ms, the same after 0.2 s and after 2 s of idle).  A decode
# loop runs in that steady state, so every workload first launches its step
# for SETTLE_S seconds of wall time, untimed, before its warm-up steps.
SETTLE_S = 0.25


def settle(fn, seconds: float = SETTLE_S) -> int:
    """Launch fn until `seconds` of wall time have passed (synchronizing every few
    launches so the queue stays short); returns the number of launches."""
    import torch
    if seconds <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def time_steps(fn, steps: int, warmup: int, settle_s: float = 0.0):
    import torch
    settle(fn, settle_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def sweep_inputs(q4, workload_id: int, m: int = 1):
    """Upload the 448 GEMVs' weights and inputs; returns device tensors and stream ids."""
    import torch
    import synth
    dev = torch.device("cuda:0")
    ws, xs, ys, ids = [], [], [], []
    for (layer, proj, n, k) in synth.decode_sweep():
        sw = synth.stream_id(1, layer, proj, synth.T_W)  # the same weights for every workload
        sx = synth.stream_id(workload_id, layer, proj, synth.T_X)
        w = torch.from_numpy(synth.q4_0(SEED, sw, n, k)).to(dev)
        x = torch.from_numpy(synth.f16_normal(SEED, sx, m * k).reshape(m, k) if m > 1
                             else synth.f16_normal(SEED, sx, k)).to(dev)
        ws.append(w)
        xs.append(x)
        ys.append(torch.empty((m, n) if m > 1 else (n,), dtype=torch.float32, device=dev))
        ids.append((sw, sx, n, k))
    torch.cuda.synchronize()
    return ws, xs, ys, ids


def bench_sweep(args):
    import torch
    q4 = load_q4()
    log("uploading the 64-layer sweep ...")
    t0 = time.time()
    ws, xs, ys, ids = sweep_inputs(q4, 1)
    log("  %.1f s" % (time.time() - t0))
    batch = q4.GemvBatch(list(zip(ws, xs, ys)))
    n_settle = settle(batch)
    ms = time_steps(batch, args.steps, args.warmup)
    gbs = SWEEP_BYTES / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16->f32", "data": "synthetic",
        "config": {"workload": "27B-shape decode weight sweep: 64 layers x (q,k,v,o 5120x5120; "
                               "gate,up 17408x5120; down 5120x17408), 448 Q4_0 GEMVs, M=1, one launch",
                   "weight_bytes": 13_400_801_280, "algorithmic_bytes_per_step": SWEEP_BYTES,
                   "seed": SEED},
        "settle_s": SETTLE_S, "settle_launches": n_settle,
        "sweeps_per_s": round(1000.0 / ms, 2),
        "pct_of_8TBps": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": counter_traffic("sweep"),
                     "kernel": "q4::k_sweep<QuadEngine<12,2,2,288>> (batch)", "launches_per_step": 1},
    }
    if args.sweep_only:  # (profiling runs: the sweep kernel alone)
        return out
    # the host's step after the sweep: final norm + LM head (151,936 x 5,120) + argmax, for the implied tokens/s
    import synth
    wl, hl, gl = lmhead_inputs()
    lg = torch.empty(synth.VOCAB, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(q4.workspace_bytes(q4.Q4_OP_LM_HEAD_NORM_ARGMAX, 1, synth.VOCAB, synth.HIDDEN),
                      dtype=torch.uint8, device="cuda")
    lm_ms = time_steps(lambda: q4.lm_head_norm_argmax(wl, hl, gl, NORM_EPS, lg, tok, workspace=wsp),
                       max(args.steps, 20) * 10, args.warmup, settle_s=SETTLE_S)
    del wl, hl, gl, lg
    ceiling = stream_ceiling()
    out.update({
        "stream_ceiling_GBps": ceiling["GBps"], "stream_ceiling_pattern": ceiling["pattern"],
        "pct_of_stream_ceiling": round(100.0 * gbs / ceiling["GBps"], 2),
        "lm_head_norm_argmax_us": round(lm_ms * 1000.0, 2),
        "implied_tok_s": round(1000.0 / (ms + lm_ms), 2),
    })
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ids)
    return out


def bench_gemv(args):
    """Single 5120x5120 GEMV, cycling through enough weight copies to exceed the last-level cache."""
    import torch
    import synth
    q4 = load_q4()
    n = k = 5120
    copies = 48  # 48 x 14.7 MB = 708 MB > 256 MB
    w0 = synth.q4_0(SEED, synth.stream_id(0, 0, 0, synth.T_W), n, k)
    ws = [torch.from_numpy(w0).cuda() for _ in range(copies)]
    x = torch.from_numpy(synth.f16_normal(SEED, synth.stream_id(0, 0, 0, synth.T_X), k)).cuda()
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    it = [0]

    def step():
        q4.q4_0_gemv(ws[it[0] % copies], x, y)
        it[0] += 1
    steps = max(args.steps, 1) * copies
    ms = time_steps(step, steps, args.warmup * copies, settle_s=SETTLE_S)
    hot_ms = time_steps(lambda: q4.q4_0_gemv(ws[0], x, y), steps, args.warmup)
    bytes_ = n * k // 32 * 18 + k * 2 + n * 4
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"metric": "Q4_0 GEMV HBM GB/s (single 5120x5120 GEMV, cold weights)", "value": round(gbs, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16->f32",
            "data": "synthetic", "config": {"workload": "single Q4_0 GEMV 5120x5120, 48 rotating weight copies"},
            "hot_cache_GBps": round(bytes_ / (hot_ms * 1e-3) / 1e9, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("gemv"),
                         "kernel": "q4::k_gemv_rows<288, false>"}}


def bench_q8(args):
    """Q8_0 GEMVs over the layers of a small dense model shaped like Qwen3 4B
    (36 layers x q 4096x2560, k and v 1024x2560, o 2560x4096, gate and up
    9728x2560, down 2560x9728: 252 GEMVs, 3.86 GB of Q8_0 weights), each with
    its own f16 input; one step = one launch of the Q8_0 batch over the 252
    GEMVs (the 252 single launches replayed from a HIP graph are timed beside it)."""
    import torch
    import synth
    q4 = load_q4()
    log("uploading the Q8_0 layers ...")
    ws, xs, ys = [], [], []
    wbytes = io = 0
    for layer in range(synth.Q8_LAYERS):
        for p, (_, n, k) in enumerate(synth.Q8_PROJ):
            w = synth.q8_0(SEED, synth.stream_id(6, layer, p, synth.T_W), n, k)
            ws.append(torch.from_numpy(w).cuda())
            xs.append(torch.from_numpy(synth.f16_normal(SEED, synth.stream_id(6, layer, p, synth.T_X), k)).cuda())
            ys.append(torch.empty(n, dtype=torch.float32, device="cuda"))
            wbytes += w.nbytes
            io += 2 * k + 4 * n

    batch = q4.Q8Batch(list(zip(ws, xs, ys)))
    n_slab, n_all = batch.plan.n_slab, batch.plan.count
    kernels = ([] if n_slab == 0 else ["q4::k_sweep<Q8Engine<8,3,448>> (%d GEMVs)" % n_slab]) + \
        ([] if n_slab == n_all else ["q4::k_q8_batch (%d GEMVs)" % (n_all - n_slab)])
    ms = time_steps(batch, args.steps, args.warmup, settle_s=SETTLE_S)

    def singles():
        for w, x, y in zip(ws, xs, ys):
            q4.q8_0_gemv(w, x, y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        singles()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        singles()
    graph_ms = time_steps(g.replay, max(2, args.steps // 3), 3)
    gbs = (wbytes + io) / (ms * 1e-3) / 1e9
    return {"metric": "Q8_0 GEMV HBM GB/s over a small dense model's layers (Qwen3-4B shapes)",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16->f32", "data": "synthetic",
            "config": {"workload": "36 layers x 7 Q8_0 GEMVs (q 4096x2560, k,v 1024x2560, o 2560x4096, gate,up "
                                   "9728x2560, down 2560x9728), one q8_0_gemv_batch call",
                       "weight_bytes": wbytes, "algorithmic_bytes_per_step": wbytes + io},
            "graph_of_single_launches_ms": round(graph_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("q8"),
                         "kernel": " + ".join(kernels), "launches_per_step": len(kernels)}}


STAGE_LAYERS = 22  # a stage of layers 0..21, the pages' example of one peer's range


def bench_handoff(args):
    """The stage hand-off: a peer's layer range (layers 0..21 of the 64-layer
    sweep: 154 GEMVs, 4.6 GB of weights) as ONE batch launch whose last GEMV
    (layer 21's down projection) writes the binary16 hidden state
    (residual + y) for the next stage; the same list without the hand-off and
    the hand-off GEMV alone (5,120 x 17,408, 16 rotating weight copies) are
    timed beside it."""
    import torch
    import synth
    q4 = load_q4()
    log("uploading layers 0..%d ..." % (STAGE_LAYERS - 1))
    ws, xs, ys = [], [], []
    io = 0
    for (layer, proj, n, k) in synth.decode_sweep():
        if layer >= STAGE_LAYERS:
            break
        ws.append(torch.from_numpy(synth.q4_0(SEED, synth.stream_id(1, layer, proj, synth.T_W), n, k)).cuda())
        xs.append(torch.from_numpy(synth.f16_normal(SEED, synth.stream_id(5, layer, proj, synth.T_X), k)).cuda())
        ys.append(torch.empty(n, dtype=torch.float32, device="cuda"))
        io += 2 * k + 4 * n
    n_last = ys[-1].numel()
    r = torch.from_numpy(4.0 * synth.f16_normal(SEED, synth.stream_id(5, STAGE_LAYERS - 1, 6, synth.T_R),
                                                n_last).astype(np.float32)).cuda()
    h16 = torch.empty(n_last, dtype=torch.float16, device="cuda")
    stage = q4.GemvBatch(list(zip(ws, xs, ys)))
    stage.set_handoff(len(ws) - 1, h16, r)
    plain = q4.GemvBatch(list(zip(ws, xs, [torch.empty_like(y) for y in ys])))
    wbytes = sum(w.numel() for w in ws)
    stage_bytes = wbytes + io - 4 * n_last + 2 * n_last + 4 * n_last  # last y: binary16 out, residual in
    for f in (stage, plain):
        time_steps(f, 1, args.warmup, settle_s=SETTLE_S)
    blocks = {"stage": [], "plain": []}
    for rr in range(4):
        for name in (("stage", "plain") if rr % 2 == 0 else ("plain", "stage")):
            blocks[name].append(time_steps(stage if name == "stage" else plain, args.steps, 0))
    ms = float(np.median(blocks["stage"]))
    plain_ms = float(np.median(blocks["plain"]))
    gbs = stage_bytes / (ms * 1e-3) / 1e9

    # the hand-off GEMV alone, cold weights
    n, k = synth.HIDDEN, synth.FFN
    copies = 16  # 16 x 50 MB > 256 MB
    w0 = ws[-1].cpu()
    wc = [w0.cuda() for _ in range(copies)]
    it = [0]

    def single():
        q4.q4_0_gemv_handoff(wc[it[0] % copies], xs[-1], r, h16)
        it[0] += 1
    single_ms = time_steps(single, args.steps * copies, args.warmup * copies)
    return {"metric": "stage hand-off: a 22-layer range of Q4_0 GEMVs ending in the binary16 hidden state, HBM GB/s",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": 4 * args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16->f32->f16", "data": "synthetic",
            "config": {"workload": "layers 0..21 of the 27B-shape sweep (154 Q4_0 GEMVs) in one batch launch, the "
                                   "last (down projection 5120x17408) writing binary16(residual + y)",
                       "weight_bytes": wbytes, "algorithmic_bytes_per_step": stage_bytes},
            "without_handoff_ms": round(plain_ms, 4), "handoff_overhead_us": round((ms - plain_ms) * 1000.0, 2),
            "single_handoff_gemv_us": round(single_ms * 1000.0, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("handoff"),
                         "kernel": "q4::k_sweep<QuadEngine<12,2,2,288>> (batch, hand-off descriptor)",
                         "launches_per_step": 1}}


def bench_lmhead(args):
    import torch
    import synth
    q4 = load_q4()
    n, k = synth.VOCAB, synth.HIDDEN
    w = torch.from_numpy(synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), n, k)).cuda()
    h = torch.from_numpy(synth.f16_normal(SEED, synth.stream_id(2, 0, 0, synth.T_X), k)).cuda()
    lg = torch.empty(n, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(q4.workspace_bytes(q4.Q4_OP_LM_HEAD_ARGMAX, 1, n, k), dtype=torch.uint8, device="cuda")
    ms = time_steps(lambda: q4.lm_head_argmax(w, h, lg, tok, wsp), args.steps * 10, args.warmup, settle_s=SETTLE_S)
    bytes_ = n * k // 32 * 18 + k * 2 + n * 4 + 4
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"metric": "LM head + greedy argmax HBM GB/s (151936x5120 Q4_0)", "value": round(gbs, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps * 10, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16->f32",
            "data": "synthetic", "config": {"workload": "LM head 151936x5120 + argmax"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("lmhead"),
                         "kernel": "q4::k_sweep<QuadEngine<11,2,2,288>,ARGMAX> + q4::k_argmax_final"}}


NORM_EPS = 1e-6


def lmhead_inputs():
    """The LM head's weights (151,936 x 5,120), a hidden state (4 z, z ~ N(0,1)) and the final norm's gain."""
    import torch
    import synth
    w = torch.from_numpy(synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), synth.VOCAB, synth.HIDDEN)).cuda()
    h = torch.from_numpy(synth.f16_scaled_normal(SEED, synth.stream_id(2, 0, 0, synth.T_X), synth.HIDDEN, 4.0)).cuda()
    g = torch.from_numpy(synth.norm_gain(SEED, synth.stream_id(2, 0, 1, synth.T_X), synth.HIDDEN)).cuda()
    return w, h, g


def bench_lmhead_norm(args):
    """The final norm fused into the LM head (151,936 x 5,120) with the greedy
    pick; the plain LM head on the same weights is timed beside it."""
    import torch
    import synth
    q4 = load_q4()
    n, k = synth.VOCAB, synth.HIDDEN
    w, h, g = lmhead_inputs()
    lg = torch.empty(n, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(q4.workspace_bytes(q4.Q4_OP_LM_HEAD_NORM_ARGMAX, 1, n, k), dtype=torch.uint8, device="cuda")
    steps = args.steps * 10
    fused = lambda: q4.lm_head_norm_argmax(w, h, g, NORM_EPS, lg, tok, workspace=wsp)  # noqa: E731
    plain = lambda: q4.lm_head_argmax(w, h, lg, tok, wsp)  # noqa: E731
    # both warmed, then timed in alternating blocks (the first blocks after the
    # inputs are written run slower, which would otherwise land on one side)
    for f in (fused, plain):
        time_steps(f, 1, args.warmup, settle_s=SETTLE_S)
    blocks = {"fused": [], "plain": []}
    for r in range(4):
        for name in (("fused", "plain") if r % 2 == 0 else ("plain", "fused")):
            blocks[name].append(time_steps(fused if name == "fused" else plain, steps, 0))
    ms = float(np.median(blocks["fused"]))
    plain_ms = float(np.median(blocks["plain"]))
    steps *= 4
    bytes_ = n * k // 32 * 18 + 2 * k * 2 + n * 4 + 4
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"metric": "final norm + LM head + greedy argmax HBM GB/s (151936x5120 Q4_0)", "value": round(gbs, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16->f32",
            "data": "synthetic", "config": {"workload": "RMS norm of h (k=5120) fused into LM head 151936x5120 + argmax"},
            "tokens_per_s": round(1.0 / (ms * 1e-3), 1), "plain_lm_head_ms": round(plain_ms, 5),
            "norm_overhead_us": round((ms - plain_ms) * 1000.0, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("lmhead_norm"),
                         "kernel": "q4::k_sweep<QuadEngine<11,2,2,288>,ARGMAX,NORM> + q4::k_argmax_final"}}


def bench_verify(args):
    """Greedy verify of an M-token draft against the LM head (151,936 x 5,120):
    the M rows' logits, their greedy tokens and the accepted prefix, per call."""
    import torch
    import synth
    q4 = load_q4()
    m = args.m or 4
    n, k = synth.VOCAB, synth.HIDDEN
    w = torch.from_numpy(synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), n, k)).cuda()
    h = torch.from_numpy(synth.f16_normal(SEED, synth.stream_id(2, 0, 1, synth.T_X), m * k).reshape(m, k)).cuda()
    draft = torch.zeros(m, dtype=torch.int32, device="cuda")
    lg = torch.empty((m, n), dtype=torch.float32, device="cuda")
    tok = torch.empty(m, dtype=torch.int32, device="cuda")
    acc = torch.empty(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(max(16, q4.workspace_bytes(q4.Q4_OP_LM_HEAD_VERIFY, m, n, k)), dtype=torch.uint8, device="cuda")
    ms = time_steps(lambda: q4.lm_head_verify(w, h, draft, lg, tok, acc, wsp), args.steps * 10, args.warmup,
                    settle_s=SETTLE_S)
    bytes_ = n * k // 32 * 18 + m * k * 2 + m * n * 4 + 2 * m * 4 + 4
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"metric": "greedy verify of an M-token draft: LM head GB/s (151936x5120 Q4_0, M=%d)" % m,
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps * 10, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16->f32", "data": "synthetic",
            "config": {"workload": "verify M=%d draft rows against the LM head 151936x5120" % m},
            "draft_tokens_per_s": round(m / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": counter_traffic("verify_m%d" % m),
                         "kernel": ("q4::k_sweep (GEMV) + k_argmax_rows" if m == 1 else
                                    "q4::k_smallm_lds (row keys fused)" if m <= 7 else
                                    "q4::k_smallm_reg + k_argmax_rows") + " + k_verify_final"}}


def bench_gemm(args, prefill: bool):
    import torch
    q4 = load_q4()
    m = args.m or (169 if prefill else 16)
    ws, xs, ys, ids = sweep_inputs(q4, 4 if prefill else 3, m=m)
    if prefill:
        # the 448 GEMMs as one prefill batch: one launch
        batch = q4.PrefillBatch(list(zip(ws, xs, ys)))
        ms = time_steps(batch, args.steps, args.warmup, settle_s=SETTLE_S)

        def step():
            for w, x, y in zip(ws, xs, ys):
                q4.q4_0_gemm_prefill(w, x, y)
        eager_ms = time_steps(step, max(1, args.steps // 2), 1)  # 448 separate launches, for reference
        how = "one batched launch"
    else:
        # the 448 GEMMs as one small-M batch: one launch (plus the K-range sum when K is split)
        batch = q4.SmallMBatch(list(zip(ws, xs, ys)))
        ms = time_steps(batch, args.steps, args.warmup, settle_s=SETTLE_S)
        eager_ms = ms
        how = "one batched launch"
    wbytes = 13_400_801_280
    io = m * (6_160_384 + 15_466_496)
    flops = 2.0 * m * 23_823_646_720
    gbs = (wbytes + io) / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    name = "prefill" if prefill else "small-M"
    rl = ({"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tf / PEAK_F16_TFLOPS, 4)} if prefill else
          {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(gbs / PEAK_HBM_GBS, 4)})
    rl["traffic"] = counter_traffic("prefill_m%d" % m if prefill else "smallm_m%d" % m)
    if prefill:
        tm = batch.plan.tile_m
        rl["kernel"] = "q4::k_prefill_q<%d,4> (batch, %d-row tiles)" % (tm // 32, tm)
    else:
        rl["kernel"] = ("q4::k_smallm_lds" if m <= 7 else "q4::k_smallm_reg") + " (batch)"
    extra = {}
    if not prefill and m >= 8:
        # beside the HBM roofline: the matrix cores (every MFMA covers 16 activation rows whatever M is)
        extra["roofline_mfma"] = {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_F16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_F16_TFLOPS, 5),
                                  "issued_16_rows": round(tf * 16 / m, 3)}
    return {**{"metric": "%s Q4_0 GEMM over the 64-layer sweep (M=%d)" % (name, m),
            "value": round(tf if prefill else gbs, 3), "unit": "TFLOP/s" if prefill else "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16->f32",
            "data": "synthetic", "config": {"workload": "%s M=%d x 448 sweep GEMMs, %s" % (name, m, how)},
            "tflops": round(tf, 3), "GBps": round(gbs, 2), "eager_ms_per_step": round(eager_ms, 4), "roofline": rl},
            **extra}


STREAM_BYTES = 16 << 30
# (pattern, workgroups of 256 threads per CU) of the read-ceiling probe: 0/1
# grid-stride cached / non-temporal loads, 2/3 one contiguous range per
# workgroup cached / non-temporal, 4 non-temporal buffer loads into an LDS ring
STREAM_PATTERNS = {0: "grid-stride, cached", 1: "grid-stride, non-temporal", 2: "range per workgroup, cached",
                   3: "range per workgroup, non-temporal", 4: "range per workgroup, non-temporal into LDS"}
STREAM_CONFIGS = [(p, w) for p in range(4) for w in (1, 2, 4, 8)] + [(4, 1), (4, 2), (4, 3)]
STREAM_BEST = [(1, 1), (3, 2), (4, 2), (4, 3)]  # the fastest configurations on MI355X


def load_stream():
    import ctypes
    from q4_dequant_gemv_block_amd import build
    if not os.path.exists(build.STREAM_LIB):
        build.build()
    lib = ctypes.CDLL(build.STREAM_LIB)
    lib.q4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.q4_stream_read.restype = ctypes.c_int
    return lib


def stream_rates(configs, steps: int, warmup: int, nbytes: int = STREAM_BYTES) -> list:
    """Read rate of a fresh nbytes buffer for each (pattern, wg_per_cu)."""
    import torch
    lib = load_stream()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.view(torch.int32).fill_(0x5A5A5A5A)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for i, (p, w) in enumerate(configs):
        def step(p=p, w=w):
            st = lib.q4_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), p, w, stream)
            if st != 0:
                raise RuntimeError("q4_stream_read(%d, %d): %d" % (p, w, st))
        ms = time_steps(step, steps, warmup, settle_s=SETTLE_S if i == 0 else 0.05)
        res.append({"pattern": p, "wg_per_cu": w, "what": STREAM_PATTERNS[p], "ms": round(ms, 4),
                    "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    del buf
    return res


def stream_ceiling() -> dict:
    """The best read rate over the fastest probe configurations (16 GiB read once)."""
    best = max(stream_rates(STREAM_BEST, 10, 2), key=lambda r: r["GBps"])
    return {"GBps": best["GBps"], "pattern": "%s, %d workgroups/CU" % (best["what"], best["wg_per_cu"])}


def bench_stream(args):
    """The device's read-bandwidth ceiling: a 16 GiB buffer read once and folded
    into one word (libq4stream), for every probe configuration, or the one
    --pattern/--wg-per-cu names.  value = the best rate."""
    configs = STREAM_CONFIGS if args.pattern < 0 else [(args.pattern, args.wg_per_cu)]
    res = stream_rates(configs, args.steps, args.warmup)
    best = max(res, key=lambda r: r["GBps"])
    return {"metric": "HBM read ceiling GB/s (16 GiB read once, read-reduce)", "value": best["GBps"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": best["ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": "read-reduce of %d bytes" % STREAM_BYTES, "best": "%s, %d workgroups/CU" % (
                best["what"], best["wg_per_cu"])},
            "pct_of_8TBps": round(100.0 * best["GBps"] / PEAK_HBM_GBS, 2), "settle_s": SETTLE_S,
            "configs": res,
            "roofline": {"bound": "hbm", "achieved": best["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(best["GBps"] / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "libq4stream pattern %d" % best["pattern"]}}


COPY_BYTES = 1 << 30


def bench_copy(args):
    """A plain device-to-device copy of 1 GiB: the known-size kernel that
    calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms = time_steps(lambda: b.copy_(a), args.steps, args.warmup, settle_s=SETTLE_S)
    return {"metric": "device copy GB/s (counter calibration)", "value": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "copy of %d bytes" % COPY_BYTES}}


def _counter_mean(csv_path: str, kernel_substr: str, counter: str) -> float:
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit("no %s samples for kernels matching %r in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals)


def record_traffic(workload: str, kernel: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                   copy_write_csv: str) -> dict:
    """HBM bytes per launch of `kernel` from rocprofv3 FETCH_SIZE and WRITE_SIZE
    runs (KiB per dispatch), each scaled by what the same counter reads for the
    1 GiB copy, written into profiles/traffic.json under `workload`."""
    copy_kernel = "copy"
    f_copy = _counter_mean(copy_fetch_csv, copy_kernel, "FETCH_SIZE")
    w_copy = _counter_mean(copy_write_csv, copy_kernel, "WRITE_SIZE")
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    fetch = _counter_mean(fetch_csv, kernel, "FETCH_SIZE") * 1024.0 * f_scale
    write = _counter_mean(write_csv, kernel, "WRITE_SIZE") * 1024.0 * w_scale
    path = os.path.join(PROFILE_DIR, "traffic.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table[workload] = {"kernel": kernel, "source_hash": kernel_source_hash(workload),
                       "bytes_per_launch": int(round(fetch + write)),
                       "fetch_bytes": int(round(fetch)), "write_bytes": int(round(write)),
                       "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    return table[workload]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # (before these, every workload settles for SETTLE_S seconds: see there)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sweep",
                    choices=["sweep", "gemv", "lmhead", "lmhead_norm", "handoff", "q8", "verify", "smallm",
                             "prefill", "copy", "stream"])
    ap.add_argument("--m", type=int, default=0)
    ap.add_argument("--pattern", type=int, default=-1, help="stream: one probe pattern (0..4) instead of all")
    ap.add_argument("--wg-per-cu", type=int, default=2, help="stream: workgroups per CU with --pattern")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-only", action="store_true",
                    help="sweep: time the sweep alone (no LM head, read ceiling or CPU baseline), for profiling")
    ap.add_argument("--record-traffic", nargs=6, metavar=("WORKLOAD", "KERNEL", "FETCH_CSV", "WRITE_CSV",
                                                          "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs and exit (no GPU needed)")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fn = {"sweep": bench_sweep, "gemv": bench_gemv, "lmhead": bench_lmhead, "lmhead_norm": bench_lmhead_norm,
          "handoff": bench_handoff, "q8": bench_q8,
          "verify": bench_verify, "copy": bench_copy, "stream": bench_stream,
          "smallm": lambda a: bench_gemm(a, False), "prefill": lambda a: bench_gemm(a, True)}[args.workload]
    out = fn(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
