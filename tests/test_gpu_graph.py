"""Entry points captured into a HIP graph: every replay, with eager work and
synchronizations between replays, matches the eager result bit for bit."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_f16, dev_u8, device, lib

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def test_graph_replays_match_eager():
    q4 = lib()
    k = 5120
    w1 = dev_u8(synth.q4_0(SEED, 11, 1000, k))
    w2 = dev_u8(synth.q4_0(SEED, 12, 3000, k))
    x1 = dev_f16(synth.f16_normal(SEED, 13, k))
    x16 = dev_f16(synth.f16_normal(SEED, 14, 16 * k).reshape(16, k))
    y1 = torch.empty(1000, dtype=torch.float32, device=device())
    y2 = torch.empty(3000, dtype=torch.float32, device=device())
    ys = torch.empty((16, 3000), dtype=torch.float32, device=device())
    yp = torch.empty((16, 1000), dtype=torch.float32, device=device())
    lg = torch.empty(3000, dtype=torch.float32, device=device())
    tok = torch.empty(1, dtype=torch.int32, device=device())
    ws_s = torch.empty(max(16, q4.workspace_bytes(q4.Q4_OP_GEMM_SMALLM, 16, 3000, k)), dtype=torch.uint8, device=device())
    ws_l = torch.empty(max(16, q4.workspace_bytes(q4.Q4_OP_LM_HEAD_ARGMAX, 1, 3000, k)), dtype=torch.uint8, device=device())
    batch = q4.GemvBatch([(w1, x1, y1), (w2, x1, y2)])

    def work():
        batch()
        q4.q4_0_gemm_smallm(w2, x16, ys, ws_s)
        q4.q4_0_gemm_prefill(w1, x16, yp)
        q4.lm_head_argmax(w2, x1, lg, tok, ws_l)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y1, y2, ys, yp, lg, tok)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (y1, y2, ys, yp, lg):
            t.fill_(float("nan"))
        tok.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, (y1, y2, ys, yp, lg, tok)):
            assert torch.equal(e, t), rep
        # eager work between replays
        q4.q4_0_gemv(w1, x1)
        torch.cuda.synchronize()
