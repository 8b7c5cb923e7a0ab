"""lm_head_argmax_noalloc (the LM head entry point that allocates nothing)
against lm_head_argmax, the entry point with a caller's workspace: logits bit
for bit, the same token, the oracle's bound and argmax rule; calls in a row,
the second with a smaller input (its keys array then still holds the first
call's keys beyond the second call's grid), the third the first size again
(the one-launch counter must be back at zero)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def test_noalloc_equals_workspace_entry_point():
    q4 = lib()
    rng = np.random.default_rng(77)
    # the second smaller; the third the first again (the one-launch counter is back at zero after each call)
    cases = [(synth.VOCAB, synth.HIDDEN, 1500), (3001, 1024, 1501), (synth.VOCAB, synth.HIDDEN, 1502)]
    for n, k, stream in cases:
        w = synth.q4_0(SEED, stream, n, k)
        h = synth.f16_normal(SEED, stream + 10, k)
        wd, hd = dev_u8(w), dev_f16(h)
        say("noalloc lm head n=%d k=%d" % (n, k))
        lg_ref, tok_ref = q4.lm_head_argmax(wd, hd)
        lg = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        q4.lm_head_argmax_noalloc(wd, hd, lg, tok)
        torch.cuda.synchronize()
        assert torch.equal(lg.view(torch.int32), lg_ref.view(torch.int32))
        assert int(tok.item()) == int(tok_ref.item())
        logits = lg.cpu().numpy()
        t = int(tok.item())
        assert t == int(np.argmax(logits))
        rows = np.unique(np.concatenate([[0, n - 1, t], rng.integers(0, n, 2000)]))
        y_ref, a_ref = oracle.gemm_rows(w[rows], k, h)
        assert_parity(logits[rows], y_ref, a_ref, "noalloc n=%d" % n)
        if n <= 4096:  # the whole vocabulary: the oracle's greedy rule
            y_all, a_all = oracle.gemm_rows(w, k, h)
            r = oracle.argmax(y_all)
            assert t == r or y_all[r] - y_all[t] < TOL * max(a_all[r], a_all[t]), (t, r)
