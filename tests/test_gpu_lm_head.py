"""lm_head_argmax: logits against the oracle, the greedy pick against the
oracle's argmax rule, planted ties and winners."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def run(w_np, h_np):
    q4 = lib()
    logits, token = q4.lm_head_argmax(dev_u8(w_np), dev_f16(h_np))
    torch.cuda.synchronize()
    return logits.cpu().numpy(), int(token.cpu().numpy()[0])


def check_pick(logits, token, y_ref, a_ref):
    # the token is the lowest-index maximum of the GPU's own logits
    assert token == int(np.argmax(logits))
    r = oracle.argmax(y_ref)
    if token != r:
        assert y_ref[r] - y_ref[token] < TOL * max(a_ref[r], a_ref[token]), (token, r)
    return r


@pytest.mark.parametrize("n", [1, 2, 31, 1000, 4099])
def test_small_vocab(n):
    k = 1024
    w = synth.q4_0(SEED, 300 + n, n, k)
    h = synth.f16_normal(SEED, 400 + n, k)
    logits, token = run(w, h)
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    assert_parity(logits, y_ref, a_ref)
    check_pick(logits, token, y_ref, a_ref)


def test_identical_rows_pick_index_zero():
    w1 = synth.q4_0(SEED, 501, 1, 512)
    w = np.repeat(w1, 3000, axis=0)
    logits, token = run(w, synth.f16_normal(SEED, 502, 512))
    assert np.all(logits == logits[0]) and token == 0


def test_full_lm_head():
    """151,936 x 5,120 (437.6 MB), every logit against the oracle, then planted ties."""
    n, k = synth.VOCAB, synth.HIDDEN
    w = synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), n, k)
    h = synth.f16_normal(SEED, synth.stream_id(2, 0, 0, synth.T_X), k)
    say("lm head full")
    logits, token = run(w, h)
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    assert_parity(logits, y_ref, a_ref, "lm head")
    r = check_pick(logits, token, y_ref, a_ref)
    say("token", token, "oracle", r)
    g = token
    # tie planted after the winner: the winner keeps its index
    w2 = w.copy()
    w2[n - 1] = w2[g]
    l2, t2 = run(w2, h)
    assert l2[n - 1] == l2[g] and t2 == g
    # tie planted before the winner: the earlier copy wins
    if g > 0:
        w3 = w.copy()
        w3[g // 2] = w3[g]
        _, t3 = run(w3, h)
        assert t3 == g // 2
    # planted winner: the best row with every scale doubled (its logit doubles, > 0)
    assert logits[g] > 0
    w4 = w.copy()
    blk = w4[17].reshape(-1, 18)
    src = w[g].reshape(-1, 18)
    d = (src[:, 0].astype(np.uint16) | (src[:, 1].astype(np.uint16) << 8)) + 0x0400
    blk[:] = src
    blk[:, 0] = (d & 0xFF).astype(np.uint8)
    blk[:, 1] = (d >> 8).astype(np.uint8)
    l4, t4 = run(w4, h)
    assert t4 == 17 and l4[17] == 2 * logits[g]


def test_widest_k_on_eight_wave_workgroups():
    """k = 32,768 with a vocabulary wide enough for the wide shape: the LM head
    (and its final-norm form) runs with 8-wave workgroups.  The logits equal
    q4_0_gemv's bit for bit, the token is their lowest-index maximum, and
    sampled rows lie within the bound."""
    q4 = lib()
    n, k = 33000, 32768
    w = synth.q4_0(SEED, 7900, n, k)
    h = synth.f16_normal(SEED, 7901, k)
    wd, hd = dev_u8(w), dev_f16(h)
    logits, token = q4.lm_head_argmax(wd, hd)
    y = q4.q4_0_gemv(wd, hd)
    torch.cuda.synchronize()
    assert torch.equal(logits, y)
    lg = logits.cpu().numpy()
    assert int(token.cpu().numpy()[0]) == int(np.argmax(lg))
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(4).integers(0, n, 126)]))
    y_ref, a_ref = oracle.gemm_rows(np.ascontiguousarray(w[rows]), k, h)
    assert_parity(lg[rows], y_ref, a_ref, "LM head k = 32768")
    # the final norm form: its x_out through the plain LM head gives the same logits and token
    g = dev_f16(synth.norm_gain(SEED, 7902, k))
    x_out = torch.empty(k, dtype=torch.float16, device="cuda")
    logits_n, token_n = q4.lm_head_norm_argmax(wd, hd, g, 1e-6, x_out=x_out)
    logits_p, token_p = q4.lm_head_argmax(wd, x_out)
    torch.cuda.synchronize()
    assert torch.equal(logits_n, logits_p) and int(token_n.item()) == int(token_p.item())
