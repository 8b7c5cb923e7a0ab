"""lm_head_verify: greedy verify of a speculative draft.  Logits against the
oracle, every row's token against the oracle's argmax rule and against the
GPU's own logits, the accepted prefix for drafts with a mismatch planted at
each position, and the tokens of the M = 1 path (lm_head_argmax per row)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def run(w_d, h_np, draft):
    q4 = lib()
    d = torch.tensor(np.asarray(draft, dtype=np.int32), device="cuda")
    logits, tokens, accepted = q4.lm_head_verify(w_d, dev_f16(h_np), d)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), tokens.cpu().numpy().astype(np.int64), int(accepted.cpu().numpy()[0])


def check_tokens(logits, tokens, y_ref, a_ref):
    """Each token is the lowest-index maximum of its own row of logits (bit-exact),
    and the oracle's greedy token unless the oracle's top two are within the bound."""
    for i in range(logits.shape[0]):
        assert tokens[i] == int(np.argmax(logits[i])), i
        r = oracle.argmax(y_ref[i])
        if tokens[i] != r:
            assert y_ref[i, r] - y_ref[i, tokens[i]] < TOL * max(a_ref[i, r], a_ref[i, tokens[i]]), (i, tokens[i], r)


@pytest.mark.parametrize("m,n,k", [(1, 3001, 1024), (2, 4099, 1024), (5, 257, 2048), (16, 3000, 5120), (16, 70, 64),
                                   (4, 1500, 32768), (1, 700, 32768)])  # k split into ranges; M = 1 at the largest k
def test_verify_parity_and_prefix(m, n, k):
    w = synth.q4_0(SEED, 7100 + m, n, k)
    h = synth.f16_normal(SEED, 7200 + m * 7 + k, m * k).reshape(m, k)
    say("verify m=%d n=%d k=%d" % (m, n, k))
    w_d = dev_u8(w)
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    logits, tokens, accepted = run(w_d, h, np.zeros(m))
    assert_parity(logits, y_ref, a_ref, "verify m=%d" % m)
    check_tokens(logits, tokens, y_ref, a_ref)
    assert accepted == oracle.accepted_prefix(tokens, np.zeros(m))
    # drafts equal to the GPU's tokens with a mismatch planted at row j (j == m: none)
    for j in range(m + 1):
        draft = tokens.copy()
        if j < m:
            draft[j] = (draft[j] + 1) % n if n > 1 else -1
        _, tok2, acc2 = run(w_d, h, draft)
        assert np.array_equal(tok2, tokens)  # deterministic
        assert acc2 == j == oracle.accepted_prefix(tokens, draft), (j, acc2)


def test_verify_matches_the_m1_path():
    """Row i's token equals lm_head_argmax on h[i] unless the two paths' logits
    (each within the bound) straddle a near-tie the oracle itself resolves within it."""
    m, n, k = 8, 5000, 2048
    w = synth.q4_0(SEED, 7301, n, k)
    h = synth.f16_normal(SEED, 7302, m * k).reshape(m, k)
    w_d = dev_u8(w)
    logits, tokens, _ = run(w_d, h, np.zeros(m))
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    q4 = lib()
    for i in range(m):
        l1, t1 = q4.lm_head_argmax(w_d, dev_f16(h[i]))
        torch.cuda.synchronize()
        t1 = int(t1.cpu().numpy()[0])
        if t1 != tokens[i]:
            assert abs(y_ref[i, t1] - y_ref[i, tokens[i]]) < TOL * max(a_ref[i, t1], a_ref[i, tokens[i]]), i


def test_verify_planted_winners_and_ties():
    """Row i's hidden state picks a planted row: a copy of one weight row placed
    later must lose the tie (lowest index wins)."""
    m, n, k = 4, 2048, 1024
    w = synth.q4_0(SEED, 7401, n, k)
    w[1500] = w[300]  # a tie between rows 300 and 1500 for every h
    h = synth.f16_normal(SEED, 7402, m * k).reshape(m, k)
    logits, tokens, _ = run(dev_u8(w), h, np.zeros(m))
    assert np.array_equal(logits[:, 300], logits[:, 1500])
    assert not np.any(tokens == 1500)
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    check_tokens(logits, tokens, y_ref, a_ref)


def test_full_vocab_verify():
    """151,936 x 5,120 with M = 4 draft rows: every logit against the oracle."""
    m, n, k = 4, synth.VOCAB, synth.HIDDEN
    w = synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), n, k)
    h = synth.f16_normal(SEED, 7501, m * k).reshape(m, k)
    say("verify full vocab m=%d" % m)
    y_ref, a_ref = oracle.gemm_rows(w, k, h)
    tokens_ref = np.array([oracle.argmax(y_ref[i]) for i in range(m)])
    draft = tokens_ref.copy()
    draft[2] = (draft[2] + 7) % n
    logits, tokens, accepted = run(dev_u8(w), h, draft)
    assert_parity(logits, y_ref, a_ref, "verify full vocab")
    check_tokens(logits, tokens, y_ref, a_ref)
    assert accepted == oracle.accepted_prefix(tokens, draft)
    say("tokens", tokens.tolist(), "oracle", tokens_ref.tolist(), "accepted", accepted)
