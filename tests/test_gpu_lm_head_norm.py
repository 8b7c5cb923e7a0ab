"""lm_head_norm_argmax: the final norm fused into the LM head.

The normed activation (x_out) against the oracle's binary16 rounding, element
by element; the logits against the oracle's product on its own normed x (the
bound of the GEMV) and against lm_head_argmax on the GPU's x (bit for bit: the
fused kernel differs only in how it stages the activation); the greedy token
against the oracle's argmax rule."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED
EPS = float(np.float32(1e-6))
# The kernel's binary32 statistics put v = h g r within this relative distance
# of the binary64 value: a difference in the binary16 rounding can only come
# from a v that close to a midpoint.
NEAR_MIDPOINT = 2.0 ** -18


def run(w_d, h_np, g_np, eps=EPS, want_x=True):
    q4 = lib()
    k = h_np.shape[0]
    x_out = torch.empty(k, dtype=torch.float16, device="cuda") if want_x else None
    logits, token = q4.lm_head_norm_argmax(w_d, dev_f16(h_np), dev_f16(g_np), eps, x_out=x_out)
    torch.cuda.synchronize()
    x = x_out.cpu().numpy().view(np.uint16) if want_x else None
    return logits.cpu().numpy(), int(token.cpu().numpy()[0]), x


def check_x(x_gpu, h, g, eps):
    """Equal to the oracle's x, or the other neighbour of a v next to a midpoint."""
    x_ref, v = oracle.rms_norm(h, g, eps)
    diff = np.nonzero(x_gpu != x_ref)[0]
    for i in diff:
        a = float(x_gpu[i:i + 1].view(np.float16)[0])
        b = float(x_ref[i:i + 1].view(np.float16)[0])
        assert np.isfinite(a) and np.isfinite(b), i
        assert np.nextafter(np.float16(b), np.float16(np.inf if a > b else -np.inf)) == np.float16(a), (i, a, b)
        mid = (a + b) / 2
        assert abs(v[i] - mid) <= NEAR_MIDPOINT * abs(v[i]), (i, v[i], a, b)
    return x_ref, len(diff)


def check_token(logits, token, y_ref, a_ref):
    assert token == int(np.argmax(logits))
    r = oracle.argmax(y_ref)
    if token != r:
        assert y_ref[r] - y_ref[token] < TOL * max(a_ref[r], a_ref[token]), (token, r)


def full_check(w, h, g, eps=EPS, what=""):
    k = h.shape[0]
    w_d = dev_u8(w)
    logits, token, x = run(w_d, h, g, eps)
    x_ref, flips = check_x(x, h, g, eps)
    y_ref, a_ref = oracle.gemm_rows(w, k, x_ref)
    ratio = assert_parity(logits, y_ref, a_ref, what + " vs oracle")
    check_token(logits, token, y_ref, a_ref)
    # the same logits and token as the plain LM head on the GPU's own x
    q4 = lib()
    l2, t2 = q4.lm_head_argmax(w_d, torch.from_numpy(x.view(np.float16).copy()).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(logits, l2.cpu().numpy()), what
    assert token == int(t2.cpu().numpy()[0]), what
    say(what, "x flips", flips, "max err/a %.3g" % ratio, "token", token)
    return logits, token, x


# shapes across the kernel's variants: narrow and wide, the four-row engine
# (k % 1024 == 0, k >= 4096) and the other, fixed and per-k activation stride
@pytest.mark.parametrize("n,k", [(70, 64), (3001, 1024), (4099, 4096), (1000, 960), (20000, 5120),
                                 (2500, 17408), (1200, 20480), (300, 32768)])
def test_norm_parity(n, k):
    w = synth.q4_0(SEED, 8100 + k, n, k)
    h = synth.f16_scaled_normal(SEED, 8200 + k, k, 4.0)
    g = synth.norm_gain(SEED, 8300 + k, k)
    full_check(w, h, g, what="n=%d k=%d" % (n, k))


@pytest.mark.parametrize("scale", [1e-3, 1.0, 300.0])
@pytest.mark.parametrize("eps", [EPS, 1.0])
def test_norm_scales_and_eps(scale, eps):
    """Hidden states from tiny (eps dominates at eps = 1) to large, with outlier dims."""
    n, k = 3000, 5120
    w = synth.q4_0(SEED, 8401, n, k)
    h = synth.f16_scaled_normal(SEED, 8402, k, scale)
    h[::640] = np.float16(40 * scale)  # a few large dims, as residual streams have
    g = synth.norm_gain(SEED, 8403, k)
    full_check(w, h, g, eps, what="scale=%g eps=%g" % (scale, eps))


def test_zero_hidden_state():
    n, k = 500, 2048
    w = synth.q4_0(SEED, 8501, n, k)
    logits, token, x = run(dev_u8(w), np.zeros(k, np.float16), synth.norm_gain(SEED, 8502, k))
    assert not np.any(x & 0x7FFF) and not np.any(logits) and token == 0


def test_deterministic_and_x_out_optional():
    n, k = 8000, 5120
    w = synth.q4_0(SEED, 8601, n, k)
    h = synth.f16_scaled_normal(SEED, 8602, k, 4.0)
    g = synth.norm_gain(SEED, 8603, k)
    w_d = dev_u8(w)
    l1, t1, x1 = run(w_d, h, g)
    l2, t2, x2 = run(w_d, h, g)
    l3, t3, _ = run(w_d, h, g, want_x=False)
    assert np.array_equal(x1, x2) and np.array_equal(l1, l2) and np.array_equal(l1, l3) and t1 == t2 == t3


def test_full_vocab_norm():
    """151,936 x 5,120: the LM head of the 27B shape, every logit against the oracle."""
    n, k = synth.VOCAB, synth.HIDDEN
    w = synth.q4_0(SEED, synth.stream_id(2, 0, 0, synth.T_W), n, k)
    h = synth.f16_scaled_normal(SEED, 8701, k, 4.0)
    g = synth.norm_gain(SEED, 8702, k)
    say("lm_head_norm full vocab")
    full_check(w, h, g, what="full vocab")


@pytest.mark.parametrize("case", ["one_row", "large_eps", "single_nonzero"])
def test_norm_degenerate_cases(case):
    """One vocabulary row; eps far above mean(h^2) (x scaled down by it); a hidden
    state with one nonzero element (x there = +-sqrt(k) g, zero elsewhere)."""
    n, k = (1, 1024) if case == "one_row" else (700, 2048)
    w = synth.q4_0(SEED, 8801, n, k)
    h = synth.f16_scaled_normal(SEED, 8802, k, 4.0)
    eps = EPS
    if case == "large_eps":
        eps = 1.0e4
    if case == "single_nonzero":
        h = np.zeros(k, np.float16)
        h[123] = np.float16(-3.0)
    g = synth.norm_gain(SEED, 8803, k)
    logits, token, x = full_check(w, h, g, eps, what=case)
    if case == "single_nonzero":
        assert np.count_nonzero(x & 0x7FFF) == 1
