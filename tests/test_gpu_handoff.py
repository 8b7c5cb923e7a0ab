"""q4_0_gemv_handoff: the stage hand-off epilogue (binary16 of residual + W x).

Bit for bit against the binary16 rounding of q4_0_gemv's binary32 output plus
the residual (numpy's float32 add and float16 rounding: the same kernel makes
both); against the oracle, every h16 lies between the binary16 values just
below and just above residual + y_ref -+ the GEMV bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def f16_down(v):
    c = v.astype(np.float16)
    return np.where(c.astype(np.float64) > v, np.nextafter(c, np.float16(-np.inf)), c)


def f16_up(v):
    c = v.astype(np.float16)
    return np.where(c.astype(np.float64) < v, np.nextafter(c, np.float16(np.inf)), c)


def check(n, k, with_residual, stream_base):
    q4 = lib()
    w = synth.q4_0(SEED, stream_base, n, k)
    x = synth.f16_normal(SEED, stream_base + 1, k)
    r = (4.0 * synth.f16_normal(SEED, stream_base + 2, n).astype(np.float32)) if with_residual else None
    w_d, x_d = dev_u8(w), dev_f16(x)
    r_d = torch.from_numpy(r).cuda() if with_residual else None
    h16 = q4.q4_0_gemv_handoff(w_d, x_d, r_d)
    y32 = q4.q4_0_gemv(w_d, x_d)
    torch.cuda.synchronize()
    h = h16.cpu().numpy()
    y = y32.cpu().numpy()
    # bit for bit: binary16(binary32(y) + residual), nearest-even
    want = (y + r).astype(np.float16) if with_residual else y.astype(np.float16)
    assert np.array_equal(h.view(np.uint16), want.view(np.uint16)), (n, k)
    # against the oracle: inside the rounding of the GEMV bound around residual + y_ref
    h_ref, y_ref, a_ref = oracle.gemv_handoff(w, k, x, r)
    base = y_ref + (r.astype(np.float64) if with_residual else 0.0)
    slack = TOL * a_ref + 2.0 ** -23 * np.abs(base)
    hv = h.astype(np.float64)
    lo, hi = f16_down(base - slack).astype(np.float64), f16_up(base + slack).astype(np.float64)
    bad = (hv < lo) | (hv > hi)
    assert not bad.any(), (n, k, np.argwhere(bad)[:5].ravel().tolist())
    same = float(np.mean(h.view(np.uint16) == h_ref))
    say("handoff n=%d k=%d residual=%s: equal to the oracle's rounding %.4f" % (n, k, with_residual, same))
    assert same > 0.99


@pytest.mark.parametrize("n,k", [(5120, 17408), (5120, 5120), (70, 64), (3001, 1024), (1000, 20480), (20000, 5120)])
@pytest.mark.parametrize("with_residual", [True, False])
def test_handoff(n, k, with_residual):
    check(n, k, with_residual, 9100 + k % 997 + n % 13)


def test_handoff_out_of_place_and_into_preallocated():
    """Writing into a caller's buffer gives the same bits; a second call overwrites."""
    q4 = lib()
    n, k = 5120, 17408
    w = dev_u8(synth.q4_0(SEED, 9201, n, k))
    x = dev_f16(synth.f16_normal(SEED, 9202, k))
    r = torch.from_numpy(synth.f16_normal(SEED, 9203, n).astype(np.float32)).cuda()
    a = q4.q4_0_gemv_handoff(w, x, r)
    out = torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
    q4.q4_0_gemv_handoff(w, x, r, out=out)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("n,k,scale", [(1, 64, 4.0), (3, 1024, 3.0e4), (129, 4096, 1.0e-6)])
def test_handoff_edges(n, k, scale):
    """A single row; residuals near the top of binary16's range; residuals far
    below the outputs."""
    q4 = lib()
    w = synth.q4_0(SEED, 9300 + n, n, k)
    x = synth.f16_normal(SEED, 9301, k)
    r = (scale * synth.f16_normal(SEED, 9302, n)).astype(np.float32)
    r = np.clip(r, -60000.0, 60000.0).astype(np.float32)
    w_d, x_d = dev_u8(w), dev_f16(x)
    h16 = q4.q4_0_gemv_handoff(w_d, x_d, torch.from_numpy(r).cuda())
    y = q4.q4_0_gemv(w_d, x_d)
    torch.cuda.synchronize()
    want = (y.cpu().numpy() + r).astype(np.float16)
    assert np.array_equal(h16.cpu().numpy().view(np.uint16), want.view(np.uint16))
