"""Every code byte value at every code position, one weight at a time.

Row r of the weights holds the byte r in all 16 code bytes of every block, so
code p of a block is r & 15 (p < 16) or r >> 4 (p >= 16), the format the
pages call "GGUF Q4_0" (taozi.news, section "支持模型与限制"); block b of row
r has the scale 2^((r + b) % 5 - 2).  With x the unit vector e_j the product
is exactly one weight per row, (code - 8) * d, an integer times a power of
two: every kernel that decodes the codes must return it bit for bit.  The
columns are the first and the last block pair of a row (block 0 of a pair
starts two bytes into a dword, block 1 four-byte aligned), at k = 4096
(whole-slab engines) and k = 1088 (the other engines and the per-step prefill
kernel)."""
import numpy as np
import pytest
import torch

from gpu_util import dev_f16, dev_u8, lib, say
import q4_encode

pytestmark = pytest.mark.gpu

N = 256


def case(k):
    nb = k // 32
    r = np.arange(N)
    codes = np.empty((N, k), dtype=np.uint8)
    blk = codes.reshape(N, nb, 32)
    blk[:, :, :16] = (r & 15)[:, None, None]
    blk[:, :, 16:] = (r >> 4)[:, None, None]
    expo = (r[:, None] + np.arange(nb)[None, :]) % 5 - 2
    d = np.ldexp(1.0, expo)
    w = q4_encode.encode(codes, d.astype(np.float16).view(np.uint16))
    cols = np.r_[0:64, k - 64:k]
    # want[i, r] = weight of row r at column cols[i]
    want = (codes[:, cols].astype(np.float64) - 8.0) * d[:, cols // 32]
    x = np.zeros((len(cols), k), dtype=np.float16)
    x[np.arange(len(cols)), cols] = 1.0
    return w, x, want.T.copy()


@pytest.mark.parametrize("k", [4096, 1088])
def test_gemv_single_and_batch(k):
    q4 = lib()
    w, x, want = case(k)
    wd = dev_u8(w)
    say("basis GEMVs", N, k, len(x))
    single = np.stack([q4.q4_0_gemv(wd, dev_f16(xi)).cpu().numpy() for xi in x])
    assert np.array_equal(single.astype(np.float64), want)
    items = [(wd, dev_f16(xi), torch.empty(N, dtype=torch.float32, device=wd.device)) for xi in x]
    q4.GemvBatch(items)()
    torch.cuda.synchronize()
    batch = np.stack([it[2].cpu().numpy() for it in items])
    assert np.array_equal(batch.astype(np.float64), want)


def test_lm_head_logits():
    q4 = lib()
    w, x, want = case(4096)
    wd = dev_u8(w)
    for i in (0, 1, 30, 33, 63, 64, 127):
        logits, tok = q4.lm_head_argmax(wd, dev_f16(x[i]))
        lg = logits.cpu().numpy().astype(np.float64)
        assert np.array_equal(lg, want[i])
        assert int(tok.cpu()[0]) == int(np.argmax(want[i]))  # first index of the maximum


@pytest.mark.parametrize("m", [4, 16])
@pytest.mark.parametrize("k", [4096, 1088])
def test_smallm(m, k):
    q4 = lib()
    w, x, want = case(k)
    wd = dev_u8(w)
    say("basis small-M", m, N, k)
    for i0 in range(0, len(x), m):
        y = q4.q4_0_gemm_smallm(wd, dev_f16(x[i0:i0 + m])).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), want[i0:i0 + m]), i0


@pytest.mark.parametrize("k", [4096, 1088])
def test_prefill(k):
    q4 = lib()
    w, x, want = case(k)
    say("basis prefill", len(x), N, k)
    y = q4.q4_0_gemm_prefill(dev_u8(w), dev_f16(x)).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), want)
