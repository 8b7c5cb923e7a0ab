"""Weight matrices larger than 4 GiB: every row offset past 2^32 bytes.

A 4 GiB matrix is too large for the oracle, so each one here is a seeded block
of P rows (P prime, so the period meets every tile and row step at a
different phase) repeated until the matrix passes 2^32 bytes, plus a ragged
tail of the block's first rows.  Every kernel of this library computes a
row's output from that row's bytes and the activations alone, in one fixed
order, so row r of the large product must equal row r mod P of the block's own
product bit for bit; the block's product is checked against the oracle.  This
covers, at byte offsets past 2^32: the Q4_0 GEMV on its 12-wave engine
(k = 5,120) and its 8-wave engine (k = 32,768), the LM head and its greedy
pick (the allocation-free entry point too), a GEMV list, small-M on both
engines, greedy verify, prefill, and the Q8_0 slab engine."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED
FOUR_GIB = 1 << 32
P = 4099      # rows of the repeated Q4_0 block (prime)
TAIL = 1000   # rows of the block that follow the last full repeat
P8 = 2053     # rows of the repeated Q8_0 block (prime)


def tile_rows(block: torch.Tensor, rb: int) -> tuple[torch.Tensor, int]:
    """The block (uint8 [P, rb] on the GPU) repeated past 4 GiB, then its
    first TAIL rows: (matrix, repeats)."""
    p = block.shape[0]
    reps = FOUR_GIB // (p * rb) + 2
    n = reps * p + TAIL
    assert (n - 1) * rb > FOUR_GIB + p * rb  # a whole block lies past 2^32 bytes
    big = torch.empty((n, rb), dtype=torch.uint8, device=block.device)
    big[:reps * p].view(reps, p, rb).copy_(block.unsqueeze(0).expand(reps, p, rb))
    big[reps * p:].copy_(block[:TAIL])
    return big, reps


def same_bits_tiled(y_big: torch.Tensor, y_block: torch.Tensor, reps: int, what: str):
    """y_big [..., reps * p + TAIL] holds y_block [..., p] repeated, bit for bit."""
    p = y_block.shape[-1]
    yb = y_big.view(torch.int32)
    ys = y_block.view(torch.int32)
    full = yb[..., :reps * p].reshape(*yb.shape[:-1], reps, p)
    eq = full == ys.unsqueeze(-2)
    if not bool(eq.all()):
        bad = torch.nonzero(~eq)[:5].tolist()
        raise AssertionError("%s: %d outputs differ from the block's, first %s" % (what, int((~eq).sum()), bad))
    assert torch.equal(yb[..., reps * p:], ys[..., :TAIL]), what + " (tail)"


def sampled(p: int, seed: int) -> np.ndarray:
    """512 distinct rows of p, the first and the last included."""
    inner = np.random.default_rng(seed).choice(np.arange(1, p - 1), 510, replace=False)
    return np.unique(np.concatenate([[0, p - 1], inner]))


@pytest.fixture(scope="module", params=[5120, 32768], ids=["k5120", "k32768"])
def q4_big(request):
    """(k, host block, device block, large matrix, repeats, x) for one k."""
    k = request.param
    block = synth.q4_0(SEED, 9800 + k % 997, P, k)
    x = synth.f16_normal(SEED, 9810 + k % 997, k)
    bd = dev_u8(block)
    big, reps = tile_rows(bd, synth.row_bytes(k))
    say("large Q4_0 matrix: %d x %d, %.2f GiB, %d repeats of %d rows" % (
        big.shape[0], k, big.numel() / 2**30, reps, P))
    yield k, block, bd, big, reps, x
    del big, bd
    torch.cuda.empty_cache()


def test_gemv(q4_big):
    q4 = lib()
    k, block, bd, big, reps, x = q4_big
    xd = dev_f16(x)
    y_block = q4.q4_0_gemv(bd, xd)
    y_big = q4.q4_0_gemv(big, xd)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemm_rows(block, k, x)
    assert_parity(y_block.cpu().numpy(), y_ref, a_ref, "gemv block k=%d" % k)
    same_bits_tiled(y_big, y_block, reps, "gemv k=%d" % k)


def test_gemv_list(q4_big):
    """The large matrix and its block as one GEMV list: each output equal to its own single call."""
    q4 = lib()
    k, block, bd, big, reps, x = q4_big
    xd = dev_f16(x)
    y_big = torch.full((big.shape[0],), float("nan"), device="cuda")
    y_block = torch.full((P,), float("nan"), device="cuda")
    batch = q4.GemvBatch([(bd, xd, y_block), (big, xd, y_big)])
    batch()
    single = q4.q4_0_gemv(bd, xd)
    torch.cuda.synchronize()
    assert torch.equal(y_block.view(torch.int32), single.view(torch.int32))
    same_bits_tiled(y_big, single, reps, "gemv list k=%d" % k)


def test_lm_head(q4_big):
    """Logits equal to the block's repeated; the token is the first maximum,
    so it lies in the first repeat; the allocation-free entry point agrees."""
    q4 = lib()
    k, block, bd, big, reps, x = q4_big
    xd = dev_f16(x)
    y_block = q4.q4_0_gemv(bd, xd)
    logits, token = q4.lm_head_argmax(big, xd)
    logits2, token2 = q4.lm_head_argmax_noalloc(big, xd)
    torch.cuda.synchronize()
    same_bits_tiled(logits, y_block, reps, "lm head k=%d" % k)
    yb = y_block.cpu().numpy()
    assert int(token.item()) == int(np.argmax(yb)), (int(token.item()), int(np.argmax(yb)))
    assert torch.equal(logits.view(torch.int32), logits2.view(torch.int32))
    assert int(token2.item()) == int(token.item())


@pytest.mark.parametrize("m", [4, 16])
def test_smallm(q4_big, m):
    """M = 4 (LDS ring; k = 32,768 in K-ranges) and M = 16 (register loads)."""
    q4 = lib()
    k, block, bd, big, reps, _ = q4_big
    xm = synth.f16_normal(SEED, 9820 + m, m * k).reshape(m, k)
    xd = dev_f16(xm)
    y_block = q4.q4_0_gemm_smallm(bd, xd)
    y_big = q4.q4_0_gemm_smallm(big, xd)
    torch.cuda.synchronize()
    rows = sampled(P, k + m)
    y_ref, a_ref = oracle.gemm_rows(block[rows], k, xm)
    assert_parity(y_block.cpu().numpy()[:, rows], y_ref, a_ref, "smallm block m=%d k=%d" % (m, k))
    same_bits_tiled(y_big, y_block, reps, "smallm m=%d k=%d" % (m, k))


def test_verify(q4_big):
    """Greedy verify of 4 draft rows over the large vocabulary: logits as the
    block's repeated, each token the first maximum of its row, the whole
    draft accepted when it proposes those tokens."""
    q4 = lib()
    k, block, bd, big, reps, _ = q4_big
    m = 4
    h = synth.f16_normal(SEED, 9830, m * k).reshape(m, k)
    hd = dev_f16(h)
    y_block = q4.q4_0_gemm_smallm(bd, hd)
    torch.cuda.synchronize()
    want = np.argmax(y_block.cpu().numpy(), axis=1).astype(np.int32)
    draft = torch.tensor(want, device="cuda")
    logits, tokens, accepted = q4.lm_head_verify(big, hd, draft)
    torch.cuda.synchronize()
    same_bits_tiled(logits, y_block, reps, "verify k=%d" % k)
    assert np.array_equal(tokens.cpu().numpy(), want)
    assert int(accepted.item()) == m


def test_prefill(q4_big):
    q4 = lib()
    k, block, bd, big, reps, _ = q4_big
    m = 40
    xm = synth.f16_normal(SEED, 9840, m * k).reshape(m, k)
    xd = dev_f16(xm)
    y_block = q4.q4_0_gemm_prefill(bd, xd)
    y_big = q4.q4_0_gemm_prefill(big, xd)
    torch.cuda.synchronize()
    rows = sampled(P, k)
    y_ref, a_ref = oracle.gemm_rows(block[rows], k, xm)
    assert_parity(y_block.cpu().numpy()[:, rows], y_ref, a_ref, "prefill block k=%d" % k)
    same_bits_tiled(y_big, y_block, reps, "prefill k=%d" % k)


def test_q8_slab_engine():
    """Q8_0 at the slab engine's largest k (28,672): 4.1 GiB of weights."""
    q4 = lib()
    k = 28672
    block = synth.q8_0(SEED, 9850, P8, k)
    x = synth.f16_normal(SEED, 9851, k)
    bd, xd = dev_u8(block), dev_f16(x)
    big, reps = tile_rows(bd, q4.q8_row_bytes(k))
    say("large Q8_0 matrix: %d x %d, %.2f GiB" % (big.shape[0], k, big.numel() / 2**30))
    y_block = q4.q8_0_gemv(bd, xd)
    y_big = q4.q8_0_gemv(big, xd)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.q8_gemm_rows(block, k, x)
    assert_parity(y_block.cpu().numpy(), y_ref, a_ref, "q8 block")
    same_bits_tiled(y_big, y_block, reps, "q8 k=%d" % k)
