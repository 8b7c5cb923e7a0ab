"""q4_0_gemv on the GPU against the binary64 oracle, hand-computed blocks and
bit-exact metamorphic relations."""
import numpy as np
import pytest
import torch

import golden_io
import oracle
import q4_encode
import synth
from gpu_util import assert_parity, dev_f16, dev_u8, device, lib, say

pytestmark = pytest.mark.gpu
SEED = synth.DEFAULT_SEED


def run_gemv(w_np, x_np):
    q4 = lib()
    w = dev_u8(w_np)
    x = dev_f16(x_np)
    y = q4.q4_0_gemv(w, x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_golden_blocks():
    for c in golden_io.q4_0_block_cases():
        say("golden", c["name"], c["k"])
        y = run_gemv(c["w"], c["x"])
        assert np.array_equal(y.astype(np.float64), c["y"]), (c["name"], y, c["y"])


def test_golden_blocks_on_fast_path():
    # each 32-wide case doubled into k = 64 (second block all codes 8 -> zero)
    zero_blk = bytes([0x00, 0x3C] + [0x88] * 16)
    for c in golden_io.q4_0_block_cases():
        if c["k"] != 32:
            continue
        w = np.stack([np.frombuffer(bytes(r) + zero_blk, dtype=np.uint8) for r in c["w"]])
        x = np.concatenate([c["x"], np.ones(32, dtype=np.float16)])
        y = run_gemv(w, x)
        assert np.array_equal(y.astype(np.float64), c["y"]), (c["name"], y, c["y"])


SHAPES = [(1, 64), (5, 64), (17, 128), (33, 1088), (64, 1024), (100, 5184), (257, 2048),
          (31, 17408), (1000, 320), (7, 96), (3, 32), (40, 5120 + 32),
          (64, 32768), (333, 20544)]  # activations past the fixed LDS stride (k > 18,432)


@pytest.mark.parametrize("n,k", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_parity_shapes(n, k):
    stream = 1000 + n * 7 + k
    w = synth.q4_0(SEED, stream, n, k)
    x = synth.f16_normal(SEED, stream + 1, k)
    say("gemv parity", n, k)
    y = run_gemv(w, x)
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    assert_parity(y, y_ref, a_ref, "gemv %dx%d" % (n, k))


def test_parity_single_gemv_5120():
    """The single 5120 x 5120 GEMV, every output."""
    n = k = 5120
    w = synth.q4_0(SEED, synth.stream_id(0, 0, 0, synth.T_W), n, k)
    x = synth.f16_normal(SEED, synth.stream_id(0, 0, 0, synth.T_X), k)
    say("gemv parity 5120x5120")
    y = run_gemv(w, x)
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    r = assert_parity(y, y_ref, a_ref, "gemv 5120")
    say("max err/a", r)
    assert r < 1e-5  # f32 blocked sums sit far inside the bound


def test_integer_inputs_exact():
    rng = np.random.default_rng(5)
    n, k = 300, 4096
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    w = q4_encode.encode(codes, np.full((n, k // 32), 0x3C00, dtype=np.uint16))
    xi = rng.integers(-8, 9, size=k)
    y = run_gemv(w, xi.astype(np.float16))
    want = (codes.astype(np.int64) - 8) @ xi
    assert np.array_equal(y.astype(np.int64), want)


def test_zero_rows_and_scales_are_exact_zero():
    rng = np.random.default_rng(6)
    n, k = 64, 1024
    w = synth.q4_0(SEED, 77, n, k).copy()
    blk = w.reshape(n, k // 32, 18)
    blk[0::3, :, 2:] = 0x88          # all codes 8
    blk[1::3, :, 0:2] = 0            # all scales +0
    x = rng.standard_normal(k).astype(np.float16)
    y = run_gemv(w, x)
    assert np.all(y[0::3] == 0) and np.all(y[1::3] == 0)
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    assert_parity(y, y_ref, a_ref)


def test_metamorphic_bit_exact():
    n, k = 1024, 5120
    w = synth.q4_0(SEED, 91, n, k)
    x = synth.f16_normal(SEED, 92, k)
    y = run_gemv(w, x)
    # two runs are identical
    assert np.array_equal(y, run_gemv(w, x))
    # negating x negates y up to the rounding of the f16 dot product, which
    # is not symmetric in sign on MI355X (test_negation_dot2_rounding)
    y_ref, a_ref = oracle.gemm_rows(w, k, x)
    yn = run_gemv(w, -x)
    assert_parity(-yn, y_ref, a_ref, "negated x")
    assert np.all(np.abs(y.astype(np.float64) + yn.astype(np.float64)) <= NEG_BOUND * a_ref)
    # doubling every scale doubles y (scales are normal f16: add one to the exponent)
    w2 = w.copy().reshape(n, k // 32, 18)
    d = (w2[:, :, 0].astype(np.uint16) | (w2[:, :, 1].astype(np.uint16) << 8)) + 0x0400
    w2[:, :, 0] = (d & 0xFF).astype(np.uint8)
    w2[:, :, 1] = (d >> 8).astype(np.uint8)
    assert np.array_equal(run_gemv(w2.reshape(n, -1), x), 2 * y)
    # permuting rows permutes y; duplicated rows give identical outputs
    perm = np.random.default_rng(3).permutation(n)
    assert np.array_equal(run_gemv(w[perm], x), y[perm])
    dup = np.concatenate([np.arange(n), [5, 5, 700, 1023]])
    yd = run_gemv(w[dup], x)
    assert np.array_equal(yd, y[dup])


# |y(x) + y(-x)| <= NEG_BOUND * a.  Binary32 additions, multiplications and
# FMAs round to nearest-even, which commutes with negation; only the f16 dot
# product steps may round a block's partial sum one unit in the last place
# the other way, and the later exact-sign operations carry that difference
# on.  Measured on MI355X: at most 16 units of the result, 2^-28 of a; the
# bound is 256 times that, far below the 1e-3 parity tolerance.
NEG_BOUND = 2.0 ** -20


def test_negation_dot2_rounding():
    """Negating x negates y exactly except where v_dot2_f32_f16 rounds a
    chain step differently for the negated inputs.  On MI355X its rounding
    is not symmetric in sign: a probe of 2^20 chains of 16 steps with
    integer weights in [-8, 7] and normal f16 activations found 206 chains
    whose -x result was not the bit negation of the +x one (one step each,
    one unit in the last place).  Here: 65,536 rows x 5,120 columns; every
    row within NEG_BOUND * a of the negation, and the rows that differ at
    all a small fraction, which is recorded."""
    n, k = 65536, 5120
    w = synth.q4_0(SEED, 12002, n, k)
    x = synth.f16_normal(SEED, 12003, k)
    y = run_gemv(w, x).astype(np.float64)
    yn = run_gemv(w, -x).astype(np.float64)
    diff = np.nonzero(y != -yn)[0]
    say("negation: %d of %d rows not bit-negated; first %s" % (diff.size, n, diff[:8].tolist()))
    # the asymmetry is there (this input shows it on MI355X: 70 rows), and rare
    assert 1 <= diff.size <= n // 100
    if diff.size:
        _, a_ref = oracle.gemm_rows(w[diff], k, x)
        ratio = np.abs(y[diff] + yn[diff]) / a_ref
        say("negation: largest |y(x) + y(-x)| / a = %.3g" % ratio.max())
        assert np.all(ratio <= NEG_BOUND)


def test_alignment_errors():
    q4 = lib()
    k, n = 64, 8
    w = torch.zeros(n * 36 + 16, dtype=torch.uint8, device=device())
    x = torch.zeros(k, dtype=torch.float16, device=device())
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_0_gemv(w[4:4 + n * 36], x)
    assert e.value.status == q4.Q4_ERR_MISALIGNED
    y = q4.q4_0_gemv(w[16:16 + n * 36], x)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
