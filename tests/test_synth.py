"""The seeded input generator: encoding, determinism, addressability, distributions."""
import numpy as np

import synth


def test_f16_encoder_matches_numpy():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(50000) * 1e-5,            # subnormal range
        rng.uniform(-70000, 70000, 50000),            # overflow boundary
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, np.inf, -np.inf,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.001, 0.02]),
    ])
    got = synth.f64_to_f16_bits(v)
    want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_encoder_ties_to_even_midpoints():
    # every midpoint between consecutive positive finite f16 values
    lo = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    hi = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    assert np.array_equal(synth.f64_to_f16_bits(mid), mid.astype(np.float16).view(np.uint16))


def test_deterministic_and_addressable():
    k = 320
    a = synth.q4_0(7, 3, 40, k)
    b = synth.q4_0(7, 3, 40, k)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.q4_0(8, 3, 40, k))
    assert not np.array_equal(a, synth.q4_0(7, 4, 40, k))
    assert np.array_equal(synth.q4_0_rows(7, 3, k, 13, 9), a[13:22])
    assert np.array_equal(synth.q4_0_row_list(7, 3, k, [39, 0, 5, 5]), a[[39, 0, 5, 5]])
    x = synth.f16_normal(7, 5, 1001)
    assert np.array_equal(x.view(np.uint16), synth.f16_normal(7, 5, 1001).view(np.uint16))
    assert np.array_equal(x[17:500].view(np.uint16), synth.f16_normal(7, 5, 483, begin=17).view(np.uint16))


def test_distributions():
    w = synth.q4_0(1, 2, 512, 1024)
    blk = w.reshape(-1, 18)
    d = (blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)
    assert d.min() >= np.float16(0.001) and d.max() <= np.float16(0.02)
    assert abs(d.mean() - 0.0105) < 2e-4
    codes = np.concatenate([blk[:, 2:] & 15, blk[:, 2:] >> 4]).ravel()
    counts = np.bincount(codes, minlength=16)
    assert counts.size == 16
    assert np.all(np.abs(counts / codes.size - 1 / 16) < 2e-3)
    x = synth.f16_normal(1, 9, 400000).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.01
    assert abs(((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3) < 0.05
    assert np.all(np.isfinite(x))


def test_sweep_shapes():
    sw = synth.decode_sweep()
    assert len(sw) == 448
    assert synth.sweep_weight_bytes() == 13_400_801_280
    assert synth.row_bytes(5120) == 2880 and synth.row_bytes(17408) == 9792


def test_q8_0_rows():
    """Q8_0 bytes: addressable rows, codes over the whole signed byte range, d in [1e-4, 2e-3]."""
    full = synth.q8_0(synth.DEFAULT_SEED, 77, 40, 256)
    assert full.shape == (40, 8 * 34)
    assert np.array_equal(synth.q8_0_rows(synth.DEFAULT_SEED, 77, 256, 13, 5), full[13:18])
    blocks = full.reshape(-1, 34)
    d = blocks[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.0001 - 1e-7 and d.max() <= 0.002 + 1e-6
    codes = blocks[:, 2:].view(np.int8).ravel().astype(np.int64)
    assert codes.min() == -128 and codes.max() == 127
    assert abs(codes.mean()) < 3.0
