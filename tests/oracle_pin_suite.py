"""Pins of the CPU oracle to facts it does not compute itself.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when the
instance disagrees with a fact fixed by the pages' reading or by mathematics:

  golden_blocks     hand-computed blocks (tests/golden/q4_0_blocks.txt)
  f16_exhaustive    all 65,536 binary16 patterns vs numpy's float16 -> float64
  basis_columns     x = e_k returns column k of W (chosen codes and scales)
  all_ones          x = 1 gives sum_b d_b (sum of the block's codes - 256)
  integer_exact     d = 1 and integer x: the exact int64 matrix product
  brute_force       tiny shapes vs numpy float64 matmul of a dense matrix built
                    from the chosen numbers (not from the bytes)
  multi_row_layout  M x N output layout on a non-square case
  argmax_golden     hand-worked argmax cases (tests/golden/argmax.txt)
  argmax_invariants y[r] >= y[i] for all i, y[r] > y[i] for i < r; numpy.argmax
                    (first occurrence) on random vectors; planted ties
  verify_prefix     hand-worked accepted-prefix cases (first mismatch ends it,
                    later matches do not count)
  verify_brute      greedy verify on tiny shapes: tokens = numpy.argmax of the
                    numpy float64 product of a dense matrix built from the
                    chosen numbers, drafts with a mismatch planted at each row
  f16_round         binary64 -> binary16 against numpy's float16 conversion on
                    every binary16 value, every midpoint between neighbours
                    (ties), one binary64 step either side of each, the
                    overflow threshold and random values across the range
  norm_golden       hand-worked final-norm cases (tests/golden/rms_norm.txt)
  norm_closed_forms constant vectors normalise to +-1; sum of v^2 = K with
                    unit gain; power-of-two scaling of h leaves x unchanged
                    and of g scales v; eps dominates a tiny h
  norm_brute        random h, g, eps against numpy float64 (pairwise mean,
                    numpy sqrt, numpy float16 rounding), lengths 1 to 5120
  lm_head_norm_brute final norm then LM head on tiny shapes: token = numpy.argmax
                    of the dense product with numpy's normed activation
  q8_golden         hand-computed Q8_0 blocks (tests/golden/q8_0_blocks.txt)
  q8_basis_columns  x = e_k returns column k of a Q8_0 matrix (chosen codes)
  q8_integer_exact  Q8_0 with d = 1 and integer x: the exact int64 product
  q8_brute          tiny Q8_0 shapes vs numpy float64 matmul of the dense
                    matrix built from the chosen numbers
  handoff_exact     the stage hand-off with d = 1, integer x and an integer
                    residual: h16 = the exact integer (|value| <= 2048 is exact
                    in binary16), and large sums round to even
  handoff_brute     tiny shapes: h16 = numpy float16 of the numpy float64 dense
                    product plus the float32 residual

``tests/test_oracle_pins.py`` runs them on the oracle; ``tests/test_oracle_mutants.py``
plants plausible mistakes into copies of the oracle's source and checks that
each mutant fails at least one pin.
"""
import numpy as np

import golden_io
import q4_encode


def golden_blocks(o):
    for c in golden_io.q4_0_block_cases():
        y, a = o.gemm_rows(c["w"], c["k"], c["x"])
        assert np.array_equal(y, c["y"]), (c["name"], y, c["y"])
        assert np.array_equal(a, c["a"]), (c["name"], a, c["a"])


def f16_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def basis_columns(o):
    rng = np.random.default_rng(11)
    n, k = 6, 96
    codes, d, w = q4_encode.random_case(rng, n, k, signed_d=True)
    for col in (0, 1, 15, 16, 17, 31, 32, 47, 48, 63, 95):
        x = np.zeros(k, dtype=np.float16)
        x[col] = 1.0
        y, a = o.gemm_rows(w, k, x)
        want = (codes[:, col].astype(np.float64) - 8.0) * d[:, col // 32]
        assert np.array_equal(y, want), (col, y, want)
        assert np.array_equal(a, np.abs(want)), col


def all_ones(o):
    rng = np.random.default_rng(12)
    n, k = 9, 256
    _, _, w = q4_encode.random_case(rng, n, k, signed_d=True)
    x = np.ones(k, dtype=np.float16)
    y, a = o.gemm_rows(w, k, x)
    blk = w.reshape(n, k // 32, 18)
    dd = blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8)
    dd = dd.view(np.float16).astype(np.float64)
    cb = blk[:, :, 2:].astype(np.int64)
    code_sum = (cb & 15).sum(axis=2) + (cb >> 4).sum(axis=2)
    want = (dd * (code_sum - 256)).sum(axis=1)
    assert np.all(np.abs(y - want) <= 1e-12 * a), (y, want)


def integer_exact(o):
    rng = np.random.default_rng(13)
    n, k = 7, 1024
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3C00, dtype=np.uint16)  # 1.0
    w = q4_encode.encode(codes, d_bits)
    xi = rng.integers(-4, 5, size=(3, k))
    y, _ = o.gemm_rows(w, k, xi.astype(np.float16))
    want = xi @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(y, want.astype(np.float64)), (y, want)


def brute_force(o):
    rng = np.random.default_rng(14)
    for n, k, m in ((1, 32, 1), (5, 64, 2), (17, 160, 3), (64, 512, 4), (33, 96, 16)):
        codes, d, w = q4_encode.random_case(rng, n, k, signed_d=True)
        x = rng.standard_normal((m, k)).astype(np.float16)
        dense = q4_encode.weights_from_numbers(codes, d)
        xf = x.astype(np.float64)
        want = xf @ dense.T
        want_a = np.abs(xf) @ np.abs(dense).T
        y, a = o.gemm_rows(w, k, x)
        assert y.shape == (m, n)
        assert np.all(np.abs(y - want) <= 1e-12 * want_a + 1e-300), (n, k, m)
        assert np.all(np.abs(a - want_a) <= 1e-12 * want_a + 1e-300), (n, k, m)


def multi_row_layout(o):
    # rows r carry a single +1 weight (scale 1) at column 2r: y[m, r] = x[m, 2r]
    n, k, m = 5, 32, 3
    codes = np.full((n, k), 8, dtype=np.uint8)
    for r in range(n):
        codes[r, 2 * r] = 9
    w = q4_encode.encode(codes, np.full((n, 1), 0x3C00, dtype=np.uint16))
    x = (np.arange(m * k).reshape(m, k) + 1).astype(np.float16)
    y, _ = o.gemm_rows(w, k, x)
    want = x.astype(np.float64)[:, 0:2 * n:2]
    assert np.array_equal(y, want), (y, want)


def argmax_golden(o):
    for c in golden_io.argmax_cases():
        assert o.argmax(c["y"]) == c["r"], c["name"]


def argmax_invariants(o):
    rng = np.random.default_rng(15)
    for size in (1, 2, 7, 1000, 151936):
        y = rng.standard_normal(size)
        r = o.argmax(y)
        assert np.all(y[r] >= y) and np.all(y[r] > y[:r])
        assert r == int(np.argmax(y))
        # planted tie after the winner: the winner keeps its index
        if size > 2:
            z = y.copy()
            j = int(rng.integers(r + 1, size)) if r + 1 < size else None
            if j is not None:
                z[j] = z[r]
                assert o.argmax(z) == r
            # planted tie before the winner: the earlier index takes over
            if r > 0:
                i = int(rng.integers(0, r))
                z = y.copy()
                z[i] = z[r]
                assert o.argmax(z) == i


def verify_prefix(o):
    cases = [([5, 3, 9, 9], [5, 3, 9, 9], 4), ([5, 3, 9, 9], [5, 3, 1, 9], 2), ([5, 3, 9, 9], [0, 3, 9, 9], 0),
             ([5, 3, 9, 9], [5, 3, 9, 8], 3), ([7], [7], 1), ([7], [6], 0), ([1, 2, 3], [1, 0, 3], 1),
             ([2, 2, 2, 2, 2], [2, 2, 2, 2, 2], 5), ([4, 4], [5, 4], 0)]
    for tokens, draft, want in cases:
        assert o.accepted_prefix(tokens, draft) == want, (tokens, draft)


def verify_brute(o):
    rng = np.random.default_rng(17)
    for m, n, k in ((1, 5, 32), (3, 40, 64), (6, 33, 96), (16, 70, 128)):
        codes, d, w = q4_encode.random_case(rng, n, k, signed_d=True)
        dense = q4_encode.weights_from_numbers(codes, d)  # float64 [n, k] from the chosen numbers
        h = rng.standard_normal((m, k)).astype(np.float16)
        want = np.argmax(h.astype(np.float64) @ dense.T, axis=1)
        for j in range(m + 1):  # mismatch planted at row j (j == m: none)
            draft = want.copy()
            if j < m:
                draft[j] = (draft[j] + 1) % n
            y, a, tokens, accepted = o.verify(w, k, h, draft)
            assert np.array_equal(tokens, want), (m, n, k)
            assert accepted == j, (m, n, k, j)


def f16_round(o):
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # +0 .. 65504
    vals = pos.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in binary64
    top = np.array([65504.0 + 8.0, 65520.0, np.nextafter(65520.0, 0.0), 1e9])  # ties at the top: 65520 -> inf
    rng = np.random.default_rng(23)
    rnd = np.exp2(rng.uniform(-30.0, 17.0, 200000)) * rng.choice([-1.0, 1.0], 200000)
    cand = np.concatenate([vals, -vals, mids, -mids, np.nextafter(mids, 0.0), np.nextafter(mids, np.inf),
                           top, -top, rnd, [0.0, -0.0, np.inf, -np.inf]])
    got = o.f64_to_f16(cand)
    with np.errstate(over="ignore"):
        want = cand.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(cand[i], got[i], want[i]) for i in bad[:5]]
    assert np.isnan(o.f64_to_f16(np.array([np.nan])).view(np.float16)[0])


def norm_golden(o):
    for c in golden_io.rms_norm_cases():
        x, v = o.rms_norm(c["h"], c["g"], c["eps"])
        assert np.array_equal(x, c["x"].view(np.uint16)), (c["name"], x.view(np.float16), c["x"])


def norm_closed_forms(o):
    k = 96
    ones = np.ones(k, dtype=np.float16)
    for c in (1.0, -3.0, 0.0078125, 2.0 ** -20, 60000.0):
        h = np.full(k, c, dtype=np.float16)
        x, v = o.rms_norm(h, ones, 0.0)
        assert np.all(v == np.sign(c)) and np.all(x.view(np.float16) == np.sign(c)), c
    rng = np.random.default_rng(29)
    for k in (1, 5, 64, 1000):
        h = rng.standard_normal(k).astype(np.float16)
        h[0] = 1.5  # not all zero
        g = (1.0 + 0.25 * rng.standard_normal(k)).astype(np.float16)
        x, v = o.rms_norm(h, np.ones(k, dtype=np.float16), 0.0)
        assert abs(np.sum(v * v) / k - 1.0) < 1e-12, k
        for s in (0.5, 2.0, 8.0):  # h stays exact in binary16 when scaled by these
            x2, v2 = o.rms_norm((h.astype(np.float64) * s).astype(np.float16), np.ones(k, dtype=np.float16), 0.0)
            assert np.array_equal(x2, x) and np.allclose(v2, v, rtol=1e-15, atol=0), (k, s)
        _, vg = o.rms_norm(h, g, 0.0)
        _, vg2 = o.rms_norm(h, (g.astype(np.float64) * 4).astype(np.float16), 0.0)
        assert np.array_equal(vg2, 4 * vg), k
        tiny = np.full(k, 2.0 ** -12, dtype=np.float16)
        _, vt = o.rms_norm(tiny, g, 1.0)  # r = 1 / sqrt(2^-24 + 1)
        assert np.allclose(vt, 2.0 ** -12 * g.astype(np.float64) / np.sqrt(1.0 + 2.0 ** -24), rtol=1e-15), k


def _numpy_norm(h, g, eps):
    h64, g64 = h.astype(np.float64), g.astype(np.float64)
    return h64 * g64 / np.sqrt(np.mean(h64 * h64) + eps)


def norm_brute(o):
    rng = np.random.default_rng(31)
    for k in (1, 2, 7, 64, 333, 5120):
        for eps in (float(np.float32(1e-6)), 0.0, 1.0):
            for scale in (1.0, 1e-3, 200.0):
                h = (scale * rng.standard_normal(k)).astype(np.float16)
                h[rng.integers(k)] = np.float16(scale)
                g = (1.0 + 0.25 * rng.standard_normal(k)).astype(np.float16)
                x, v = o.rms_norm(h, g, eps)
                want_v = _numpy_norm(h, g, eps)
                assert np.allclose(v, want_v, rtol=1e-13, atol=0), (k, eps, scale)
                # the two sides sum in different orders, so v may differ in its last
                # bits; none of these seeds puts a v that close to a rounding midpoint
                assert np.array_equal(x, want_v.astype(np.float16).view(np.uint16)), (k, eps, scale)


def lm_head_norm_brute(o):
    rng = np.random.default_rng(37)
    for n, k in ((5, 32), (40, 64), (33, 96), (70, 128)):
        codes, d, w = q4_encode.random_case(rng, n, k, signed_d=True)
        dense = q4_encode.weights_from_numbers(codes, d)
        h = (4.0 * rng.standard_normal(k)).astype(np.float16)
        g = (1.0 + 0.25 * rng.standard_normal(k)).astype(np.float16)
        eps = float(np.float32(1e-6))
        x_np = _numpy_norm(h, g, eps).astype(np.float16)
        y_np = dense @ x_np.astype(np.float64)
        y, a, token, x = o.lm_head_norm(w, k, h, g, eps)
        assert np.array_equal(x, x_np.view(np.uint16)), (n, k)
        assert np.allclose(y, y_np, rtol=1e-12, atol=1e-12), (n, k)
        assert token == int(np.argmax(y_np)), (n, k)


def q8_golden(o):
    for c in golden_io.q8_0_block_cases():
        y, a = o.q8_gemm_rows(c["w"], c["k"], c["x"])
        assert np.array_equal(y, c["y"]), (c["name"], y, c["y"])
        assert np.array_equal(a, c["a"]), (c["name"], a, c["a"])


def q8_basis_columns(o):
    rng = np.random.default_rng(47)
    n, k = 5, 96
    codes, d, w = q4_encode.random_case_q8(rng, n, k)
    for col in (0, 1, 2, 31, 32, 33, 63, 64, 95):
        x = np.zeros(k, dtype=np.float16)
        x[col] = 1.0
        y, a = o.q8_gemm_rows(w, k, x)
        want = codes[:, col].astype(np.float64) * d[:, col // 32]
        assert np.array_equal(y, want), (col, y, want)
        assert np.array_equal(a, np.abs(want)), col


def q8_integer_exact(o):
    rng = np.random.default_rng(53)
    for n, k in ((3, 32), (17, 160), (4, 1024)):
        codes = rng.integers(-128, 128, size=(n, k))
        w = q4_encode.encode_q8(codes, np.full((n, k // 32), 0x3C00, dtype=np.uint16))  # d = 1
        x = rng.integers(-16, 17, size=k).astype(np.float16)
        y, a = o.q8_gemm_rows(w, k, x)
        want = codes @ x.astype(np.int64)
        assert np.array_equal(y, want.astype(np.float64)), (n, k)
        assert np.array_equal(a, (np.abs(codes) @ np.abs(x.astype(np.int64))).astype(np.float64)), (n, k)


def q8_brute(o):
    rng = np.random.default_rng(59)
    for m, n, k in ((1, 5, 32), (3, 40, 64), (2, 33, 96), (4, 70, 128)):
        codes, d, w = q4_encode.random_case_q8(rng, n, k)
        dense = q4_encode.weights_from_numbers_q8(codes, d)
        x = rng.standard_normal((m, k)).astype(np.float16)
        y, a = o.q8_gemm_rows(w, k, x)
        want = x.astype(np.float64) @ dense.T
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12), (m, n, k)
        assert np.allclose(a, np.abs(x.astype(np.float64)) @ np.abs(dense).T, rtol=1e-12, atol=0), (m, n, k)


def handoff_exact(o):
    rng = np.random.default_rng(41)
    for n, k in ((7, 32), (33, 96)):
        codes = rng.integers(0, 16, size=(n, k))
        w = q4_encode.encode(codes, np.full((n, k // 32), 0x3C00, dtype=np.uint16))  # d = 1
        x = rng.integers(-3, 4, size=k).astype(np.float16)
        exact = (codes - 8) @ x.astype(np.int64)
        res = rng.integers(-500, 500, size=n).astype(np.float32)
        h16, y, a = o.gemv_handoff(w, k, x, res)
        assert np.array_equal(y, exact.astype(np.float64)), (n, k)
        want = exact + res.astype(np.int64)
        assert np.all(np.abs(want) <= 2048)
        assert np.array_equal(h16.view(np.float16).astype(np.float64), want.astype(np.float64)), (n, k)
        h0, _, _ = o.gemv_handoff(w, k, x)
        assert np.array_equal(h0.view(np.float16).astype(np.float64), exact.astype(np.float64)), (n, k)
    # one row, K = 32, every code 15 (weight 7), d = 1, x = 1: y = 224; residual 2048 - 224 + 1 -> 2049,
    # a tie between 2048 and 2050 in binary16 (spacing 2 above 2048): even mantissa -> 2048
    w = q4_encode.encode(np.full((1, 32), 15), np.full((1, 1), 0x3C00, dtype=np.uint16))
    h16, y, _ = o.gemv_handoff(w, 32, np.ones(32, dtype=np.float16), np.array([1825.0], dtype=np.float32))
    assert y[0] == 224.0 and h16.view(np.float16)[0] == 2048.0
    h16, _, _ = o.gemv_handoff(w, 32, np.ones(32, dtype=np.float16), np.array([1827.0], dtype=np.float32))
    assert h16.view(np.float16)[0] == 2052.0  # 2051: tie between 2050 and 2052 -> 2052 (even)


def handoff_brute(o):
    rng = np.random.default_rng(43)
    for n, k in ((5, 32), (40, 64), (70, 128)):
        codes, d, w = q4_encode.random_case(rng, n, k, signed_d=True)
        dense = q4_encode.weights_from_numbers(codes, d)
        x = rng.standard_normal(k).astype(np.float16)
        res = (3.0 * rng.standard_normal(n)).astype(np.float32)
        want = (dense @ x.astype(np.float64) + res.astype(np.float64)).astype(np.float16)
        h16, y, a = o.gemv_handoff(w, k, x, res)
        assert np.array_equal(h16, want.view(np.uint16)), (n, k)


ALL = [golden_blocks, f16_exhaustive, basis_columns, all_ones, integer_exact,
       brute_force, multi_row_layout, argmax_golden, argmax_invariants, verify_prefix, verify_brute,
       f16_round, norm_golden, norm_closed_forms, norm_brute, lm_head_norm_brute, handoff_exact, handoff_brute,
       q8_golden, q8_basis_columns, q8_integer_exact, q8_brute]


def failures(o):
    """Names of the pins the instance fails (an error counts as a failure)."""
    bad = []
    for pin in ALL:
        try:
            pin(o)
        except Exception:  # noqa: BLE001 - any error means the pin did not hold
            bad.append(pin.__name__)
    return bad
