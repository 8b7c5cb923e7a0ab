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


ALL = [golden_blocks, f16_exhaustive, basis_columns, all_ones, integer_exact,
       brute_force, multi_row_layout, argmax_golden, argmax_invariants, verify_prefix, verify_brute]


def failures(o):
    """Names of the pins the instance fails (an error counts as a failure)."""
    bad = []
    for pin in ALL:
        try:
            pin(o)
        except Exception:  # noqa: BLE001 - any error means the pin did not hold
            bad.append(pin.__name__)
    return bad
