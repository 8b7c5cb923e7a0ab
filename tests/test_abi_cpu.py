"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (no GPU is touched: every call here fails validation
before anything would be enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import q4_dequant_gemv_block_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4gemv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4.LIB_PATH):
        from q4_dequant_gemv_block_amd import build
        build.build()
    return q4.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"Q4_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for required in ("q4_0_gemv", "q4_0_gemm_smallm", "q4_0_gemm_prefill", "lm_head_argmax"):
        assert required in names
    assert sorted(q4.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", q4.LIB_PATH]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_symbols():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else of ours leaks out with default visibility
    ours = {n for n in exported if n.startswith(("q4", "q8", "lm_head"))}
    assert ours == set(declared_symbols())


def test_abi_version(lib):
    assert lib.q4_abi_version() == 1


def test_workspace_bytes(lib):
    assert lib.q4_workspace_bytes(q4.Q4_OP_GEMV, 1, 5120, 5120) == 0
    assert lib.q4_workspace_bytes(q4.Q4_OP_GEMM_SMALLM, 1, 5120, 5120) == 0
    assert lib.q4_workspace_bytes(q4.Q4_OP_GEMM_SMALLM, 16, 5120, 5120) == 0  # 16 rows of 5120 fit LDS
    assert lib.q4_workspace_bytes(q4.Q4_OP_GEMM_SMALLM, 16, 5120, 17408) > 0
    ws = lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_ARGMAX, 1, 151936, 5120)
    assert ws >= 8 and ws % 8 == 0
    assert lib.q4_workspace_bytes(99, 1, 1, 32) == 0


def test_smallm_k_range_workspace_rule(lib):
    # The activations of one K-range (all M rows) live in the LDS the weights
    # leave free (M <= 7: 160 KiB - 8 waves x 2 slots x 5,376 bytes of weight
    # rings; M > 7: all 160 KiB), in whole 16-pair spans: 128 bytes per pair and row, plus 16
    # bytes per row of padding unless dropping it (the swizzled layout) takes
    # fewer ranges.  A GEMM needs partial sums (nranges x M x N floats) only
    # when its K does not fit one range.
    def expect(m, n, k):
        np_ = k // 64
        # M <= 7: the LDS-ring engine (8 waves x 2 slots x 5,376 bytes of weights)
        row_chunks = (160 * 1024 - (8 * 2 * 5376 if m <= 7 else 0)) // (16 * m)
        fit_pad = max(16, (row_chunks - 1) // 8 // 16 * 16)
        fit_swz = max(16, row_chunks // 8 // 16 * 16)
        fit = fit_swz if -(-np_ // fit_swz) < -(-np_ // fit_pad) else fit_pad
        p = min(fit, (np_ + 15) // 16 * 16)
        nr = -(-np_ // p)
        return nr * m * n * 4 if nr > 1 else 0

    op = q4.Q4_OP_GEMM_SMALLM
    assert lib.q4_workspace_bytes(op, 16, 5120, 5120) == 0  # 16 x 80 pairs x 128 bytes: exactly 160 KiB
    assert lib.q4_workspace_bytes(op, 16, 5120, 17408) == 4 * 16 * 5120 * 4  # 80 + 80 + 80 + 32 pairs
    assert lib.q4_workspace_bytes(op, 4, 5120, 17408) == 2 * 4 * 5120 * 4  # 144 + 128 pairs
    assert lib.q4_workspace_bytes(op, 8, 5120, 5120) == 0
    assert lib.q4_workspace_bytes(op, 2, 5120, 17408) == 0
    for m in (2, 3, 5, 8, 9, 12, 16):
        for k in (64, 1024, 4096, 5120, 13824, 17408, 32768):
            assert lib.q4_workspace_bytes(op, m, 4608, k) == expect(m, 4608, k), (m, k)


def test_gemv_plan_bytes_layout(lib):
    # head (16 bytes) + one 56-byte descriptor per GEMV + 16-byte chunks; the
    # chunks partition the row steps, so there are at least one and at most
    # as many as row steps.
    D = q4.GemvDesc
    for count, n, k in ((1, 8, 64), (3, 5120, 5120), (448, 5120, 5120), (7, 151936, 5120)):
        span = 1 << 32  # larger than any tensor here, so the fake tensors never overlap
        arr = (D * count)(*[D(span * (3 * i + 1), span * (3 * i + 2), span * (3 * i + 3), n, k)
                            for i in range(count)])
        nbytes = lib.q4_0_gemv_batch_plan_bytes(arr, count)
        rest = nbytes - 16 - 56 * count
        assert rest > 0 and rest % 16 == 0, (count, n, k, nbytes)
        assert 1 <= rest // 16 <= count * n


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args, code", [
    ((0, FAKE, FAKE * 4, 8, 64), q4.Q4_ERR_INVALID_ARG),           # null w
    ((FAKE, FAKE * 2, FAKE * 4, 0, 64), q4.Q4_ERR_INVALID_ARG),     # n = 0
    ((FAKE, FAKE * 2, FAKE * 4, 8, 48), q4.Q4_ERR_INVALID_ARG),     # k % 32
    ((FAKE, FAKE * 2, FAKE * 4, 8, 0), q4.Q4_ERR_INVALID_ARG),      # k = 0
    ((FAKE + 4, FAKE * 2, FAKE * 4, 8, 64), q4.Q4_ERR_MISALIGNED),  # w not 16-aligned
    ((FAKE, FAKE * 2 + 8, FAKE * 4, 8, 64), q4.Q4_ERR_MISALIGNED),  # x not 16-aligned
    ((FAKE, FAKE * 2, FAKE * 4 + 2, 8, 64), q4.Q4_ERR_MISALIGNED),  # y not 4-aligned
    ((FAKE, FAKE * 2, FAKE + 16, 8, 64), q4.Q4_ERR_INVALID_ARG),    # y overlaps w
])
def test_gemv_validation(lib, args, code):
    assert lib.q4_0_gemv(*args, None) == code
    assert lib.q4_last_error()


def test_smallm_validation(lib):
    assert lib.q4_0_gemm_smallm(FAKE, FAKE * 2, FAKE * 8, 17, 8, 64, None, 0, None) == q4.Q4_ERR_INVALID_ARG
    assert b"m = 17" in lib.q4_last_error()
    assert lib.q4_0_gemm_smallm(FAKE, FAKE * 2, FAKE * 8, 0, 8, 64, None, 0, None) == q4.Q4_ERR_INVALID_ARG
    need = lib.q4_workspace_bytes(q4.Q4_OP_GEMM_SMALLM, 16, 5120, 17408)  # K split in four ranges
    assert need > 0 and need % 4 == 0
    w, x, y = FAKE * 64, FAKE * 4096, FAKE * 8192
    assert lib.q4_0_gemm_smallm(w, x, y, 16, 5120, 17408, None, 0, None) == q4.Q4_ERR_WORKSPACE
    assert lib.q4_0_gemm_smallm(w, x, y, 16, 5120, 17408, FAKE * 16384, need - 4, None) == q4.Q4_ERR_WORKSPACE
    # workspace overlapping the output
    assert lib.q4_0_gemm_smallm(w, x, y, 16, 5120, 17408, y + 64, need, None) == q4.Q4_ERR_INVALID_ARG


def test_prefill_validation(lib):
    assert lib.q4_0_gemm_prefill(FAKE, FAKE * 2, FAKE * 8, 0, 8, 64, None, 0, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemm_prefill(FAKE, FAKE * 2, FAKE * 8, 4, 8, 40, None, 0, None) == q4.Q4_ERR_INVALID_ARG


def test_prefill_plan_bytes_layout(lib):
    # two 288-byte work heads (the k % 256 == 0 part and the rest: a 32-byte
    # counter block and eight 32-byte per-XCD tile ranges), then one 64-byte
    # descriptor per GEMM
    for count in (1, 2, 7, 448):
        assert lib.q4_0_gemm_prefill_batch_plan_bytes(count) == 2 * 288 + 64 * count
    assert lib.q4_0_gemm_prefill_batch_plan_bytes(0) == 0
    assert lib.q4_0_gemm_prefill_batch_plan_bytes((1 << 20) + 1) == 0


def test_lm_head_validation(lib):
    w, h, lg, tok = FAKE, FAKE * 2, FAKE * 4, FAKE * 8
    need = lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_ARGMAX, 1, 1000, 64)
    assert lib.lm_head_argmax(w, h, lg, tok, 1000, 64, None, 0, None) == q4.Q4_ERR_WORKSPACE
    assert lib.lm_head_argmax(w, h, lg, tok, 1000, 64, FAKE * 16, need - 8, None) == q4.Q4_ERR_WORKSPACE
    assert lib.lm_head_argmax(w, h, lg, 0, 1000, 64, FAKE * 16, need, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.lm_head_argmax(w, h, lg, tok + 2, 1000, 64, FAKE * 16, need, None) == q4.Q4_ERR_MISALIGNED
    # token inside the logits
    assert lib.lm_head_argmax(w, h, lg, lg + 8, 1000, 64, FAKE * 16, need, None) == q4.Q4_ERR_INVALID_ARG
    # k % 64 != 0 is not supported here
    assert lib.lm_head_argmax(w, h, lg, tok, 1000, 96, FAKE * 16, need, None) == q4.Q4_ERR_INVALID_ARG


def test_lm_head_noalloc_validation(lib):
    """The entry point without a workspace refuses bad arguments before it
    looks up its array or launches anything."""
    w, h, lg, tok = FAKE, FAKE * 2, FAKE * 4, FAKE * 8

    def call(w=w, h=h, lg=lg, tok=tok, n=1000, k=64):
        return lib.lm_head_argmax_noalloc(w, h, lg, tok, n, k, None)

    assert call(w=None) == q4.Q4_ERR_INVALID_ARG
    assert call(tok=None) == q4.Q4_ERR_INVALID_ARG
    assert call(tok=tok + 2) == q4.Q4_ERR_MISALIGNED
    assert call(w=w + 4) == q4.Q4_ERR_MISALIGNED
    assert call(tok=lg + 8) == q4.Q4_ERR_INVALID_ARG  # token inside the logits
    assert call(lg=h) == q4.Q4_ERR_INVALID_ARG  # logits over the hidden state
    assert call(k=96) == q4.Q4_ERR_INVALID_ARG
    assert call(k=32768 + 64) == q4.Q4_ERR_INVALID_ARG
    assert call(n=0) == q4.Q4_ERR_INVALID_ARG
    assert b"lm_head_argmax_noalloc" in lib.q4_last_error()


def test_q8_gemv_validation(lib):
    w, x, y = FAKE, FAKE * 2, FAKE * 3
    n, k = 1000, 96

    def call(w=w, x=x, y=y, n=n, k=k):
        return lib.q8_0_gemv(w, x, y, n, k, None)

    assert call(w=None) == q4.Q4_ERR_INVALID_ARG
    assert call(w=w + 2) == q4.Q4_ERR_MISALIGNED
    assert call(x=x + 4) == q4.Q4_ERR_MISALIGNED
    assert call(y=y + 2) == q4.Q4_ERR_MISALIGNED
    assert call(k=80) == q4.Q4_ERR_INVALID_ARG
    assert call(k=32768 + 32) == q4.Q4_ERR_INVALID_ARG
    assert call(n=0) == q4.Q4_ERR_INVALID_ARG
    # y over the weights (1000 rows x 102 bytes) or over x
    assert call(y=w + 100000) == q4.Q4_ERR_INVALID_ARG
    assert call(y=x) == q4.Q4_ERR_INVALID_ARG


def test_q8_batch_validation(lib):
    D = q4.GemvDesc
    plan = q4.Q8Plan()
    assert lib.q8_0_gemv_batch_plan_bytes(None, 0) == 0
    buf = FAKE * 64
    good = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 96), D(FAKE * 8, FAKE * 2, FAKE * 6, 8, 64))
    nbytes = lib.q8_0_gemv_batch_plan_bytes(good, 2)
    assert nbytes >= 2 * 48 + 32
    # the two outputs overlap
    arr = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 96), D(FAKE * 8, FAKE * 2, FAKE * 4 + 16, 8, 64))
    assert lib.q8_0_gemv_batch_plan(arr, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # an output over another descriptor's weights
    arr = (D * 2)(D(FAKE, FAKE * 2, FAKE * 8 + 64, 8, 96), D(FAKE * 8, FAKE * 2, FAKE * 6, 8, 64))
    assert lib.q8_0_gemv_batch_plan(arr, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # k not a multiple of 32, k too large, w misaligned
    for bad in (D(FAKE, FAKE * 2, FAKE * 4, 8, 80), D(FAKE, FAKE * 2, FAKE * 4, 8, 32768 + 32),
                D(FAKE + 2, FAKE * 2, FAKE * 4, 8, 96)):
        arr = (D * 1)(bad)
        assert lib.q8_0_gemv_batch_plan(arr, 1, buf, nbytes, ctypes.byref(plan), None) != q4.Q4_OK
    # plan buffer too small, misaligned, over a tensor; null plan at launch
    assert lib.q8_0_gemv_batch_plan(good, 2, buf, 16, ctypes.byref(plan), None) == q4.Q4_ERR_WORKSPACE
    assert lib.q8_0_gemv_batch_plan(good, 2, buf + 8, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_MISALIGNED
    assert lib.q8_0_gemv_batch_plan(good, 2, FAKE * 4, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q8_0_gemv_batch(None, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q8_0_gemv_batch(ctypes.byref(q4.Q8Plan()), None) == q4.Q4_ERR_INVALID_ARG


def test_q8_batch_splits_by_kernel(lib):
    """A Q8_0 list is split by the kernel a single call would take: k % 512 == 0
    in [2048, 28672] with w 16-byte aligned goes to the slab kernel (the plan's
    first part: a 16-byte head, 72-byte descriptors and 16-byte chunks, its
    size rounded up to 16), the rest to the per-block kernel (second part)."""
    D = q4.GemvDesc
    W, X, Y, W2, X2, Y2 = (FAKE << 12) * 1, (FAKE << 12) * 2, (FAKE << 12) * 3, (FAKE << 12) * 4, (FAKE << 12) * 5, \
        (FAKE << 12) * 6
    slab = D(W, X, Y, 1000, 2560)
    other = [D(W2, X2, Y2, 1000, 96),      # k not a multiple of 512
             D(W2 + 4, X2, Y2, 1000, 2560),  # w 4- but not 16-byte aligned
             D(W2, X2, Y2, 1000, 1536),    # k below 2048
             D(W2, X2, Y2, 10, 29184)]     # k above 28672

    def nbytes(*ds):
        return lib.q8_0_gemv_batch_plan_bytes((D * len(ds))(*ds), len(ds))

    s1 = nbytes(slab)
    assert s1 >= 16 + 72 + 16 and s1 % 16 == 0 and s1 - 16 - 72 - 16 < 16 * 1000  # head, descriptor, chunks; rounded to 16
    for o in other:
        o1 = nbytes(o)
        assert o1 >= 32 + 48 + 16 and (o1 - 32 - 48) % 8 == 0, o1  # head, one descriptor, grid + 1 ranges
        assert nbytes(slab, o) == s1 + o1
    assert nbytes(D(W, X, Y, 1000, 28672)) % 16 == 0  # the largest k on the slab kernel
    assert lib.q4_last_error().decode() == ""


def test_gemv_handoff_validation(lib):
    w, x, r, out = FAKE, FAKE * 2, FAKE * 3, FAKE * 4
    n, k = 1000, 64

    def call(w=w, x=x, r=r, out=out, n=n, k=k):
        return lib.q4_0_gemv_handoff(w, x, r, out, n, k, None)

    assert call(w=None) == q4.Q4_ERR_INVALID_ARG
    assert call(out=None) == q4.Q4_ERR_INVALID_ARG
    assert call(x=x + 8) == q4.Q4_ERR_MISALIGNED
    assert call(out=out + 1) == q4.Q4_ERR_MISALIGNED
    assert call(r=r + 2) == q4.Q4_ERR_MISALIGNED
    assert call(k=96) == q4.Q4_ERR_INVALID_ARG
    assert call(n=0) == q4.Q4_ERR_INVALID_ARG
    # the output over the weights, over x, over the residual
    assert call(out=w + 64) == q4.Q4_ERR_INVALID_ARG
    assert call(out=x) == q4.Q4_ERR_INVALID_ARG
    assert call(out=r + 8) == q4.Q4_ERR_INVALID_ARG
    assert b"overlaps" in lib.q4_last_error()


def test_lm_head_norm_validation(lib):
    w, h, g, lg, tok, xo, ws = FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 8, FAKE * 9, FAKE * 16
    n, k = 1000, 64
    need = lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_NORM_ARGMAX, 1, n, k)
    assert need == lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_ARGMAX, 1, n, k) > 0

    def call(w=w, h=h, g=g, eps=1e-6, lg=lg, tok=tok, xo=xo, n=n, k=k, ws=ws, nb=need):
        return lib.lm_head_norm_argmax(w, h, g, eps, lg, tok, xo, n, k, ws, nb, None)

    assert call(ws=None, nb=0) == q4.Q4_ERR_WORKSPACE
    assert call(nb=need - 8) == q4.Q4_ERR_WORKSPACE
    assert call(ws=ws + 4) == q4.Q4_ERR_MISALIGNED
    assert call(g=None) == q4.Q4_ERR_INVALID_ARG
    assert call(tok=None) == q4.Q4_ERR_INVALID_ARG
    assert call(g=g + 2) == q4.Q4_ERR_MISALIGNED
    assert call(xo=xo + 2) == q4.Q4_ERR_MISALIGNED
    assert call(tok=tok + 2) == q4.Q4_ERR_MISALIGNED
    for bad in (0.0, -1e-6, float("inf"), float("nan")):
        assert call(eps=bad) == q4.Q4_ERR_INVALID_ARG, bad
    assert b"eps" in lib.q4_last_error()
    # x_out over the logits, over gamma, over the token; workspace over gamma; token in the logits
    assert call(xo=lg + 16) == q4.Q4_ERR_INVALID_ARG
    assert call(xo=g) == q4.Q4_ERR_INVALID_ARG
    assert call(tok=xo + 4) == q4.Q4_ERR_INVALID_ARG
    assert call(ws=g) == q4.Q4_ERR_INVALID_ARG
    assert call(tok=lg + 8) == q4.Q4_ERR_INVALID_ARG
    # logits over h
    assert call(lg=h) == q4.Q4_ERR_INVALID_ARG
    # k % 64 != 0 is not supported here; k not a multiple of 32 at all
    assert call(k=96) == q4.Q4_ERR_INVALID_ARG
    assert call(k=80) == q4.Q4_ERR_INVALID_ARG


def test_verify_validation(lib):
    w, h, lg = FAKE * 64, FAKE * 4096, FAKE * 8192
    tok, dr, acc, ws = FAKE * 12288, FAKE * 12289, FAKE * 12290, FAKE * 16384
    n, k = 151936, 5120
    need = lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_VERIFY, 4, n, k)
    assert need >= 4 * 8 and need % 8 == 0
    assert lib.q4_workspace_bytes(q4.Q4_OP_LM_HEAD_VERIFY, 17, n, k) == 0
    ok = (w, h, lg, tok, dr, acc)
    assert lib.lm_head_verify(*ok, 0, n, k, ws, need, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.lm_head_verify(*ok, 17, n, k, ws, need, None) == q4.Q4_ERR_INVALID_ARG
    assert b"m = 17" in lib.q4_last_error()
    assert lib.lm_head_verify(w, h, lg, tok, None, acc, 4, n, k, ws, need, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.lm_head_verify(w, h, lg, tok + 2, dr, acc, 4, n, k, ws, need, None) == q4.Q4_ERR_MISALIGNED
    assert lib.lm_head_verify(*ok, 4, n, k, None, 0, None) == q4.Q4_ERR_WORKSPACE
    assert lib.lm_head_verify(*ok, 4, n, k, ws, need - 8, None) == q4.Q4_ERR_WORKSPACE
    assert lib.lm_head_verify(*ok, 4, n, k, ws + 8, need, None) == q4.Q4_ERR_MISALIGNED
    # accepted inside the tokens, tokens inside the logits, workspace over the draft
    assert lib.lm_head_verify(w, h, lg, tok, dr, tok + 4, 4, n, k, ws, need, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.lm_head_verify(w, h, lg, lg + 64, dr, acc, 4, n, k, ws, need, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.lm_head_verify(w, h, lg, tok, dr, acc, 4, n, k, dr, need, None) == q4.Q4_ERR_INVALID_ARG
    # k % 64 != 0 is not supported here
    assert lib.lm_head_verify(*ok, 4, n, 96, ws, need, None) == q4.Q4_ERR_INVALID_ARG


def test_batch_plan_validation(lib):
    D = q4.GemvDesc
    plan = q4.GemvPlan()
    buf = FAKE * 64
    good = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 2, FAKE * 6, 8, 64))
    nbytes = lib.q4_0_gemv_batch_plan_bytes(good, 2)
    assert nbytes > 0
    # a list the plan would refuse has no size
    arr = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 2, FAKE * 4 + 16, 8, 64))
    assert lib.q4_0_gemv_batch_plan_bytes(arr, 2) == 0
    assert lib.q4_0_gemv_batch_plan_bytes(None, 2) == 0
    # the two outputs overlap
    assert lib.q4_0_gemv_batch_plan(arr, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # k not a multiple of 64
    arr = (D * 1)(D(FAKE, FAKE * 2, FAKE * 4, 8, 96))
    assert lib.q4_0_gemv_batch_plan(arr, 1, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # plan buffer too small, count 0, output overlapping another descriptor's input
    arr = (D * 1)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64))
    assert lib.q4_0_gemv_batch_plan(arr, 1, buf, 1, ctypes.byref(plan), None) == q4.Q4_ERR_WORKSPACE
    assert lib.q4_0_gemv_batch_plan(arr, 0, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    arr = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 4, FAKE * 6, 8, 64))
    assert lib.q4_0_gemv_batch_plan(arr, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # the plan buffer overlapping a tensor
    assert lib.q4_0_gemv_batch_plan(good, 2, FAKE * 8, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # an unfilled plan is refused
    assert lib.q4_0_gemv_batch(ctypes.byref(q4.GemvPlan()), None) == q4.Q4_ERR_INVALID_ARG


def test_smallm_batch_plan_validation(lib):
    D = q4.GemvDesc
    plan = q4.GemmPlan()
    buf = FAKE * 64
    nbytes = lib.q4_0_gemm_smallm_batch_plan_bytes(2)
    assert nbytes > 0 and lib.q4_0_gemm_smallm_batch_plan_bytes(0) == 0
    good = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 2, FAKE * 6, 8, 64))
    # m outside [2, 16]
    for m in (1, 17):
        assert lib.q4_0_gemm_smallm_batch_plan(good, 2, m, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # k not a multiple of 64
    arr = (D * 1)(D(FAKE, FAKE * 2, FAKE * 4, 8, 96))
    assert lib.q4_0_gemm_smallm_batch_plan(arr, 1, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # outputs of m x n floats overlapping (8 x 2 x 4 bytes from FAKE*4 reach FAKE*4 + 64)
    arr = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 2, FAKE * 4 + 32, 8, 64))
    assert lib.q4_0_gemm_smallm_batch_plan(arr, 2, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # plan buffer too small, misaligned, overlapping a tensor
    assert lib.q4_0_gemm_smallm_batch_plan(good, 2, 2, buf, 8, ctypes.byref(plan), None) == q4.Q4_ERR_WORKSPACE
    assert lib.q4_0_gemm_smallm_batch_plan(good, 2, 2, buf + 4, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_MISALIGNED
    assert lib.q4_0_gemm_smallm_batch_plan(good, 2, 2, FAKE * 8, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    # an unfilled plan is refused
    assert lib.q4_0_gemm_smallm_batch(ctypes.byref(q4.GemmPlan()), None, 0, None) == q4.Q4_ERR_INVALID_ARG


def test_prefill_batch_plan_validation(lib):
    D = q4.GemvDesc
    plan = q4.PrefillPlan()
    buf = FAKE * 64
    nbytes = lib.q4_0_gemm_prefill_batch_plan_bytes(2)
    assert nbytes > 0 and lib.q4_0_gemm_prefill_batch_plan_bytes(0) == 0
    good = (D * 2)(D(FAKE, FAKE * 2, FAKE * 4, 8, 64), D(FAKE * 8, FAKE * 2, FAKE * 6, 8, 64))
    assert lib.q4_0_gemm_prefill_batch_plan(good, 2, 0, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    arr = (D * 1)(D(FAKE, FAKE * 2, FAKE * 4, 8, 96))
    assert lib.q4_0_gemm_prefill_batch_plan(arr, 1, 2, buf, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemm_prefill_batch_plan(good, 2, 2, buf, 8, ctypes.byref(plan), None) == q4.Q4_ERR_WORKSPACE
    assert lib.q4_0_gemm_prefill_batch_plan(good, 2, 2, FAKE * 8, nbytes, ctypes.byref(plan), None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemm_prefill_batch(ctypes.byref(q4.PrefillPlan()), None) == q4.Q4_ERR_INVALID_ARG


def test_batch_handoff_validation(lib):
    plan = q4.GemvPlan()
    y = FAKE * 4
    assert lib.q4_0_gemv_batch_handoff(None, y, None, FAKE, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemv_batch_handoff(ctypes.byref(plan), y, None, FAKE, None) == q4.Q4_ERR_INVALID_ARG
    plan.device, plan.count, plan.max_k, plan.grid, plan.nchunks, plan.flags = FAKE * 64, 3, 5120, 256, 300, 0
    assert lib.q4_0_gemv_batch_handoff(ctypes.byref(plan), None, None, FAKE, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemv_batch_handoff(ctypes.byref(plan), y, None, None, None) == q4.Q4_ERR_INVALID_ARG
    assert lib.q4_0_gemv_batch_handoff(ctypes.byref(plan), y, None, FAKE + 1, None) == q4.Q4_ERR_MISALIGNED
    assert lib.q4_0_gemv_batch_handoff(ctypes.byref(plan), y, FAKE + 2, FAKE, None) == q4.Q4_ERR_MISALIGNED


def test_header_is_plain_c(tmp_path):
    """The boundary header compiles as C99 (pedantic), with no C++ or HIP types."""
    src = tmp_path / "use.c"
    src.write_text('#include "q4gemv.h"\nint main(void) { return q4_abi_version() == Q4_ABI_VERSION ? 0 : 1; }\n')
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                           "-I", os.path.dirname(HEADER), str(src)])
