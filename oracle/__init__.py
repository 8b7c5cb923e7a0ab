"""CPU oracle for the Q4_0 dequantize-and-multiply path (binary64, plain loops).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the product package never imports
it and shares no code with it.  The arithmetic lives in ``q4_oracle.c`` (the
definition it follows is written out in that file's header); this module only
compiles it with gcc and marshals numpy arrays.

Pinned by ``tests/test_oracle_pins.py`` (hand-computed blocks and final-norm
cases in ``tests/golden/``, exhaustive binary16 decode and binary16 rounding
against numpy, closed forms, exact integer products, brute force on tiny
shapes, argmax invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB = os.path.join(_HERE, "libq4oracle.so")
_lock = threading.Lock()
_default = None

# Per-output tolerance factor: |y_gpu - y| <= TOL * a, a = sum |w_k x_k|.
TOL = 1e-3


def build(force: bool = False) -> str:
    """Compile q4_oracle.c (gcc -O3, OpenMP over outputs, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """The oracle's entry points over one compiled copy of q4_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.q4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.q4o_f16_to_f64.restype = ctypes.c_double
        lib.q4o_f16_to_f64_array.argtypes = [vp, i64, vp]
        lib.q4o_gemm_rows.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        lib.q4o_gemm_rows.restype = ctypes.c_int
        lib.q4o_argmax.argtypes = [vp, i64]
        lib.q4o_argmax.restype = i64
        lib.q4o_accepted_prefix.argtypes = [vp, vp, i64]
        lib.q4o_accepted_prefix.restype = i64
        lib.q4o_f64_to_f16.argtypes = [ctypes.c_double]
        lib.q4o_f64_to_f16.restype = ctypes.c_uint16
        lib.q4o_f64_to_f16_array.argtypes = [vp, i64, vp]
        lib.q4o_rms_norm.argtypes = [vp, vp, i64, ctypes.c_double, vp, vp]
        lib.q4o_gemv_handoff.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        lib.q4o_gemv_handoff.restype = ctypes.c_int
        lib.q4o_q8_gemm_rows.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        lib.q4o_set_threads.argtypes = [ctypes.c_int]
        lib.q4o_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def set_threads(self, n: int) -> int:
        """Team size of the oracle's parallel loops from now on (timing only);
        returns the size in effect."""
        self.lib.q4o_set_threads(int(n))
        return int(self.lib.q4o_threads())

    def threads(self) -> int:
        return int(self.lib.q4o_threads())

    def f16_to_f64(self, bits) -> np.ndarray:
        """Exact binary16 -> binary64 of uint16 bit patterns."""
        b = _f16bits(np.asarray(bits))
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.q4o_f16_to_f64_array(b.ctypes.data, b.size, out.ctypes.data)
        return out

    def gemm_rows(self, w_rows: np.ndarray, k: int, x) -> tuple[np.ndarray, np.ndarray]:
        """(y, a) for packed rows uint8[n, K/32*18] and f16 activations [M, K] (or [K]).

        y[m, i] = sum_k w[i, k] x[m, k] and a[m, i] = sum_k |w[i, k] x[m, k]|, binary64,
        shapes [M, n] (or [n] for a 1-D x).
        """
        assert k % 32 == 0
        w = _u8(w_rows).reshape(-1, k // 32 * 18)
        xb = _f16bits(np.asarray(x))
        one_d = xb.ndim == 1
        xb = np.ascontiguousarray(xb.reshape(-1, k))
        m, n = xb.shape[0], w.shape[0]
        y = np.empty((m, n), dtype=np.float64)
        a = np.empty((m, n), dtype=np.float64)
        if self.lib.q4o_gemm_rows(w.ctypes.data, n, k, xb.ctypes.data, m, y.ctypes.data, a.ctypes.data):
            raise MemoryError("oracle: no memory for the decoded activations")
        if one_d:
            return y[0], a[0]
        return y, a

    def argmax(self, y) -> int:
        """Lowest index among the maxima of a binary64 vector."""
        v = np.ascontiguousarray(np.asarray(y, dtype=np.float64)).ravel()
        assert v.size >= 1
        return int(self.lib.q4o_argmax(v.ctypes.data, v.size))


    def accepted_prefix(self, tokens, draft) -> int:
        """Leading positions where tokens[i] == draft[i] (stops at the first mismatch)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64)).ravel()
        d = np.ascontiguousarray(np.asarray(draft, dtype=np.int64)).ravel()
        assert t.size == d.size
        return int(self.lib.q4o_accepted_prefix(t.ctypes.data, d.ctypes.data, t.size))

    def verify(self, w_rows: np.ndarray, k: int, h, draft):
        """Greedy verify of a draft: (y, a, tokens, accepted) for hidden states h [M, K]
        (f16) and the draft's M tokens: y, a as gemm_rows, tokens[i] = argmax(y[i]),
        accepted = accepted_prefix(tokens, draft)."""
        y, a = self.gemm_rows(w_rows, k, np.asarray(h).reshape(-1, k))
        tokens = np.array([self.argmax(y[i]) for i in range(y.shape[0])], dtype=np.int64)
        return y, a, tokens, self.accepted_prefix(tokens, draft)

    def f64_to_f16(self, v) -> np.ndarray:
        """binary64 -> binary16 bit patterns (uint16), nearest, ties to even."""
        a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.q4o_f64_to_f16_array(a.ctypes.data, a.size, out.ctypes.data)
        return out

    def rms_norm(self, h, g, eps: float) -> tuple[np.ndarray, np.ndarray]:
        """The final norm of one hidden state: (x, v) for f16 h and gain g [K];
        v = h * g / sqrt(mean(h^2) + eps) in binary64, x its binary16 bit patterns."""
        hb = np.ascontiguousarray(_f16bits(np.asarray(h)).ravel())
        gb = np.ascontiguousarray(_f16bits(np.asarray(g)).ravel())
        assert hb.size == gb.size >= 1
        v = np.empty(hb.size, dtype=np.float64)
        x = np.empty(hb.size, dtype=np.uint16)
        self.lib.q4o_rms_norm(hb.ctypes.data, gb.ctypes.data, hb.size, float(eps), v.ctypes.data, x.ctypes.data)
        return x, v

    def lm_head_norm(self, w_rows: np.ndarray, k: int, h, g, eps: float):
        """Final norm, then the LM head: (y, a, token, x) for f16 h and g [K]; x is the
        normed activation (binary16 bits), y, a as gemm_rows on x, token = argmax(y)."""
        x, _ = self.rms_norm(h, g, eps)
        y, a = self.gemm_rows(w_rows, k, x)
        return y, a, self.argmax(y), x

    def q8_gemm_rows(self, w_rows: np.ndarray, k: int, x) -> tuple[np.ndarray, np.ndarray]:
        """(y, a) as gemm_rows, for packed Q8_0 rows uint8[n, K/32*34]."""
        assert k % 32 == 0
        w = _u8(w_rows).reshape(-1, k // 32 * 34)
        xb = _f16bits(np.asarray(x))
        one_d = xb.ndim == 1
        xb = np.ascontiguousarray(xb.reshape(-1, k))
        m, n = xb.shape[0], w.shape[0]
        y = np.empty((m, n), dtype=np.float64)
        a = np.empty((m, n), dtype=np.float64)
        self.lib.q4o_q8_gemm_rows(w.ctypes.data, n, k, xb.ctypes.data, m, y.ctypes.data, a.ctypes.data)
        if one_d:
            return y[0], a[0]
        return y, a

    def gemv_handoff(self, w_rows: np.ndarray, k: int, x, residual=None):
        """The stage hand-off: (h16, y, a) for packed rows [n], f16 x [K] and an optional
        float32 residual [n]: y, a as gemm_rows, h16 = binary16 bits of residual + y."""
        w = _u8(w_rows).reshape(-1, k // 32 * 18)
        xb = np.ascontiguousarray(_f16bits(np.asarray(x)).ravel())
        assert xb.size == k
        n = w.shape[0]
        r = None
        if residual is not None:
            r = np.ascontiguousarray(np.asarray(residual, dtype=np.float32).ravel())
            assert r.size == n
        h16 = np.empty(n, dtype=np.uint16)
        y = np.empty(n, dtype=np.float64)
        a = np.empty(n, dtype=np.float64)
        if self.lib.q4o_gemv_handoff(w.ctypes.data, n, k, xb.ctypes.data, None if r is None else r.ctypes.data,
                                     h16.ctypes.data, y.ctypes.data, a.ctypes.data):
            raise MemoryError("oracle: no memory for the decoded activations")
        return h16, y, a


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())  # rebuilt when the source is newer than the library
    return _default


def f16_to_f64(bits) -> np.ndarray:
    return default().f16_to_f64(bits)


def gemm_rows(w_rows: np.ndarray, k: int, x) -> tuple[np.ndarray, np.ndarray]:
    return default().gemm_rows(w_rows, k, x)


def argmax(y) -> int:
    return default().argmax(y)


def accepted_prefix(tokens, draft) -> int:
    return default().accepted_prefix(tokens, draft)


def verify(w_rows: np.ndarray, k: int, h, draft):
    return default().verify(w_rows, k, h, draft)


def f64_to_f16(v) -> np.ndarray:
    return default().f64_to_f16(v)


def rms_norm(h, g, eps: float):
    return default().rms_norm(h, g, eps)


def lm_head_norm(w_rows: np.ndarray, k: int, h, g, eps: float):
    return default().lm_head_norm(w_rows, k, h, g, eps)


def gemv_handoff(w_rows: np.ndarray, k: int, x, residual=None):
    return default().gemv_handoff(w_rows, k, x, residual)


def q8_gemm_rows(w_rows: np.ndarray, k: int, x) -> tuple[np.ndarray, np.ndarray]:
    return default().q8_gemm_rows(w_rows, k, x)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


def _f16bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16
    return x


def time_gemm_rows(w_rows: np.ndarray, k: int, x) -> float:
    """Wall-clock seconds of one gemm_rows call (used by the CPU baseline)."""
    t0 = time.perf_counter()
    gemm_rows(w_rows, k, x)
    return time.perf_counter() - t0
