"""Seeded synthetic inputs for the Q4_0 GEMV workloads.

Input bytes only: packed Q4_0 weight rows and f16 activations, produced by the
counter-based generator in ``gen.c`` (SplitMix64, Steele/Lea/Flood 2014).  Both
the CPU oracle and the GPU path consume what this module writes; this module
contains none of the method's arithmetic (no block decode, no products).

Workload shapes follow the decode engine described on "Every Device Brings a
Slice: How SwarmLLM Runs a 27B Model Across Browser Tabs" (originshq.com),
section "The Architecture: Layers Distributed, Activations in Flight": a
5,120-wide hidden state and 64 transformer layers (62 + 2 in the two-device
benchmark of taozi.news, section "基准成绩").  The per-layer projection shapes
(q/k/v/o 5120x5120, gate/up 17408x5120, down 5120x17408) and the value
distributions (codes uniform on 0..15, scale uniform on [0.001, 0.02], f16
activations N(0,1)) are the synthetic stand-in for the Qwen 27B GGUF file,
which is not available here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

DEFAULT_SEED = 0x51A40000

# Projection order within one layer and the (N, K) of each.
HIDDEN = 5120
FFN = 17408
LAYERS = 64
PROJ = (
    ("q", HIDDEN, HIDDEN),
    ("k", HIDDEN, HIDDEN),
    ("v", HIDDEN, HIDDEN),
    ("o", HIDDEN, HIDDEN),
    ("gate", FFN, HIDDEN),
    ("up", FFN, HIDDEN),
    ("down", HIDDEN, FFN),
)
VOCAB = 151936
# The small dense model the Q8_0 workload is shaped after (Qwen3 4B: hidden
# 2,560, 32 query and 8 key/value heads of 128, MLP 9,728, 36 layers; from
# that model's public configuration, which the pages do not give).
Q8_LAYERS = 36
Q8_PROJ = (
    ("q", 4096, 2560),
    ("k", 1024, 2560),
    ("v", 1024, 2560),
    ("o", 2560, 4096),
    ("gate", 9728, 2560),
    ("up", 9728, 2560),
    ("down", 2560, 9728),
)

# Tensor kinds inside a stream id.
T_W, T_X, T_R = 0, 1, 2  # weights, activations, residual stream


def stream_id(workload: int, layer: int, proj: int, tensor: int) -> int:
    """Stream id of one tensor: workload 0..15, layer 0..4095, proj 0..255, tensor 0..15."""
    return (((workload * 4096 + layer) * 256 + proj) * 16) + tensor


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())  # rebuilt when gen.c is newer than the library
            u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
            lib.synth_f64_to_f16.argtypes = [ctypes.c_double]
            lib.synth_f64_to_f16.restype = ctypes.c_uint16
            lib.synth_f64_to_f16_array.argtypes = [vp, i64, vp]
            lib.synth_u64.argtypes = [u64, u64, u64]
            lib.synth_u64.restype = u64
            lib.synth_q4_0_rows.argtypes = [u64, u64, i64, i64, i64, vp]
            lib.synth_q4_0_row_list.argtypes = [u64, u64, i64, vp, i64, vp]
            lib.synth_f16_normal.argtypes = [u64, u64, i64, i64, vp]
            lib.synth_q8_0_rows.argtypes = [u64, u64, i64, i64, i64, vp]
            _lib = lib
    return _lib


def row_bytes(k: int) -> int:
    """Bytes of one packed row of K columns (K/32 blocks of 18 bytes)."""
    assert k % 32 == 0
    return k // 32 * 18


def f64_to_f16_bits(v) -> np.ndarray:
    """Round doubles to binary16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64)).ravel()
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f64_to_f16_array(a.ctypes.data, a.size, out.ctypes.data)
    return out.reshape(np.shape(v))


def u64(seed: int, stream: int, index: int) -> int:
    return int(_load().synth_u64(seed, stream, index))


def q4_0_rows(seed: int, stream: int, k: int, row_begin: int, row_count: int,
              out: np.ndarray | None = None) -> np.ndarray:
    """Packed Q4_0 rows [row_begin, row_begin+row_count) of a K-column matrix, uint8[rows, K/32*18]."""
    rb = row_bytes(k)
    if out is None:
        out = np.empty((row_count, rb), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == row_count * rb
    _load().synth_q4_0_rows(seed, stream, k, row_begin, row_count, out.ctypes.data)
    return out


def q4_0(seed: int, stream: int, n: int, k: int, out: np.ndarray | None = None) -> np.ndarray:
    """A whole packed Q4_0 matrix of N rows and K columns, uint8[N, K/32*18]."""
    return q4_0_rows(seed, stream, k, 0, n, out)


def q4_0_row_list(seed: int, stream: int, k: int, rows) -> np.ndarray:
    """Arbitrary rows of the same matrix (row ids may repeat), uint8[len(rows), K/32*18]."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((r.size, row_bytes(k)), dtype=np.uint8)
    _load().synth_q4_0_row_list(seed, stream, k, r.ctypes.data, r.size, out.ctypes.data)
    return out


def q8_0_rows(seed: int, stream: int, k: int, row_begin: int, row_count: int) -> np.ndarray:
    """Packed Q8_0 rows [row_begin, row_begin+row_count) of a K-column matrix, uint8[rows, K/32*34]."""
    assert k % 32 == 0
    out = np.empty((row_count, k // 32 * 34), dtype=np.uint8)
    _load().synth_q8_0_rows(seed, stream, k, row_begin, row_count, out.ctypes.data)
    return out


def q8_0(seed: int, stream: int, n: int, k: int) -> np.ndarray:
    """A whole packed Q8_0 matrix of N rows and K columns, uint8[N, K/32*34]."""
    return q8_0_rows(seed, stream, k, 0, n)


def f16_normal(seed: int, stream: int, count: int, begin: int = 0) -> np.ndarray:
    """count f16 N(0,1) values (elements begin.. of the stream), as numpy float16."""
    out = np.empty(count, dtype=np.uint16)
    _load().synth_f16_normal(seed, stream, begin, count, out.ctypes.data)
    return out.view(np.float16)


def f16_scaled_normal(seed: int, stream: int, count: int, scale: float, begin: int = 0) -> np.ndarray:
    """count values scale * z rounded to f16 (z the f16 N(0,1) stream), as numpy float16."""
    z = f16_normal(seed, stream, count, begin).astype(np.float64)
    return f64_to_f16_bits(scale * z).view(np.float16)


def norm_gain(seed: int, stream: int, count: int) -> np.ndarray:
    """count gains of a final norm, 1 + 0.25 z rounded to f16 (z the f16 N(0,1) stream)."""
    z = f16_normal(seed, stream, count).astype(np.float64)
    return f64_to_f16_bits(1.0 + 0.25 * z).view(np.float16)


def decode_sweep():
    """The 448 (layer, proj, N, K) GEMVs of one 64-layer weight sweep, in order."""
    return [(l, p, n, k) for l in range(LAYERS) for p, (_, n, k) in enumerate(PROJ)]


def sweep_weight_bytes() -> int:
    return sum(n * row_bytes(k) for _, _, n, k in decode_sweep())
