"""Test-side ENCODER of packed Q4_0 rows from integer codes and f16 scales.

This is the inverse direction of what the oracle does (it packs, it never
decodes), so that tests can state expected values from the numbers they chose
before packing.  Packing rule (the reading of the format the pages name
"GGUF Q4_0"): bytes 0-1 of a block = f16 scale bits, little-endian; byte 2+j =
code j | code (j+16) << 4.
"""
import numpy as np


def encode(codes: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    """codes uint8[n, K] in 0..15, d_bits uint16[n, K/32] -> uint8[n, K/32*18]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    assert k % 32 == 0 and codes.max(initial=0) <= 15
    nb = k // 32
    d_bits = np.asarray(d_bits, dtype=np.uint16).reshape(n, nb)
    out = np.zeros((n, nb, 18), dtype=np.uint8)
    c = codes.reshape(n, nb, 32)
    out[:, :, 0] = (d_bits & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d_bits >> 8).astype(np.uint8)
    out[:, :, 2:] = c[:, :, :16] | (c[:, :, 16:] << 4)
    return out.reshape(n, nb * 18)


def random_case(rng: np.random.Generator, n: int, k: int, d_lo=0.001, d_hi=0.02, signed_d=False):
    """Random codes, scales (exact f16 values) and packed rows; returns (codes, d, packed)."""
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    d = rng.uniform(d_lo, d_hi, size=(n, k // 32))
    if signed_d:
        d *= rng.choice([-1.0, 1.0], size=d.shape)
    d16 = d.astype(np.float16)
    packed = encode(codes, d16.view(np.uint16))
    return codes, d16.astype(np.float64), packed


def weights_from_numbers(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Dense float64 weights (code - 8) * d from the numbers a test chose (not from bytes)."""
    n, k = codes.shape
    return (codes.astype(np.float64) - 8.0) * np.repeat(d, 32, axis=1).reshape(n, k)


def encode_q8(codes: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    """Q8_0: codes int8[n, K] in -128..127, d_bits uint16[n, K/32] -> uint8[n, K/32*34]
    (bytes 0-1 = f16 scale bits, little-endian; byte 2+j = code j as a two's-complement byte)."""
    codes = np.asarray(codes)
    n, k = codes.shape
    assert k % 32 == 0 and codes.min(initial=0) >= -128 and codes.max(initial=0) <= 127
    nb = k // 32
    d_bits = np.asarray(d_bits, dtype=np.uint16).reshape(n, nb)
    out = np.zeros((n, nb, 34), dtype=np.uint8)
    out[:, :, 0] = (d_bits & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d_bits >> 8).astype(np.uint8)
    out[:, :, 2:] = codes.astype(np.int8).view(np.uint8).reshape(n, nb, 32)
    return out.reshape(n, nb * 34)


def random_case_q8(rng: np.random.Generator, n: int, k: int, d_lo=0.0005, d_hi=0.005):
    """Random Q8_0 codes (-128..127), signed scales (exact f16) and packed rows; (codes, d, packed)."""
    codes = rng.integers(-128, 128, size=(n, k))
    d = rng.uniform(d_lo, d_hi, size=(n, k // 32)) * rng.choice([-1.0, 1.0], size=(n, k // 32))
    d16 = d.astype(np.float16)
    return codes, d16.astype(np.float64), encode_q8(codes, d16.view(np.uint16))


def weights_from_numbers_q8(codes: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Dense float64 Q8_0 weights code * d from the numbers a test chose."""
    n, k = codes.shape
    return codes.astype(np.float64) * np.repeat(d, 32, axis=1).reshape(n, k)
