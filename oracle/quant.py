"""Symmetric per-token-per-KV-head quantisation (test infrastructure).

PASK Appendix B.5 gives the low-precision rule for INT4: every token-KV-head
K (and separately V) row gets its own symmetric scale, the maximum absolute
value divided by 7, rounded to FP16 and bounded below by FP16's smallest
positive value; codes are value/scale rounded to the nearest integer and
clipped to [-7, 7]; zero rows get zero codes and unit scale; dequantised
value = code * scale. The int8 tier here is the same rule with 7 -> 127.

Readings where the page is silent: "smallest positive representable value"
is the smallest FP16 subnormal, 2**-24; "rounded to the nearest integer"
breaks ties to even.

INT4 storage (PASK Appendix B.5): two signed nibbles per byte, an odd
dimension padded with a zero code. Read here as: dimension 2i in the low
nibble and 2i+1 in the high nibble of byte i, each nibble the code's 4-bit
two's complement.
"""
import numpy as np

from . import numfmt

FP16_MIN_POSITIVE = 2.0 ** -24


def quantize_row(x, qmax=127):
    """x: [d] float64 (exact widened bf16). Returns (codes int8 [d], scale fp16 bits)."""
    x = np.asarray(x, np.float64)
    amax = np.max(np.abs(x))
    if amax == 0.0:
        return np.zeros(x.shape, np.int8), numfmt.f64_to_fp16_bits(1.0)
    s_bits = numfmt.f64_to_fp16_bits(amax / qmax)
    s = max(numfmt.fp16_bits_to_f64(s_bits), FP16_MIN_POSITIVE)
    s_bits = numfmt.f64_to_fp16_bits(s)
    codes = np.clip(np.rint(x / s), -qmax, qmax).astype(np.int8)
    return codes, s_bits


def quantize_rows(X, qmax=127):
    """X: [n, d] float64 -> (codes [n, d] int8, scales [n] fp16 bits)."""
    X = np.asarray(X, np.float64)
    codes = np.zeros(X.shape, np.int8)
    scales = np.zeros(X.shape[0], np.uint16)
    for t in range(X.shape[0]):
        codes[t], scales[t] = quantize_row(X[t], qmax)
    return codes, scales


def dequantize_rows(codes, scale_bits):
    return np.asarray(codes, np.float64) * numfmt.fp16_bits_to_f64(scale_bits)[:, None]


def pack_nibbles(codes):
    """codes: [..., d] ints in [-8, 7] -> uint8 [..., ceil(d/2)] (zero-padded)."""
    c = np.asarray(codes, np.int64)
    if c.shape[-1] % 2:
        c = np.concatenate([c, np.zeros(c.shape[:-1] + (1,), np.int64)], axis=-1)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, d):
    """uint8 [..., ceil(d/2)] -> int8 codes [..., d]."""
    b = np.asarray(packed, np.int64)
    nib = np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib[..., :d].astype(np.int8)
