"""Exact number-format conversions used by the oracle (test infrastructure).

bf16 is IEEE binary32 with the low 16 bits dropped: 1 sign bit, 8 exponent
bits, 7 stored mantissa bits. Widening is exact. Narrowing from float64 is a
single round-to-nearest-even at the bf16 grid, written out with frexp/rint so
that no intermediate float32 rounding happens.
"""
import numpy as np

BF16_MIN_SUBNORMAL_EXP = -133   # smallest bf16 subnormal is 2**-133
BF16_MIN_NORMAL_EXP = -126


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> bf16 bit patterns, one round-to-nearest-even.

    Normal range: 8 significant bits, so the grid spacing for x = m * 2**e
    (0.5 <= |m| < 1) is 2**(e-8). Below 2**-126 the spacing is fixed at
    2**-133 (bf16 subnormals). Values that round past the largest finite
    bf16 become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = e - 1 >= BF16_MIN_NORMAL_EXP
    q_norm = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    q_sub = np.ldexp(np.rint(np.ldexp(x, -BF16_MIN_SUBNORMAL_EXP)),
                     BF16_MIN_SUBNORMAL_EXP)
    q = np.where(normal, q_norm, q_sub)
    with np.errstate(over="ignore"):
        # q is exactly representable in bf16, hence in float32 (or overflows).
        f32 = q.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def round_bf16(x):
    """float64 -> nearest bf16 value, returned as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def fp16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_fp16_bits(x):
    """float64 -> IEEE binary16 bits, one round-to-nearest-even (numpy's
    float64->float16 cast rounds once, directly from float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
