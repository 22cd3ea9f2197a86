"""bf16 rounding for the oracle (test infrastructure; see the package header).

Rounds float64 directly to bf16, round-to-nearest-even, never through float32 (a detour
through float32 is a double rounding that can land on the other neighbour). A value that
underflows to zero keeps its sign (TensorFold pull request #1123, "What this changes",
first paragraph: the bf16 rounding file with the sign fix). Values at or beyond the
overflow threshold become infinities of their sign; NaN stays NaN.

bf16 is float32 with the low 16 mantissa bits dropped: 8 exponent bits (bias 127),
7 stored mantissa bits, subnormals down to 2**-133.
"""

import numpy as np

_MIN_NORMAL_EXP = -126      # smallest normal bf16 is 2**-126
_MANT_BITS = 7              # stored mantissa bits
_QUANTUM_SUB = 2.0 ** -133  # spacing of subnormals (and of the lowest binade)
_TWO_128 = 2.0 ** 128


def to_bf16_bits(x):
    """float64 array -> uint16 bf16 bit patterns, RNE, signed underflow, overflow to inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    ax = np.abs(x)
    nan = np.isnan(x)
    inf = np.isinf(x)
    fin = ~(nan | inf)
    # quantum (spacing of bf16 values) in the binade of |x|
    mant, exp = np.frexp(np.where(fin, ax, 1.0))     # ax = mant * 2**exp, mant in [0.5,1)
    e = exp.astype(np.int64) - 1                     # floor(log2 ax) for ax > 0
    normal = fin & (ax >= 2.0 ** _MIN_NORMAL_EXP)
    quantum = np.where(normal, np.ldexp(1.0, (e - _MANT_BITS).clip(-1074, 1023)), _QUANTUM_SUB)
    # ax / quantum and the product below are exact (powers of two, far from f64 limits)
    q = np.rint(np.where(fin, ax, 0.0) / quantum)    # np.rint rounds half to even
    r = q * quantum
    over = fin & (r >= _TWO_128)
    r = np.where(over | ~fin, 0.0, r)
    # r is an exact bf16 value, hence an exact float32 value: take its top 16 bits
    mag = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mag = np.where(over | inf, np.uint16(0x7F80), mag)
    mag = np.where(nan, np.uint16(0x7FC0), mag)
    out = mag | np.where(sign & ~nan, np.uint16(0x8000), np.uint16(0))
    return out.astype(np.uint16)


def to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact widening)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def order_key(bits):
    """Integer key that sorts bf16 values in value order with -0 below +0 (NaN excluded)."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag - 1, mag)


def is_nan(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
