"""Pins for the oracle's float64 -> bf16 rounding.

* float32-representable inputs: torch's float32 -> bfloat16 conversion (RNE) is a library
  routine that must agree bit for bit;
* general float64 inputs: exact rational rounding (fractions), nearest with ties to even;
* signed underflow (TensorFold pull request #1123, first paragraph: an underflow to zero
  keeps its sign), overflow to infinity and NaN.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16


def frac_to_bf16_bits(x):
    """Exact RNE of a float (taken exactly as a rational) to bf16 bits."""
    if x != x:
        return 0x7FC0
    if x in (float("inf"), float("-inf")):
        return 0x7F80 | (0x8000 if x < 0 else 0)
    neg = np.signbit(x)
    F = abs(Fraction(x))
    if F == 0:
        return 0x8000 if neg else 0
    e = F.numerator.bit_length() - F.denominator.bit_length()
    if Fraction(2) ** e > F:
        e -= 1
    quantum = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    t = F / quantum
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** 128:
        mag = 0x7F80
    else:
        mag = struct.unpack("<I", struct.pack("<f", float(r)))[0] >> 16
    return mag | (0x8000 if neg else 0)


def test_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_ties_and_neighbours_float32():
    # exact midpoints between adjacent bf16 values, both parities, plus one f32 ulp either side
    base = np.arange(0, 0x7F7F, 37, dtype=np.uint32) << 16
    mids = (base | 0x8000).view(np.float32)
    for f in (mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))):
        f = f[np.isfinite(f)]
        for s in (f, -f):
            ref = torch.from_numpy(s.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(bf16.to_bf16_bits(s.astype(np.float64)), ref)


def test_float64_values_exact_rationals():
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * np.exp(rng.uniform(-100, 100, 3000)))
    # float64 values a hair off bf16 midpoints (not float32-representable)
    for b in rng.integers(0x0080, 0x7F7F, 500):
        mid = float(struct.unpack("<f", struct.pack("<I", (int(b) << 16) | 0x8000))[0])
        xs += [np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), mid]
    xs += [2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 0.5000001,
           2.0 ** -126 * (1 - 2.0 ** -9), 1e-300, -1e-300, 3.39e38, 3.3961e38, 3.4e38, 1e39,
           -1e39, 0.0, -0.0]
    xs = np.array(xs, dtype=np.float64)
    got = bf16.to_bf16_bits(xs)
    ref = np.array([frac_to_bf16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_signed_underflow_overflow_nan():
    x = np.array([-1e-50, 1e-50, -0.0, 0.0, np.inf, -np.inf, np.nan, -np.nan, 1e40, -1e40])
    b = bf16.to_bf16_bits(x)
    assert list(b[:6]) == [0x8000, 0x0000, 0x8000, 0x0000, 0x7F80, 0xFF80]
    assert bf16.is_nan(b[6]) and bf16.is_nan(b[7])
    assert list(b[8:]) == [0x7F80, 0xFF80]


def test_widening_roundtrip():
    allb = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = bf16.to_f64(allb)
    ok = ~bf16.is_nan(allb)
    assert np.array_equal(bf16.to_bf16_bits(f)[ok], allb[ok])


def test_order_key():
    vals = np.array([-np.inf, -2.0, -1e-40, -0.0, 0.0, 1e-40, 1.0, np.inf])
    b = bf16.to_bf16_bits(vals)
    k = bf16.order_key(b)
    assert np.all(np.diff(k) > 0)
    assert k[3] == -1 and k[4] == 0
