"""Pins of the q/k preparation oracle (oracle/prepare.py) to facts that do not come from it.

Sources: TensorFold pull request #1257, "What this changes" (rotate-half RoPE on the bf16
projection rows with the fp32 angle fl32(pos * inv), inv = fp32 1/theta^(2j/d); L2 with eps
on the sum; q scaled by an fp32 vector; bf16 roundings after the rotation, after the
normalisation and after the q scale; the two planted controls that skip one of those
roundings) and the
"Exact Numerical Contract" page, "Preparation" (per-head RMSNorm, eps 1e-5, fp32, rounded
to bf16; split-half RoPE on dims 0-95 with bf16 coefficients and fp32 arithmetic, rounded
to bf16; dims 96-127 unrotated).
"""

import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import bf16, prepare as P

THETA = 10000.0


def _x(rng, shape, scale=1.0):
    return bf16.to_bf16_bits(rng.standard_normal(shape) * scale)


def test_position_zero_is_the_identity_rotation():
    rng = np.random.default_rng(1)
    x = _x(rng, (3, 4, 256))
    c, s = P.rope_coeffs(np.zeros(3, np.int64), 256, THETA)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    # rope_l2 at position 0 is the L2 norm of the projection itself
    xf = bf16.to_f64(x)
    want = bf16.to_bf16_bits(xf / np.sqrt((xf * xf).sum(-1, keepdims=True) + np.float32(1e-6)))
    assert np.array_equal(P.point(P.ROPE_L2, x, np.zeros(3, np.int64), 256, THETA), want)


def test_first_pair_is_a_textbook_rotation_by_pos_radians():
    # inv_0 = theta^0 = 1, so pair (0, R/2) turns by fl32(pos) radians
    for pos in (1, 7, 1000, 199_801, 2 ** 20 + 3):
        c, s = P.rope_coeffs(np.array([pos]), 128, THETA)
        a = float(np.float32(pos))
        assert abs(c[0, 0] - math.cos(a)) <= 2 ** -24 and abs(s[0, 0] - math.sin(a)) <= 2 ** -24


def test_inverse_frequencies_follow_theta_power():
    # angle_j / pos = inv_j = theta^(-2j/R) to fp32 (pos = 1 gives the angle exactly)
    c, s = P.rope_coeffs(np.array([1]), 96, THETA)
    ang = np.arctan2(s[0], c[0])
    j = np.arange(48)
    np.testing.assert_allclose(ang, THETA ** (-2.0 * j / 96), rtol=3e-7, atol=0)


def test_rotation_preserves_pair_norms():
    rng = np.random.default_rng(2)
    x = bf16.to_f64(_x(rng, (50, 2, 128)))
    pos = rng.integers(0, 300_000, 50)
    c, s = P.rope_coeffs(pos, 128, THETA)
    y = P._rope_point(x, c[:, None], s[:, None], 128)
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.all(np.abs(n1 - n0) <= 2 ** -21 * n0 + 1e-300)


def test_constant_heads_normalise_exactly():
    d = 256
    x = bf16.to_bf16_bits(np.full((1, 1, d), 3.0))
    # L2: 3 / sqrt(256 * 9 + 1e-6) = 1/16 * (1 - 2e-11) -> bf16 1/16
    n = P.point(P.ROPE_L2, x, np.array([0]), d, THETA)
    assert np.all(bf16.to_f64(n) == 1.0 / 16)
    # RMS: 3 / sqrt(9 + 1e-5) = 0.99999944 -> bf16 1.0 (pos 0: no rotation)
    n = P.point(P.RMS_ROPE, x, np.array([0]), 96, THETA)
    assert np.all(bf16.to_f64(n) == 1.0)


def test_q_scale_by_power_of_two_is_exact():
    rng = np.random.default_rng(3)
    x = _x(rng, (4, 2, 256))
    pos = np.array([0, 10, 5000, 199_900])
    n = bf16.to_f64(P.point(P.ROPE_L2, x, pos, 256, THETA))
    q = bf16.to_f64(P.point(P.ROPE_L2, x, pos, 256, THETA, qs=np.full(256, 4.0, np.float32)))
    assert np.array_equal(q, 4.0 * n)


def _brute(mode, xbits, pos, R, qs=None):
    """Exact rational evaluation of the recipe for one head, independent of the oracle: the
    fp32 angle and coefficients by exact comparison against 60-digit cos/sin, every sum
    exact, sqrt to 60 digits, every rounding by exact comparison with bf16 neighbours."""
    mpmath.mp.dps = 60
    d = len(xbits)

    def bf16_of(v):
        # exact RNE to bf16 of a rational or mpf, via the two bf16 neighbours
        v = Fraction(v) if not isinstance(v, Fraction) else v
        if v == 0:
            return Fraction(0)
        sgn = 1 if v > 0 else -1
        a = abs(v)
        e = math.floor(math.log2(float(a)))
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        q = Fraction(2) ** (e - 7)
        k = a / q
        fl = math.floor(k)
        r = k - fl
        if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        return sgn * fl * q

    x = [Fraction(float(bf16.to_f64(np.uint16(b)))) for b in xbits]
    half = R // 2
    posf = np.float32(pos)
    coef = []
    for j in range(half):
        inv = np.float32(mpmath.power(THETA, mpmath.mpf(-2 * j) / R))
        ang = float(np.float32(posf * inv))
        cj = mpmath.cos(mpmath.mpf(ang))
        sj = mpmath.sin(mpmath.mpf(ang))
        coef.append((Fraction(float(np.float32(float(cj)))), Fraction(float(np.float32(float(sj))))))

    def rope(v, co):
        y = list(v)
        for j in range(half):
            c, s = co[j]
            y[j] = v[j] * c - v[j + half] * s
            y[j + half] = v[j + half] * c + v[j] * s
        return y

    if mode == P.ROPE_L2:
        r = [bf16_of(t) for t in rope(x, coef)]
        ss = sum(t * t for t in r) + Fraction(float(np.float32(1e-6)))
        f = 1 / mpmath.sqrt(mpmath.mpf(ss.numerator) / ss.denominator)
        n = [bf16_of(Fraction(str(mpmath.mpf(t.numerator) / t.denominator * f))) for t in r]
        if qs is not None:
            n = [bf16_of(Fraction(float(np.float32(qs[i]))) * n[i]) for i in range(d)]
        return n
    msq = sum(t * t for t in x) / d + Fraction(float(np.float32(1e-5)))
    f = 1 / mpmath.sqrt(mpmath.mpf(msq.numerator) / msq.denominator)
    n = [bf16_of(Fraction(str(mpmath.mpf(t.numerator) / t.denominator * f))) for t in x]
    cob = [(bf16_of(c), bf16_of(s)) for c, s in coef]
    return [bf16_of(t) for t in rope(n, cob)]


@pytest.mark.parametrize("mode,d,R", [(P.ROPE_L2, 8, 8), (P.ROPE_L2, 16, 16), (P.RMS_ROPE, 16, 12),
                                      (P.RMS_ROPE, 8, 8)])
def test_brute_force_tiny_heads(mode, d, R):
    rng = np.random.default_rng(d * 7 + R)
    for trial in range(6):
        x = _x(rng, (1, 1, d), scale=rng.uniform(0.3, 3.0))
        pos = int(rng.integers(0, 250_000))
        qs = rng.uniform(0.5, 3.0, d).astype(np.float32) if (mode == P.ROPE_L2 and trial % 2) else None
        got = bf16.to_f64(P.point(mode, x, np.array([pos]), R, THETA, qs=qs))[0, 0]
        want = _brute(mode, x[0, 0], pos, R, qs)
        assert [Fraction(float(g)) for g in got] == want, (mode, trial)


def _controls_red(fn_bad, mode, R, d, qs=None, min_frac=0.05):
    rng = np.random.default_rng(11)
    x = _x(rng, (64, 4, d))
    pos = rng.integers(0, 260_000, 64)
    lo, hi = P.interval(mode, x, pos, R, THETA, qs=qs)
    assert P.accept(P.point(mode, x, pos, R, THETA, qs=qs), lo, hi).all()
    bad = fn_bad(x, pos)
    return (~P.accept(bad, lo, hi)).mean() >= min_frac


def test_controls_dropped_rounding_points_go_red():
    d = R = 256
    qs = np.random.default_rng(5).uniform(0.5, 2.0, d).astype(np.float32)

    def drop_rope(x, pos):            # the rotated head not rounded
        c, s = P.rope_coeffs(pos, R, THETA)
        r = P._rope_point(bf16.to_f64(x), c[:, None], s[:, None], R)
        n = r / np.sqrt((r * r).sum(-1, keepdims=True) + np.float32(1e-6))
        return bf16.to_bf16_bits(qs.astype(np.float64) * bf16.to_f64(bf16.to_bf16_bits(n)))

    def drop_norm(x, pos):            # q's normalized head not rounded
        c, s = P.rope_coeffs(pos, R, THETA)
        r = bf16.to_f64(bf16.to_bf16_bits(P._rope_point(bf16.to_f64(x), c[:, None], s[:, None], R)))
        n = r / np.sqrt((r * r).sum(-1, keepdims=True) + np.float32(1e-6))
        return bf16.to_bf16_bits(qs.astype(np.float64) * n)

    assert _controls_red(drop_rope, P.ROPE_L2, R, d, qs=qs, min_frac=0.002)
    assert _controls_red(drop_norm, P.ROPE_L2, R, d, qs=qs, min_frac=0.05)


def test_controls_wrong_pairing_and_frequencies_go_red():
    d, R = 128, 96

    def interleaved(x, pos):          # pairs (2j, 2j + 1) instead of (j, j + R/2)
        xf = bf16.to_f64(x)
        n = bf16.to_f64(bf16.to_bf16_bits(xf / np.sqrt((xf * xf).mean(-1, keepdims=True) + np.float32(1e-5))))
        c, s = P.rope_coeffs(pos, R, THETA)
        cb = bf16.to_f64(bf16.to_bf16_bits(c))[:, None]
        sb = bf16.to_f64(bf16.to_bf16_bits(s))[:, None]
        y = n.copy()
        a, b = n[..., 0:R:2], n[..., 1:R:2]
        y[..., 0:R:2] = a * cb - b * sb
        y[..., 1:R:2] = b * cb + a * sb
        return bf16.to_bf16_bits(y)

    def full_width_frequencies(x, pos):   # inv = theta^(-2j/d) with d = 128 instead of R = 96
        xf = bf16.to_f64(x)
        n = bf16.to_f64(bf16.to_bf16_bits(xf / np.sqrt((xf * xf).mean(-1, keepdims=True) + np.float32(1e-5))))
        c, s = P.rope_coeffs(pos, 128, THETA)
        cb = bf16.to_f64(bf16.to_bf16_bits(c[:, :48]))[:, None]
        sb = bf16.to_f64(bf16.to_bf16_bits(s[:, :48]))[:, None]
        return bf16.to_bf16_bits(P._rope_point(n, cb, sb, R))

    assert _controls_red(interleaved, P.RMS_ROPE, R, d)
    assert _controls_red(full_width_frequencies, P.RMS_ROPE, R, d)


def test_interval_is_mostly_one_value():
    rng = np.random.default_rng(7)
    x = _x(rng, (32, 8, 256))
    pos = rng.integers(0, 260_000, 32)
    # a general fp32 scale (a scale like 1.5 puts half the products on exact bf16 ties,
    # where both neighbours are correct)
    qs = rng.uniform(0.5, 3.0, 256).astype(np.float32)
    for mode, R, q in ((P.ROPE_L2, 256, qs), (P.ROPE_L2, 256, None), (P.RMS_ROPE, 192, None)):
        lo, hi = P.interval(mode, x, pos, R, THETA, qs=q)
        assert (lo != hi).mean() < 0.01, mode
