"""Acceptance interval around the float64 value (test infrastructure; see the package header).

Mechanics follow TensorFold pull request #1123, "What this changes", range-checker bullet:
the two ends of a real interval around the float64 value are rounded to bf16 and an output
is compared with them in value order, -0 below +0; a one-value interval demands the same
bits; NaN matches only NaN; infinities are compared by their bits.

The interval is [x - w, x + w] with half-width (two tiers):

  tier "G" (the parity gate):  w = 2**-8 |x| + (e_P + 2**-16) S
  tier "S" (strict, used to show planted mistakes go red):  w = (e_P + 2**-16) S

  x    the float64 value, S = sum_j p_j |v_j| / l (>= |x|), both from ``attend``;
  e_P  the representation error of P fed to P.V: 0 for fp32 P (decode), and for P as three
       bf16 parts whose sum is fp32's P exactly (TensorFold pull request #1622, review
       answer: the three-part 16-bit split; exact for P >= 2**-110), 2**-16 for P as two
       bf16 halves (Window.p32 bullet: fp32's probabilities to 2**-16), 2**-8 for P as one
       bf16 (the page's gate-4 remark gives P's own bound as 2**-8);
  2**-8 |x|   one bf16 ulp relative to the value;
  2**-16 S    an allowance for fp32 sums, exponentials and the score spread, which carry
              absolute error in proportion to S, not to |x|.

Readings: the page states the mechanics but not a closed form for the fp32 allowance; the
fixed 2**-16 S term is this repository's reading, derived in the design doc.
"""

import numpy as np

from . import bf16

E_P_FP32 = 0.0
E_P_THREE = 0.0
E_P_P32 = 2.0 ** -16
E_P_BF16 = 2.0 ** -8


def half_width(x, S, e_p, tier="G"):
    x = np.asarray(x, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    w = (e_p + 2.0 ** -16) * S
    if tier == "G":
        w = w + 2.0 ** -8 * np.abs(x)
    elif tier != "S":
        raise ValueError(tier)
    return w


def accept(out_bits, x, S, e_p, tier="G"):
    """Boolean array: does each bf16 output lie in its interval?"""
    out = np.asarray(out_bits).astype(np.uint16)
    x = np.asarray(x, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        w = half_width(x, S, e_p, tier)
        lo_b = bf16.to_bf16_bits(x - w)
        hi_b = bf16.to_bf16_bits(x + w)
    k = bf16.order_key(out)
    ok = (k >= bf16.order_key(lo_b)) & (k <= bf16.order_key(hi_b)) & ~bf16.is_nan(out)
    xnan = np.isnan(x)
    xinf = np.isinf(x)
    ok = np.where(xnan, bf16.is_nan(out), ok)
    ok = np.where(xinf, out == bf16.to_bf16_bits(x), ok)
    # a finite x whose interval is not finite (S overflowed): any finite-or-matching output
    wbad = ~xnan & ~xinf & ~np.isfinite(w)
    ok = np.where(wbad, ~bf16.is_nan(out), ok)
    return ok


# The literal one-ulp rule. A value y with |y - x| <= 2**-9 |x| rounds to a bf16 within one
# step of bf16(x), in every binade and at binade edges: the bf16 spacing s next to x is at
# least 2**-8 |x| (2**-133 among subnormals), and from anywhere in the rounding cell of
# r = bf16(x) a move of at most s / 2 ends at or before the neighbour's value. An output
# outside {r and its two neighbours} therefore carries an error above 2**-9 |x|; with the
# error at most (e_P + 2**-16) S (the S term of the half-width), that needs
# |x| < 2**9 (e_P + 2**-16) S: a cancelling output, far below the scale S of its terms.
LITERAL_STEP = 2.0 ** -9


def literal_bound(e_p):
    """Largest |x| / S an output outside the one-step set can have under the S allowance."""
    return (e_p + 2.0 ** -16) / LITERAL_STEP


def literal_stats(out_bits, x):
    """Counts for the literal one-ulp statistic: equal to bf16(x), and within one bf16 step."""
    out = np.asarray(out_bits).astype(np.uint16)
    r = bf16.to_bf16_bits(x)
    fin = np.isfinite(x)
    ko = bf16.order_key(out)
    kr = bf16.order_key(r)
    # neighbours in value order; -0 and +0 are adjacent keys
    eq = (out == r) | (np.isnan(x) & bf16.is_nan(out))
    near = eq | (fin & (np.abs(ko - kr) <= 1) & ~bf16.is_nan(out))
    return {"n": int(out.size), "equal": int(eq.sum()), "within_1ulp": int(near.sum())}


def literal_outside(out_bits, x, S):
    """The outputs outside the one-step set: their count and the largest |x| / S among them
    (0 when there are none)."""
    out = np.asarray(out_bits).astype(np.uint16)
    x = np.asarray(x, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    r = bf16.to_bf16_bits(x)
    eq = (out == r) | (np.isnan(x) & bf16.is_nan(out))
    near = eq | (np.isfinite(x) & (np.abs(bf16.order_key(out) - bf16.order_key(r)) <= 1)
                 & ~bf16.is_nan(out))
    far = ~near
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(S > 0, np.abs(x) / np.where(S > 0, S, 1.0), np.inf)
    worst = float(ratio[far].max()) if far.any() else 0.0
    return int(far.sum()), worst


def report(out_bits, x, S, e_p):
    """Summary dict used by tests and the bench: gate counts and the literal statistic
    (equal to bf16(x), within one step, outside, and the largest |x| / S outside)."""
    g = accept(out_bits, x, S, e_p, "G")
    s = accept(out_bits, x, S, e_p, "S")
    d = literal_stats(out_bits, x)
    outside, worst = literal_outside(out_bits, x, S)
    d.update({"outside": outside, "worst_x_over_S": worst,
              "tier_G_fail": int((~g).sum()), "tier_S_fail": int((~s).sum())})
    return d
