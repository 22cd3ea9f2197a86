"""Float64 oracle of the q/k row preparation on the input side of the attention
(test infrastructure; see the package header).

Two recipes from the pages, each with its rounding points:

  "rope_l2"  TensorFold pull request #1257 ("tf_qk_rows_l2"), "What this changes":
             r = bf16(rope(x)) with fp32 cos/sin of the fp32 angle, then
             n = bf16(l2(r)) with l2(r) = r * (1 / sqrt(sum r^2 + 1e-6)) (eps on the sum),
             then, for q only, q = bf16(qs * n) with an fp32 vector qs.
  "rms_rope" "Exact Numerical Contract" (vortex_exact_attention), "Preparation":
             n = bf16(x / sqrt(mean x^2 + 1e-5)) (per-head RMSNorm, fp32), then
             r = bf16(rope(n)) on the first R dims with bf16 cos/sin coefficients and fp32
             arithmetic; dims R.. pass unrotated.

RoPE is rotate-half (split-half) over the first R dims: for j < R/2, with the pair
(j, j + R/2),  y_j = x_j c_j - x_{j+R/2} s_j,  y_{j+R/2} = x_{j+R/2} c_j + x_j s_j.
Angle (pull request #1257): a_j = fl32(fl32(pos) * inv_j) with the fp32 inverse
inv_j = fl32(theta^(-2j/R)); c_j, s_j are the fp32 cos/sin of a_j (here correctly rounded
from float64, a cosf/sinf within the page's 2 ulp), and bf16(c_j), bf16(s_j) in "rms_rope".

Values are float64 between the rounding points, which are the only places rounding is
taken (to bf16, nearest-even, directly from float64). ``interval`` propagates, stage by
stage, the set of bf16 values a faithful fp32 implementation may produce at each rounding
point, so that a value lying within fp32 error of a bf16 rounding boundary at one stage
is judged correctly at the next: every input of a stage is carried as the real interval
between its lowest and highest allowed bf16 value.

fp32 allowances (this repository's reading; the pages give the rounding points and the
float64 comparison, not a closed form): RoPE 2**-22 (|x_j c| + |x_k s|) (products,
one sum and the coefficients' last bit); the norm factor 2**-20 relative (a fp32 sum of
at most 256 squares, sqrt and reciprocal); the q scale 2**-23 relative.
"""

import numpy as np

from . import bf16

ROPE_L2 = "rope_l2"
RMS_ROPE = "rms_rope"
L2_EPS = 1e-6
RMS_EPS = 1e-5

_W_ROPE = 2.0 ** -22
_W_NORM = 2.0 ** -20
_W_SCALE = 2.0 ** -23


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rope_coeffs(pos, rope_dims, theta):
    """fp32 cos and sin [len(pos), R/2] as float64 values (pull request #1257 angle)."""
    half = rope_dims // 2
    j = np.arange(half, dtype=np.float64)
    inv = _f32(np.power(float(theta), -2.0 * j / rope_dims))           # fp32 inverse
    posf = np.asarray(pos, dtype=np.float64).astype(np.float32)          # fl32(pos)
    ang = (posf[:, None] * inv.astype(np.float32)[None, :]).astype(np.float64)  # fp32 product
    return _f32(np.cos(ang)), _f32(np.sin(ang))


def _rope_point(x, c, s, rope_dims):
    """Rotate-half of x [..., d] (float64) with coefficients [..., R/2]; dims >= R copied."""
    half = rope_dims // 2
    y = x.copy()
    a, b = x[..., :half], x[..., half:rope_dims]
    y[..., :half] = a * c - b * s
    y[..., half:rope_dims] = b * c + a * s
    return y


def _rope_width(x_abs_max, c, s, rope_dims):
    """fp32 allowance of the rotation given |x| bounds."""
    half = rope_dims // 2
    w = np.zeros_like(x_abs_max)
    a, b = x_abs_max[..., :half], x_abs_max[..., half:rope_dims]
    w[..., :half] = _W_ROPE * (a * np.abs(c) + b * np.abs(s))
    w[..., half:rope_dims] = _W_ROPE * (b * np.abs(c) + a * np.abs(s))
    return w


def _round_set(lo, hi):
    """Real interval -> (lowest, highest) allowed bf16 bits."""
    with np.errstate(invalid="ignore", over="ignore"):
        return bf16.to_bf16_bits(lo), bf16.to_bf16_bits(hi)


def _as_interval(lo_b, hi_b):
    return bf16.to_f64(lo_b), bf16.to_f64(hi_b)


def _mul_interval(alo, ahi, blo, bhi):
    """Interval product (all finite)."""
    p = np.stack([alo * blo, alo * bhi, ahi * blo, ahi * bhi])
    return p.min(axis=0), p.max(axis=0)


def _sq_interval(lo, hi):
    """Interval of x^2 for x in [lo, hi]."""
    m = np.minimum(np.abs(lo), np.abs(hi))
    m = np.where((lo <= 0) & (hi >= 0), 0.0, m)
    return m * m, np.maximum(lo * lo, hi * hi)


def point(mode, x_bits, pos, rope_dims, theta, qs=None):
    """The recipe at its rounding points, every rounding taken on the float64 value.
    x_bits uint16 [rows, heads, d]; pos [rows]; qs float32 [d] or None. Returns uint16 bits."""
    x = bf16.to_f64(x_bits)
    d = x.shape[-1]
    c, s = rope_coeffs(pos, rope_dims, theta)
    c, s = c[:, None, :], s[:, None, :]
    if mode == ROPE_L2:
        r = bf16.to_f64(bf16.to_bf16_bits(_rope_point(x, c, s, rope_dims)))
        ssum = (r * r).sum(axis=-1, keepdims=True)
        n_bits = bf16.to_bf16_bits(r / np.sqrt(ssum + _f32(L2_EPS)))
        if qs is None:
            return n_bits
        return bf16.to_bf16_bits(_f32(qs)[None, None, :] * bf16.to_f64(n_bits))
    if mode == RMS_ROPE:
        msq = (x * x).sum(axis=-1, keepdims=True) / d
        n = bf16.to_f64(bf16.to_bf16_bits(x / np.sqrt(msq + _f32(RMS_EPS))))
        cb = bf16.to_f64(bf16.to_bf16_bits(c))
        sb = bf16.to_f64(bf16.to_bf16_bits(s))
        return bf16.to_bf16_bits(_rope_point(n, cb, sb, rope_dims))
    raise ValueError(mode)


def interval(mode, x_bits, pos, rope_dims, theta, qs=None):
    """Lowest and highest allowed bf16 bits of every output (uint16 arrays), propagating
    the allowed sets through the rounding points (finite inputs)."""
    x = bf16.to_f64(x_bits)
    d = x.shape[-1]
    c, s = rope_coeffs(pos, rope_dims, theta)
    c, s = c[:, None, :], s[:, None, :]
    if mode == ROPE_L2:
        y = _rope_point(x, c, s, rope_dims)
        w = _rope_width(np.abs(x), c, s, rope_dims)
        rlo, rhi = _as_interval(*_round_set(y - w, y + w))
        slo, shi = _sq_interval(rlo, rhi)
        eps = _f32(L2_EPS)
        f_lo = 1.0 / np.sqrt(shi.sum(axis=-1, keepdims=True) + eps)
        f_hi = 1.0 / np.sqrt(slo.sum(axis=-1, keepdims=True) + eps)
        nlo, nhi = _mul_interval(rlo, rhi, f_lo, f_hi)
        nlo = nlo - _W_NORM * np.abs(nlo)
        nhi = nhi + _W_NORM * np.abs(nhi)
        lo_b, hi_b = _round_set(nlo, nhi)
        if qs is None:
            return lo_b, hi_b
        q = _f32(qs)[None, None, :]
        a, b = _as_interval(lo_b, hi_b)
        qlo, qhi = _mul_interval(a, b, q, q)
        return _round_set(qlo - _W_SCALE * np.abs(qlo), qhi + _W_SCALE * np.abs(qhi))
    if mode == RMS_ROPE:
        msq = (x * x).sum(axis=-1, keepdims=True) / d
        n = x / np.sqrt(msq + _f32(RMS_EPS))
        nlo, nhi = _as_interval(*_round_set(n - _W_NORM * np.abs(n), n + _W_NORM * np.abs(n)))
        cb = bf16.to_f64(bf16.to_bf16_bits(c))
        sb = bf16.to_f64(bf16.to_bf16_bits(s))
        half = rope_dims // 2
        ylo, yhi = nlo.copy(), nhi.copy()
        alo, ahi = nlo[..., :half], nhi[..., :half]
        blo, bhi = nlo[..., half:rope_dims], nhi[..., half:rope_dims]
        # y_j = a c - b s and y_{j+h} = b c + a s: interval sums of interval products
        p1 = _mul_interval(alo, ahi, cb, cb)
        p2 = _mul_interval(blo, bhi, sb, sb)
        ylo[..., :half], yhi[..., :half] = p1[0] - p2[1], p1[1] - p2[0]
        p3 = _mul_interval(blo, bhi, cb, cb)
        p4 = _mul_interval(alo, ahi, sb, sb)
        ylo[..., half:rope_dims], yhi[..., half:rope_dims] = p3[0] + p4[0], p3[1] + p4[1]
        # bf16 x bf16 products are exact in fp32; the one sum rounds (2**-24 of its size)
        wr = 2.0 ** -23 * np.maximum(np.abs(ylo), np.abs(yhi))
        wr[..., rope_dims:] = 0.0
        return _round_set(ylo - wr, yhi + wr)
    raise ValueError(mode)


def _key0(bits):
    """bf16 value-order key with -0 and +0 taken as one value (the pages fix no sign for
    a zero produced by the preparation)."""
    b = np.asarray(bits).astype(np.uint16)
    return bf16.order_key(np.where(b == 0x8000, np.uint16(0), b))


def accept(out_bits, lo_bits, hi_bits):
    """Boolean array: output inside [lo, hi] in bf16 value order (finite, non-NaN)."""
    k = _key0(out_bits)
    return (k >= _key0(lo_bits)) & (k <= _key0(hi_bits)) & ~bf16.is_nan(out_bits)
