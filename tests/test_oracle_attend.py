"""Pins for the float64 attention oracle, independent of the oracle's own code.

* brute force on tiny inputs: key visibility by enumerating a per-key predicate, q . k as
  exact rationals (bf16 values are dyadic), exp and division in 60-digit mpmath, exact
  rational rounding to bf16;
* closed forms: a one-key row returns v bit for bit; equal scores give the exact mean of
  integer values; a key whose score leads by >= 200 returns its v;
* invariants: batch, stream slot, declared cache length and prompt chunking do not change a
  row (TensorFold pull request #1123, "Receipt", exactness bullet);
* non-finite classes for the page's gate-1 plants ("Receipt", kernel-contract bullet).
"""

from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import attend, bf16
from sliding_window_gqa_amd import workloads

mpmath.mp.dps = 60


def rand_bf16(rng, shape, scale=1.0):
    return workloads._bf16_bits(rng.standard_normal(shape) * scale)


def brute_row_head(q, kc, vc, t, pos, last, win, ring, h, scale):
    """One (row, head) by enumeration and exact arithmetic. Returns (x as mpf list, bits)."""
    Hq, d = q.shape
    G = Hq // kc.shape[2]
    g = h // G
    keys = [j for j in range(0, last + 1) if win == 0 or j > pos - win]
    qf = [Fraction(float(v)) for v in bf16.to_f64(q[h])]
    c = Fraction(float(np.float32(scale)))
    s = []
    for j in keys:
        kf = bf16.to_f64(kc[t, j % ring, g])
        s.append(c * sum(a * Fraction(float(b)) for a, b in zip(qf, kf)))
    m = max(s)
    p = [mpmath.exp(mpmath.mpf(sj.numerator) / sj.denominator - mpmath.mpf(m.numerator) / m.denominator)
         for sj in s]
    l = mpmath.fsum(p)
    xs = []
    for dd in range(d):
        num = mpmath.fsum(pj * mpmath.mpf(float(bf16.to_f64(vc[t, j % ring, g, dd])))
                          for pj, j in zip(p, keys))
        xs.append(num / l)
    return xs


def mpf_to_bits(x):
    # the mpf carries ~200 bits; Fraction of it is exact, then exact RNE
    man, exp = mpmath.frexp(x)
    f = Fraction(int(man * 2**200)) * Fraction(2) ** (int(exp) - 200)
    return f


def rational_bits(F):
    if F == 0:
        return 0, False
    neg = F < 0
    F = abs(F)
    e = F.numerator.bit_length() - F.denominator.bit_length()
    if Fraction(2) ** e > F:
        e -= 1
    quantum = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    t = F / quantum
    fl = t.numerator // t.denominator
    rem = t - fl
    near_mid = abs(rem - Fraction(1, 2)) < Fraction(1, 2**40)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    import struct
    mag = struct.unpack("<I", struct.pack("<f", float(fl * quantum)))[0] >> 16
    return (mag | (0x8000 if neg else 0)), near_mid


CASES = [
    # (d, Hq, Hkv, win, ring, streams, positions)
    (4, 2, 1, 3, 7, 1, [0, 2, 6, 9]),
    (8, 4, 2, 5, 5, 2, [4, 11, 3]),
    (8, 3, 1, 0, 40, 1, [0, 17, 39]),
    (16, 4, 4, 40, 64, 1, [63, 100]),
    (16, 8, 2, 1, 9, 3, [5, 0, 30]),
    (256, 2, 1, 12, 16, 1, [40]),
]


@pytest.mark.parametrize("d,Hq,Hkv,win,ring,S,positions", CASES)
def test_decode_matches_brute_force(d, Hq, Hkv, win, ring, S, positions):
    rng = np.random.default_rng(d * 1000 + Hq * 10 + win)
    R = len(positions)
    q = rand_bf16(rng, (R, Hq, d))
    kc = rand_bf16(rng, (S, ring, Hkv, d), 0.5)
    vc = rand_bf16(rng, (S, ring, Hkv, d))
    stream = np.arange(R) % S
    pos = np.array(positions)
    scale = 0.7 if d < 256 else 0.125
    x, Sx, out = attend.decode(q, kc, vc, stream, pos, win, ring, scale)
    for r in range(R):
        for h in range(Hq):
            xs = brute_row_head(q[r], kc, vc, stream[r], int(pos[r]), int(pos[r]), win, ring, h, scale)
            for dd in range(d):
                F = mpf_to_bits(xs[dd])
                bits, near = rational_bits(F)
                assert abs(x[r, h, dd] - float(xs[dd])) <= 1e-13 * max(1.0, Sx[r, h, dd])
                if not near:
                    assert out[r, h, dd] == bits, (r, h, dd)


def test_prompt_with_hi_matches_brute_force():
    rng = np.random.default_rng(77)
    n, Hq, Hkv, d, p0, win, ring = 9, 4, 2, 8, 5, 4, 11
    q = rand_bf16(rng, (n, Hq, d))
    kr = rand_bf16(rng, (ring, Hkv, d), 0.5)
    vr = rand_bf16(rng, (ring, Hkv, d))
    hi = p0 + np.arange(n)
    hi[2:6] = p0 + 5                       # an image span: rows 2..5 see each other
    x, Sx, out = attend.prompt(q, kr, vr, p0, win, ring, 0.9, hi=hi)
    for i in range(n):
        for h in range(Hq):
            xs = brute_row_head(q[i], kr[None], vr[None], 0, p0 + i, int(hi[i]), win, ring, h, 0.9)
            for dd in range(d):
                bits, near = rational_bits(mpf_to_bits(xs[dd]))
                assert abs(x[i, h, dd] - float(xs[dd])) <= 1e-13 * max(1.0, Sx[i, h, dd])
                if not near:
                    assert out[i, h, dd] == bits


def test_window_edges_from_the_workloads():
    # tiny decode: window 64 at position 299 sees keys 236..299, chunks 0 and 1
    assert attend.key_window(299, 64) == (236, 299)
    assert attend.chunk_range(299, 64) == (0, 1)
    assert 256 - 236 == 20 and 299 - 256 + 1 == 44
    # image rows 40..300 of the 12B prompt at p0 5000 see 1024..1284 keys
    lo, last = attend.key_window(5040, 1024, 5300)
    assert last - lo + 1 == 1284
    lo, last = attend.key_window(5300, 1024, 5300)
    assert last - lo + 1 == 1024
    # window 0: every key from 0
    assert attend.key_window(17, 0) == (0, 17)
    # early rows clamp at key 0
    assert attend.key_window(5, 1024) == (0, 5)


def test_one_key_row_returns_v():
    rng = np.random.default_rng(3)
    q = rand_bf16(rng, (2, 4, 256))
    kc = rand_bf16(rng, (1, 10, 2, 256))
    vc = rand_bf16(rng, (1, 10, 2, 256))
    # window 1, or position 0: exactly one visible key
    x, S, out = attend.decode(q, kc, vc, np.zeros(2, int), np.array([7, 0]), 1, 10, 1.0)
    assert np.array_equal(out[0, 0], vc[0, 7, 0]) and np.array_equal(out[0, 3], vc[0, 7, 1])
    assert np.array_equal(out[1, 1], vc[0, 0, 0])


def test_equal_scores_give_exact_integer_mean():
    # q = 0: every weight is exactly 1, so x is the plain mean of the visible values
    d, n = 256, 64
    rng = np.random.default_rng(4)
    vals = rng.integers(-128, 129, size=(n, d)).astype(np.float64)
    vals[:, :8] = np.where(np.arange(n)[:, None] % 2 == 0, 3072.0, -2048.0)
    vc = workloads._bf16_bits(vals)[None, :, None, :]
    assert np.array_equal(bf16.to_f64(vc[0, :, 0]), vals)      # integers exact in bf16
    q = np.zeros((1, 1, d), dtype=np.uint16)
    kc = rand_bf16(rng, (1, n, 1, d))
    x, S, out = attend.decode(q, kc, vc, [0], [n - 1], 0, n, 1.0)
    mean = np.array([sum(Fraction(int(v)) for v in col) / n for col in vals.T])
    assert all(Fraction(float(a)) == b for a, b in zip(x[0, 0], mean))
    assert (x[0, 0, :8] == 512.0).all()


def test_peaked_key_returns_its_v():
    rng = np.random.default_rng(5)
    d, n = 256, 50
    q = rand_bf16(rng, (1, 2, d))
    kc = workloads._bf16_bits(rng.standard_normal((1, n, 1, d)) * 0.01)
    qf = bf16.to_f64(q[0, 1])
    kc[0, 30, 0] = workloads._bf16_bits(qf * (250.0 / (qf @ qf)))   # score ~250 vs ~0
    vc = rand_bf16(rng, (1, n, 1, d))
    x, S, out = attend.decode(q, kc, vc, [0], [49], 0, n, 1.0)
    assert np.array_equal(out[0, 1], vc[0, 30, 0])


def test_invariants_batch_stream_cache_length_chunking():
    rng = np.random.default_rng(6)
    Hq, Hkv, d, win, ring = 4, 2, 16, 24, 40
    q = rand_bf16(rng, (5, Hq, d))
    kc = rand_bf16(rng, (2, ring, Hkv, d))
    vc = rand_bf16(rng, (2, ring, Hkv, d))
    pos = np.array([3, 77, 39, 120, 41])
    st = np.array([0, 1, 1, 0, 1])
    _, _, full = attend.decode(q, kc, vc, st, pos, win, ring, 1.0)
    # alone
    _, _, one = attend.decode(q[3:4], kc, vc, st[3:4], pos[3:4], win, ring, 1.0)
    assert np.array_equal(one[0], full[3])
    # another stream slot holding the same ring
    kc2 = np.stack([kc[1], kc[0]])
    vc2 = np.stack([vc[1], vc[0]])
    _, _, swp = attend.decode(q, kc2, vc2, 1 - st, pos, win, ring, 1.0)
    assert np.array_equal(swp, full)
    # a linear cache declared 16x longer (window 0 reading keys 0..pos)
    lin_k = rand_bf16(rng, (1, 16 * 50, Hkv, d))
    lin_v = rand_bf16(rng, (1, 16 * 50, Hkv, d))
    a = attend.decode(q[:1], lin_k[:, :50], lin_v[:, :50], [0], [30], 0, 50, 1.0)[2]
    b = attend.decode(q[:1], lin_k, lin_v, [0], [30], 0, 16 * 50, 1.0)[2]
    assert np.array_equal(a, b)
    # cutting a prompt into two calls leaves each row's bits unchanged
    n, p0 = 12, 30
    qp = rand_bf16(rng, (n, Hq, d))
    whole = attend.prompt(qp, kc[0], vc[0], p0, win, ring, 1.0)[2]
    for cut in (1, 5, 11):
        first = attend.prompt(qp[:cut], kc[0], vc[0], p0, win, ring, 1.0)[2]
        second = attend.prompt(qp[cut:], kc[0], vc[0], p0 + cut, win, ring, 1.0)[2]
        assert np.array_equal(np.concatenate([first, second]), whole)


def _nonfinite_setup():
    rng = np.random.default_rng(8)
    Hq, Hkv, d, ring = 4, 2, 8, 32
    q = rand_bf16(rng, (4, Hq, d))
    kc = rand_bf16(rng, (1, ring, Hkv, d), 0.3)
    vc = rand_bf16(rng, (1, ring, Hkv, d))
    return q, kc, vc, np.zeros(4, int), np.array([10, 11, 12, 20]), 4, ring


NAN = 0x7FC0
PINF = 0x7F80
NINF = 0xFF80


def test_nonfinite_nan_query():
    q, kc, vc, st, pos, win, ring = _nonfinite_setup()
    q[1, 2, 3] = NAN
    x = attend.decode(q, kc, vc, st, pos, win, ring, 1.0)[0]
    assert np.isnan(x[1, 2]).all()
    assert np.isfinite(np.delete(x.reshape(16, -1), 1 * 4 + 2, axis=0)).all()


def test_nonfinite_nan_key_reaches_only_rows_that_see_it():
    q, kc, vc, st, pos, win, ring = _nonfinite_setup()
    kc[0, 12, 1, 0] = NAN                       # key 12, key head 1 (query heads 2, 3)
    x = attend.decode(q, kc, vc, st, pos, win, ring, 1.0)[0]
    for r, p in enumerate(pos):
        sees = p - win < 12 <= p
        assert np.isnan(x[r, 2:4]).all() == sees
        assert np.isfinite(x[r, 0:2]).all()
        if not sees:
            assert np.isfinite(x[r, 2:4]).all()


def test_nonfinite_inf_value_seen_by_later_rows():
    q, kc, vc, st, pos, win, ring = _nonfinite_setup()
    vc[0, 12, 0, 5] = PINF                      # only rows at 12 and above (window 4) see key 12
    x = attend.decode(q, kc, vc, st, pos, win, ring, 1.0)[0]
    assert np.isfinite(x[0]).all() and np.isfinite(x[1]).all()
    assert (x[2, 0:2, 5] == np.inf).all()
    mask = np.ones_like(x[2], bool)
    mask[0:2, 5] = False
    assert np.isfinite(x[2][mask]).all() and np.isfinite(x[3]).all()


def test_nonfinite_opposite_infinities_make_nan():
    q, kc, vc, st, pos, win, ring = _nonfinite_setup()
    vc[0, 9, 1, 2] = PINF
    vc[0, 10, 1, 2] = NINF
    x = attend.decode(q, kc, vc, st, pos, win, ring, 1.0)[0]
    assert np.isnan(x[0, 2:4, 2]).all()         # the row at 10 sees keys 7..10


def test_nonfinite_inf_at_a_negligible_key_stays_inf():
    # float64's weight e^-200 is tiny but nonzero, so +inf * e^-200 = +inf (fp32 would make 0)
    d, ring = 8, 16
    q = np.zeros((1, 1, d), np.uint16)
    q[0, 0] = workloads._bf16_bits(np.full(d, 1.0))
    kc = np.zeros((1, ring, 1, d), np.uint16)
    kc[0, 3, 0] = workloads._bf16_bits(np.full(d, 25.0))    # score 200
    kc[0, 4, 0] = workloads._bf16_bits(np.full(d, 0.0))     # score 0: weight e^-200
    vc = workloads._bf16_bits(np.ones((1, ring, 1, d)))
    vc[0, 4, 0, 1] = PINF
    x = attend.decode(q, kc, vc, [0], [4], 2, ring, 1.0)[0]
    assert x[0, 0, 1] == np.inf
    assert (x[0, 0, [0, 2, 3]] == 1.0).all()


def test_planted_mistakes_fail_the_brute_force():
    """A window one key too wide, or a transposed head map, makes the brute-force check fail."""
    rng = np.random.default_rng(9)
    d, Hq, Hkv, win, ring = 8, 4, 2, 3, 9
    q = rand_bf16(rng, (1, Hq, d))
    kc = rand_bf16(rng, (1, ring, Hkv, d), 0.5)
    vc = rand_bf16(rng, (1, ring, Hkv, d))
    xs = [brute_row_head(q[0], kc, vc, 0, 6, 6, win, ring, h, 1.0) for h in range(Hq)]
    ref = np.array([[float(v) for v in row] for row in xs])
    good = attend.decode(q, kc, vc, [0], [6], win, ring, 1.0)[0][0]
    assert np.allclose(good, ref, rtol=0, atol=1e-13)
    wide = attend.decode(q, kc, vc, [0], [6], win + 1, ring, 1.0)[0][0]
    assert not np.allclose(wide, ref, rtol=0, atol=1e-6)
    # heads mapped h -> h % Hkv instead of h // G
    perm = q[:, [0, 2, 1, 3]]
    swapped = attend.decode(perm, kc, vc, [0], [6], win, ring, 1.0)[0][0][[0, 2, 1, 3]]
    assert not np.allclose(swapped, ref, rtol=0, atol=1e-6)
