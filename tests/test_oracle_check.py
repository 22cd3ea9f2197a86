"""Pins for the acceptance interval (``oracle.check``).

* the mechanics of TensorFold pull request #1123's range-checker bullet: value order with
  -0 below +0, a one-value interval demands the same bits, NaN matches only NaN,
  infinities compare by bits;
* discrimination, after the page's planted controls ("Receipt", kernel-contract bullet): a
  float32 emulation of chunked decode with an ordered merge passes the strict tier, while
  the same emulation with one planted mistake (window one key early, merge without
  exp(m_c - M), merge rounding toward zero, P rounded to one bf16 under the p32 interval)
  fails it; P as three bf16 parts passes the strict interval of fp32 P. The emulation is
  CPU test code built from numpy float32 steps.
* the three-part split (TensorFold pull request #1622, review answer): nearest-even bf16
  parts of fp32 values sum back exactly down to 2**-110, checked with torch's conversion.
"""

import numpy as np
import pytest

from oracle import attend, bf16, check
from sliding_window_gqa_amd import workloads


def b(x):
    return bf16.to_bf16_bits(np.array(x, dtype=np.float64))


def test_signed_zero_order():
    # x = 0 with S = 0: the interval is the single value +0; -0 is outside it
    assert check.accept(b([0.0]), [0.0], [0.0], 0.0).all()
    assert not check.accept(b([-0.0]), [0.0], [0.0], 0.0).any()
    # a tiny negative value rounds to -0; +0 lies above it
    assert check.accept(b([-0.0]), [-1e-45], [0.0], 0.0).all()
    assert not check.accept(b([0.0]), [-1e-45], [0.0], 0.0).any()
    # an interval straddling zero holds both zeros
    assert check.accept(b([-0.0, 0.0]), [1e-45, 1e-45], [1.0, 1.0], 0.0).all()


def test_one_value_interval_is_bit_exact():
    x = np.array([1.0 + 2.0 ** -10])            # well inside one bf16 cell, S tiny
    assert check.accept(b([1.0]), x, [2.0 ** -30], 0.0, "S").all()
    nxt = np.array([0x3F81], np.uint16)
    assert not check.accept(nxt, x, [2.0 ** -30], 0.0, "S").any()
    # tier G adds one ulp of relative width: the neighbour is accepted there
    assert check.accept(nxt, x, [2.0 ** -30], 0.0, "G").all()


def test_nan_and_infinities():
    nan = np.array([0x7FC0], np.uint16)
    assert check.accept(nan, [np.nan], [np.nan], 0.0).all()
    assert not check.accept(b([1.0]), [np.nan], [np.nan], 0.0).any()
    assert not check.accept(nan, [1.0], [1.0], 0.0).any()
    assert check.accept(b([np.inf]), [np.inf], [np.inf], 0.0).all()
    assert not check.accept(b([-np.inf]), [np.inf], [np.inf], 0.0).any()
    assert not check.accept(b([3.0e38]), [np.inf], [np.inf], 0.0).any()


def test_literal_stats_counts():
    x = np.array([1.0, 1.0, 1.0, 2.0])
    out = np.array([0x3F80, 0x3F81, 0x3F82, 0x4000], np.uint16)
    st = check.literal_stats(out, x)
    assert st == {"n": 4, "equal": 2, "within_1ulp": 3}


def _steps(a_bits, b_bits):
    return np.abs(bf16.order_key(a_bits) - bf16.order_key(b_bits))


def test_literal_step_lemma():
    """|y - x| <= 2**-9 |x| keeps bf16(y) within one step of bf16(x): across binades, at
    powers of two from both sides, on rounding midpoints and among subnormals; a relative
    error of 2**-7 does not (so the claim has content)."""
    rng = np.random.default_rng(11)
    e = rng.integers(-140, 120, size=200000)
    m = rng.uniform(1.0, 2.0, size=e.size)
    x = np.ldexp(m, e) * rng.choice([-1.0, 1.0], size=e.size)
    # exact powers of two, their neighbours and the rounding midpoints around them
    p2 = np.ldexp(1.0, np.arange(-135, 100))
    x = np.concatenate([x, p2, p2 * (1 - 2.0 ** -9), p2 * (1 + 2.0 ** -8), p2 * (1 - 2.0 ** -8)])
    for t in (-1.0, -0.5, 0.5, 1.0):
        y = x + t * check.LITERAL_STEP * np.abs(x)
        assert _steps(bf16.to_bf16_bits(y), bf16.to_bf16_bits(x)).max() <= 1, t
    y = x + 2.0 ** -7 * np.abs(x)
    assert _steps(bf16.to_bf16_bits(y), bf16.to_bf16_bits(x)).max() >= 2


def test_literal_outside_report():
    x = np.array([1.0, 1.0, 1.0, -3.0, 0.25])
    S = np.array([1.0, 2.0 ** 8, 4.0, 3.0, 1.0])
    # 1.0 + 3 steps (|x|/S = 2**-8), one step, equal, -3 + 2 steps (|x|/S = 1), equal
    out = np.array([0x3F83, 0x3F81, 0x3F80, 0xC042, 0x3E80], np.uint16)
    n_out, worst = check.literal_outside(out, x, S)
    assert (n_out, worst) == (2, 1.0)
    n_out, worst = check.literal_outside(out[:3], x[:3], S[:3])
    assert (n_out, worst) == (1, 1.0)
    n_out, worst = check.literal_outside(out[1:3], x[1:3], S[1:3])
    assert (n_out, worst) == (0, 0.0)
    rep = check.report(out, x, S, check.E_P_FP32)
    assert (rep["outside"], rep["equal"], rep["within_1ulp"]) == (2, 2, 3)
    # the bound: 2**9 (e_P + 2**-16)
    assert check.literal_bound(check.E_P_FP32) == 2.0 ** -7
    assert check.literal_bound(check.E_P_P32) == 2.0 ** -6


# ---- float32 emulation of chunked decode (CPU test code, numpy float32 steps) -----------

def emulate_decode(q, kc, vc, stream, pos, win, ring, chunk=256, early=0, no_rescale=False,
                   truncate=False):
    """Decode partials per absolute chunk, then an ordered merge, in float32."""
    R, Hq, d = q.shape
    G = Hq // kc.shape[2]
    out = np.empty((R, Hq, d), np.uint16)
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    for r in range(R):
        lo, last = attend.key_window(pos[r], win)
        lo = max(0, lo - early)
        for h in range(Hq):
            ms, ls, os_ = [], [], []
            for c in range(lo // chunk, last // chunk + 1):
                keys = np.arange(max(lo, c * chunk), min(last, c * chunk + chunk - 1) + 1)
                K = f(kc[stream[r], keys % ring, h // G])
                V = f(vc[stream[r], keys % ring, h // G])
                s = (K @ f(q[r, h])).astype(np.float32)
                m = s.max()
                p = np.exp(s - m).astype(np.float32)
                ms.append(m); ls.append(p.sum(dtype=np.float32)); os_.append((p @ V).astype(np.float32))
            M = max(ms)
            num = np.zeros(d, np.float32)
            den = np.float32(0)
            for m, l, o in zip(ms, ls, os_):
                a = np.float32(1) if no_rescale else np.exp(np.float32(m - M))
                num = (num + a * o).astype(np.float32)
                den = np.float32(den + a * l)
            y = (num / den).astype(np.float32)
            out[r, h] = (y.view(np.uint32) >> 16).astype(np.uint16) if truncate else \
                workloads._bf16_bits(y)
    return out


@pytest.fixture(scope="module")
def small_decode():
    return workloads.decode_case("checker discrimination", 6, 4, 2, 256, 300, 700, 2,
                                 [299, 512, 690, 1000, 1400, 255], seed=11, peak_every=2)


def _strict_fails(case, out):
    x, S, _ = attend.decode(case.q, case.k, case.v, case.stream, case.pos, case.win, case.ring, 1.0)
    return int((~check.accept(out, x, S, check.E_P_FP32, "S")).sum())


def test_fp32_emulation_passes_strict(small_decode):
    c = small_decode
    out = emulate_decode(c.q, c.k, c.v, c.stream, c.pos, c.win, c.ring)
    assert _strict_fails(c, out) == 0


@pytest.mark.parametrize("kw", [{"early": 1}, {"no_rescale": True}, {"truncate": True}])
def test_planted_mistakes_go_red(small_decode, kw):
    c = small_decode
    out = emulate_decode(c.q, c.k, c.v, c.stream, c.pos, c.win, c.ring, **kw)
    assert _strict_fails(c, out) > 0


def _f(a):
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32)


def _bf(a):
    """float32 -> float32 value of its bf16 rounding (torch's nearest-even conversion)."""
    return _f(workloads._bf16_bits(np.asarray(a, dtype=np.float32)))


def _p_parts(p, parts):
    """fp32 P as `parts` bf16 parts: each the rounding of what the earlier parts leave."""
    out, rest = [], p.astype(np.float32)
    for _ in range(parts):
        b_ = _bf(rest)
        out.append(b_)
        rest = (rest - b_).astype(np.float32)
    return out


def _emulate_prompt(case, parts):
    """float32 emulation of a prompt with P fed to P.V as `parts` bf16 parts (products of
    the parts with v summed in float64, as exact MFMA products with fp32-accurate sums)."""
    out = np.empty_like(case.q)
    for i in range(case.n):
        lo, last = attend.key_window(case.p0 + i, case.win)
        keys = np.arange(lo, last + 1) % case.ring
        for h in range(case.hq):
            K, V = _f(case.k[keys, 0]), _f(case.v[keys, 0])
            s = (K @ _f(case.q[i, h])).astype(np.float32)
            p = np.exp(s - s.max()).astype(np.float32)
            pp = sum(x.astype(np.float64) for x in _p_parts(p, parts))
            y = ((pp @ V.astype(np.float64)).astype(np.float32) / p.sum(dtype=np.float32)).astype(np.float32)
            out[i, h] = workloads._bf16_bits(y)
    return out


@pytest.fixture(scope="module")
def p_control():
    case = workloads.prompt_case("p32 control", 24, 2, 1, 256, 40, 64, 128, seed=12)
    x, S, _ = attend.prompt(case.q, case.k, case.v, case.p0, case.win, case.ring, 1.0)
    return case, x, S


def test_one_bf16_p_goes_red_under_the_p32_interval(p_control):
    case, x, S = p_control
    fails = {n: int((~check.accept(_emulate_prompt(case, n), x, S, check.E_P_P32, "S")).sum())
             for n in (1, 2)}
    assert fails[2] == 0
    assert fails[1] > 0


def test_three_part_p_passes_the_fp32_interval(p_control):
    # three parts carry fp32's P exactly: the strict interval of fp32 P (e_P = 0) holds
    case, x, S = p_control
    out = _emulate_prompt(case, 3)
    assert int((~check.accept(out, x, S, check.E_P_THREE, "S")).sum()) == 0


def test_three_part_split_is_exact_down_to_2_pow_minus_110():
    # P = m 2^(e-23) with a 24-bit m: three nearest-even bf16 parts (8 significant bits
    # each) hold all 24 bits as long as the last part's lowest bit, 2^(e-23), is at least
    # bf16's smallest subnormal 2^-133, i.e. e >= -110. Above P's range in the kernels
    # (P <= 2^8) nothing changes.
    rng = np.random.default_rng(5)
    e = rng.integers(-110, 9, 200_000)
    m = rng.integers(2 ** 23, 2 ** 24, 200_000)
    edge = np.array([2 ** 23, 2 ** 24 - 1, 2 ** 23 + 2 ** 15, 2 ** 23 + 2 ** 15 + 2 ** 7, 2 ** 24 - 2 ** 8 - 1])
    e = np.concatenate([e, np.full(edge.size, -110), np.full(edge.size, 8)])
    m = np.concatenate([m, edge, edge])
    p = (m.astype(np.float64) * 2.0 ** (e - 23)).astype(np.float32)
    hi, mid, lo = _p_parts(p, 3)
    assert np.array_equal(hi.astype(np.float64) + mid + lo, p.astype(np.float64))
    # two parts leave up to 2^-16 relative (the p32 bound), one part 2^-8 (half a bf16 ulp
    # at the bottom of a binade)
    two = hi.astype(np.float64) + mid
    rel2 = np.abs(two - p) / p
    assert rel2.max() <= 2.0 ** -16 and rel2.max() > 2.0 ** -18
    rel1 = np.abs(hi.astype(np.float64) - p) / p
    assert rel1.max() <= 2.0 ** -8 and rel1.max() > 2.0 ** -9
    # below 2^-110 the last part loses bits
    q = (m[:1000].astype(np.float64) * 2.0 ** (-112 - 23)).astype(np.float32)
    h3 = _p_parts(q, 3)
    assert not np.array_equal(h3[0].astype(np.float64) + h3[1] + h3[2], q.astype(np.float64))
