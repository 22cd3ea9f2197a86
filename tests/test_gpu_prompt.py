"""GPU parity of the MFMA prompt kernel (wa_prompt) against the float64 oracle.

Gate: every bf16 output inside its tier-G interval (oracle.check) with e_P = 2**-16 for p32,
2**-8 for P as one bf16 and 0 for P as three bf16 parts (which must also meet the strict
interval of fp32 P). Masks are pinned by peaked-edge probes; chunk invariance
(TensorFold pull request #1123, "Receipt", exactness bullet: cutting a prompt chunk into two
calls must leave each row's bits unchanged) and repeatability by byte equality.
"""

import numpy as np
import pytest
import torch

from oracle import attend, check
from sliding_window_gqa_amd import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def e_p(p32):
    """Representation error of P: p32 False/0 one bf16, True/1 two parts, 2 three parts."""
    return {0: check.E_P_BF16, 1: check.E_P_P32, 2: check.E_P_THREE}[int(p32)]


def _gate(case, label, p32=None, rows=None):
    p32 = case.p32 if p32 is None else p32
    gu.log(f"prompt case: {label} n={case.n} p0={case.p0} hq={case.hq} hkv={case.hkv} "
           f"d={case.d} win={case.win} ring={case.ring} p32={p32} hi={case.hi is not None}")
    out = gu.run_prompt(case, p32=p32)
    if rows is not None:
        out = out[rows]
    x, S, _ = gu.oracle_prompt(case, rows=rows)
    rep, ok = gu.compare(out, x, S, e_p(p32), label)
    assert ok.all()
    return out, rep


def test_prompt_12b_p32_image_rows():
    _gate(workloads.prompt_12b(), "12B prompt p32 image rows")


def test_prompt_31b_bf16p():
    _gate(workloads.prompt_31b(), "31B prompt bf16 P")


def test_long_prompt_sampled():
    """The long prompt at full size on its seeded sample of rows, with P as one bf16 (the
    default), as two halves (p32, its variant) and as three parts: one float64 reference, three
    calls on the same inputs; the literal one-step rule is asserted for the last two."""
    case = workloads.long_prompt()
    rows = workloads.long_prompt_sample_rows(case.n)
    x, S, _ = gu.oracle_prompt(case, rows=rows)
    for p32, name in ((0, "bf16 P"), (1, "p32"), (2, "three parts")):
        label = f"long prompt 37810x56x128 sampled, {name}"
        gu.log(f"prompt case: {label} n={case.n} hq={case.hq} d={case.d} p32={p32}")
        out = gu.run_prompt(case, p32=p32)[rows]
        rep, ok = gu.compare(out, x, S, e_p(p32), label)
        assert ok.all()
        if p32 == 2:
            assert rep["tier_S_fail"] == 0, rep


THREE = 2      # Window.p32 value: P as three bf16 parts


def _gate_strict(case, label, rows=None):
    """Three parts carry fp32's P exactly: tier G and the strict interval of fp32 P."""
    out, rep = _gate(case, label, p32=THREE, rows=rows)
    assert rep["tier_S_fail"] == 0, rep
    return out


def test_prompt_12b_three_parts():
    _gate_strict(workloads.prompt_12b(), "12B prompt, P in three parts, image rows")


def test_prompt_31b_three_parts():
    _gate_strict(workloads.prompt_31b(), "31B prompt, P in three parts")


def test_long_prompt_small_three_parts():
    _gate_strict(workloads.long_prompt(n=3001, heads=4), "long prompt 3001x4x128, P in three parts")


@pytest.mark.parametrize("n,hq,hkv,d,p0,win,ring,span", [
    (7, 3, 1, 256, 40, 16, 64, None),
    (129, 16, 2, 128, 77, 100, 300, (0, 128)),
    (200, 8, 8, 128, 1000, 0, 1200, None),
    (300, 32, 16, 256, 1300, 1024, 1536, (10, 90)),
])
def test_three_parts_shapes(n, hq, hkv, d, p0, win, ring, span):
    hi = None
    if span is not None:
        hi = p0 + np.arange(n)
        a, b = span
        hi[a:b + 1] = p0 + b
    case = workloads.prompt_case("three parts", n, hq, hkv, d, p0, win, ring, seed=7 * n + d,
                                 hi=hi, peak_every=3)
    _gate_strict(case, f"three parts n{n} {hq}/{hkv}x{d} p0={p0} win{win} ring{ring}")


def test_three_parts_chunk_invariance_and_repeat():
    case = workloads.prompt_case("12B shape, three parts", 512, 16, 8, 256, 5000, 1024, 1536,
                                 seed=1003, p32=THREE)
    full = _split_check(case, (1, 255, 256, 257, 300))
    assert np.array_equal(gu.run_prompt(case), full)


def test_long_prompt_small_p32():
    case = workloads.long_prompt(n=3001, heads=4)
    _gate(case, "long prompt 3001x4x128 p32", p32=True)


SHAPES = [
    # n, hq, hkv, d, p0, win, ring, p32, image span (a, b) or None
    (1, 2, 1, 256, 0, 1024, 1536, False, None),
    (7, 3, 1, 256, 40, 16, 64, True, None),
    (33, 16, 1, 256, 300, 64, 128, False, (3, 20)),
    (200, 8, 8, 128, 1000, 0, 1200, True, None),
    (513, 16, 8, 256, 5000, 1024, 1536, False, (40, 300)),
    (129, 16, 2, 128, 77, 100, 300, True, (0, 128)),
    (70, 4, 4, 128, 0, 0, 70, False, None),
]


@pytest.mark.parametrize("n,hq,hkv,d,p0,win,ring,p32,span", SHAPES)
def test_prompt_shapes(n, hq, hkv, d, p0, win, ring, p32, span):
    hi = None
    if span is not None:
        hi = p0 + np.arange(n)
        a, b = span
        hi[a:b + 1] = p0 + b
    case = workloads.prompt_case("shape", n, hq, hkv, d, p0, win, ring, seed=n + hq + d,
                                 hi=hi, p32=p32, peak_every=3)
    _gate(case, f"prompt shape n{n} {hq}/{hkv}x{d} p0={p0} win{win} ring{ring}")


SHORT_RINGS = [
    # n, hq, hkv, d, p0, win, ring, p32: rings shorter than one 64-key tile, so that an
    # edge tile's keys wrap around the ring several times (window 8 over 11 slots, ...)
    (4, 2, 1, 256, 100, 8, 11, True),
    (4, 2, 1, 128, 100, 8, 11, False),
    (30, 4, 2, 256, 500, 20, 49, THREE),
    (12, 2, 2, 128, 3, 0, 15, True),
    (9, 3, 1, 256, 61, 5, 13, False),
]


@pytest.mark.parametrize("n,hq,hkv,d,p0,win,ring,p32", SHORT_RINGS)
def test_prompt_short_rings(n, hq, hkv, d, p0, win, ring, p32):
    """Keys of a ring shorter than a tile come from slot j mod ring on every tile."""
    case = workloads.prompt_case("short ring", n, hq, hkv, d, p0, win, ring, seed=3 * n + ring,
                                 p32=p32, peak_every=2)
    _gate(case, f"short ring n{n} {hq}/{hkv}x{d} p0={p0} win{win} ring{ring}")


def _split_check(case, cuts):
    full = gu.run_prompt(case)
    for cut in cuts:
        a = gu.run_prompt(case, rows=(0, cut))
        b = gu.run_prompt(case, rows=(cut, case.n))
        assert np.array_equal(np.concatenate([a, b]), full), (case.name, cut)
    return full


def test_prompt_chunk_invariance_and_repeat():
    """Cutting the prompt into two calls leaves each row's bits unchanged. A chunk must hold
    an image's rows whole (hi[i] < p0 + n), so the image-span workload is cut only outside
    its span (rows 40..300);
    the same shape without an image span, and the causal 31B workload, are cut anywhere."""
    case = workloads.prompt_12b()
    full = _split_check(case, (1, 17, 39, 40, 301, 302, 400, 511))
    for _ in range(3):
        assert np.array_equal(gu.run_prompt(case), full)
    plain = workloads.prompt_case("12B shape, no image span", 512, 16, 8, 256, 5000, 1024, 1536,
                                  seed=1003, p32=True)
    _split_check(plain, (1, 17, 255, 256, 257, 300))
    _split_check(workloads.prompt_31b(), (1, 100, 200, 255, 256, 257, 332))


def test_prompt_mask_edges_bit_exact():
    """A key at lo_i or last_i with a score lead of 200 wins outright; at lo_i - 1 or
    last_i + 1 it takes no part. Probed on many rows at once, with an image span."""
    n, p0, win, ring, d = 96, 1300, 1024, 1536, 256
    rng = np.random.default_rng(5)
    hi = p0 + np.arange(n)
    hi[10:41] = p0 + 40
    for p32 in (True, False, THREE):
        for which in ("lo", "last", "lo-1", "last+1"):
            case = workloads.prompt_case("edges", n, 1, 1, d, p0, win, ring, seed=8, hi=hi,
                                         p32=p32, peak_every=0)
            marks = {}
            used = set()
            for i in range(0, n, 3):
                lo, last = attend.key_window(p0 + i, win, int(hi[i]))
                key = {"lo": lo, "last": last, "lo-1": lo - 1, "last+1": last + 1}[which]
                if key in used or key > p0 + n - 1:
                    continue
                used.add(key)
                # the key is visible to other rows too: only row i's query aligns with it
                qh = (case.q[i, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                case.k[key % ring, 0] = workloads._bf16_bits(qh * (200.0 / (qh @ qh)))
                vb = workloads._bf16_bits(rng.standard_normal(d) * 4)
                case.v[key % ring, 0] = vb
                marks[i] = vb
            out = gu.run_prompt(case)
            x, S, _ = gu.oracle_prompt(case)
            assert check.accept(out, x, S, e_p(p32)).all(), (which, p32)
            for i, vb in marks.items():
                # a row that another row's probe key also reaches is judged by the gate only
                hit = np.array_equal(out[i, 0], vb)
                if which in ("lo", "last"):
                    assert hit, (which, p32, i)
                else:
                    assert not hit, (which, p32, i)


def test_prompt_integer_sums():
    """Every key alike: weights exactly 1 (exact in one bf16 too), integer values; the
    output is the exact mean."""
    n, p0, win, ring, d = 64, 2000, 1024, 1536, 256
    for p32 in (True, False, THREE):
        case = workloads.prompt_case("sums", n, 2, 1, d, p0, win, ring, seed=6, p32=p32,
                                     peak_every=0)
        case.k[:] = case.k[0, 0]
        slot_vals = 96.0 + (np.arange(ring) * 7) % 32
        case.v[:, 0] = workloads._bf16_bits(slot_vals[:, None] * np.ones(d))
        out = gu.run_prompt(case)
        for i in range(n):
            lo, last = attend.key_window(p0 + i, win)
            mean = slot_vals[np.arange(lo, last + 1) % ring].sum() / (last - lo + 1)
            want = workloads._bf16_bits(np.array([np.float32(mean)]))[0]
            assert np.all(out[i] == want), (p32, i)


def test_prompt_nan_query_neighbour():
    """A NaN query in one row: its neighbours' bits are those they get alone, beside it, and
    split across calls (bf16 P and p32)."""
    for p32 in (False, True):
        case = workloads.prompt_case("nan neighbour", 40, 2, 1, 256, 700, 256, 1024, seed=10,
                                     p32=p32)
        clean = gu.run_prompt(case)
        case.q[17, 1, 5] = 0x7FC0
        bad = gu.run_prompt(case)
        assert np.all(np.isnan((bad[17, 1].astype(np.uint32) << 16).view(np.float32)))
        keep = np.ones((40, 2), bool)
        keep[17, 1] = False
        assert np.array_equal(bad[keep], clean[keep])
        a = gu.run_prompt(case, rows=(0, 17))
        b = gu.run_prompt(case, rows=(17, 40))
        assert np.array_equal(np.concatenate([a, b])[keep], clean[keep])


def test_prompt_nonfinite_key_and_column():
    NAN, PINF, NINF = 0x7FC0, 0x7F80, 0xFF80
    case = workloads.prompt_case("nan key", 50, 4, 2, 256, 300, 64, 512, seed=12, p32=True)
    case.k[320 % 512, 1, 0] = NAN               # rows 20..49 of key head 1 see key 320
    out = gu.run_prompt(case)
    x, S, _ = gu.oracle_prompt(case)
    assert np.isnan(x[20:, 2:4]).all() and np.isfinite(x[:20]).all()
    assert check.accept(out, x, S, e_p(True)).all()
    case = workloads.prompt_case("inf column", 50, 4, 2, 256, 300, 64, 512, seed=13, p32=False)
    case.v[290, 0, 3] = PINF                    # every row sees keys 290 and 291
    case.v[291, 0, 3] = NINF
    out = gu.run_prompt(case)
    x, S, _ = gu.oracle_prompt(case)
    assert np.isnan(x[:, 0:2, 3]).all()
    assert check.accept(out, x, S, e_p(False)).all()


@pytest.mark.parametrize("win,p32", [(64, False), (64, True), (0, False), (64, 2), (0, 2)])
def test_prompt_inf_value_unseen_by_tile_neighbours(win, p32):
    """Rows that do not see an infinite value but share its key tile get 0 * inf in the MFMA
    P.V product; their float64 re-run gives float64's finite result, and the rows that do
    see it keep +inf. Covers the split (window) and the unsplit (window 0) paths."""
    if win == 0:
        case = workloads.prompt_case("inf unseen", 50, 4, 2, 256, 300, 0, 350, seed=13, p32=p32)
        case.hi = np.full(50, 300 + 49, np.int32)
        case.hi[:4] = 300 + np.arange(4)      # rows 0..3: causal; others see everything
        case.v[240, 0, 3] = 0x7F80
        out = gu.run_prompt(case)
        x, S, _ = gu.oracle_prompt(case)
        assert np.isinf(x[:, 0:2, 3]).all()
        assert check.accept(out, x, S, e_p(p32)).all()
        case.v[240, 0, 3] = case.v[241, 0, 3]
        case.v[349, 0, 3] = 0x7F80            # the last key: only rows 4..49 see it
        out = gu.run_prompt(case)
        x, S, _ = gu.oracle_prompt(case)
        assert np.isinf(x[4:, 0:2, 3]).all() and np.isfinite(x[:4]).all()
        assert check.accept(out, x, S, e_p(p32)).all()
        return
    case = workloads.prompt_case("inf unseen", 50, 4, 2, 256, 300, win, 512, seed=13, p32=p32)
    case.v[240, 0, 3] = 0x7F80                  # only rows 0..3 reach key 240
    out = gu.run_prompt(case)
    x, S, _ = gu.oracle_prompt(case)
    assert np.isinf(x[:4, 0:2, 3]).all() and np.isfinite(x[4:]).all()
    assert check.accept(out, x, S, e_p(p32)).all()


def _cancelling_values(rng, keys, heads, d):
    """bf16 bits [keys, heads, d]: per (head, dim) column, keys/2 magnitudes 2^E (1 + F/128),
    E uniform in -20..20, each placed once with + and once with - at random keys, so every
    column sums to exactly 0 while its partial sums reach 2^20 and more."""
    e = rng.integers(-20, 21, size=(keys // 2, heads, d))
    f = rng.integers(0, 128, size=(keys // 2, heads, d))
    mag = np.ldexp(1.0 + f / 128.0, e)
    vals = np.concatenate([mag, -mag], axis=0)
    for h in range(heads):
        for c in range(d):
            vals[:, h, c] = vals[rng.permutation(keys), h, c]
    return workloads._bf16_bits(vals)


@pytest.mark.parametrize("p32", [0, 1, 2])
def test_mfma_accumulation_under_cancellation(p32):
    """The matrix cores' fp32 accumulation, measured: q = 0 gives every key the weight 1
    exactly (in every P representation), and values in exactly cancelling +/- pairs give an
    exact output of 0, so a nonzero output is the accumulation error of P.V over 1,024 keys.
    It is logged in units of 2^-24 S (S = mean |v|) and held to the strict interval of
    e_P = 0, whose 2^-16 S allowance must cover it."""
    n, hq, hkv, d, p0 = 24, 4, 4, 256, 1000
    rng = np.random.default_rng(41 + p32)
    case = workloads.prompt_case("cancellation", n, hq, hkv, d, p0, 0, p0 + n, seed=41,
                                 hi=np.full(n, p0 + n - 1), p32=p32, peak_every=0)
    case.q[:] = 0
    case.v[:] = _cancelling_values(rng, p0 + n, hkv, d)
    out = gu.run_prompt(case)
    x, S, _ = gu.oracle_prompt(case)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    worst = float(np.max(np.abs(got - x) / S))
    gu.log(f"[mfma accumulation p32={p32}] worst |out - x| / S = {worst:.3e} "
           f"= {worst * 2 ** 24:.1f} x 2^-24; allowance 2^-16 = 256 x 2^-24")
    assert check.accept(out, x, S, check.E_P_THREE, "S").all()


@pytest.mark.parametrize("n,hq,hkv,d,p32", [(40, 4, 2, 256, True), (40, 4, 2, 256, THREE),
                                            (40, 2, 2, 128, False)])
def test_slot_stride_at_the_31_bit_limit(n, hq, hkv, d, p32):
    """K/V slots as far apart as wa_prompt accepts (a 64-key tile's span a few hundred KB under
    2^31 bytes): the rows match the oracle and the same ring laid out densely, bit for bit."""
    from sliding_window_gqa_amd import api
    p0, win, ring = 100, 24, 64
    case = workloads.prompt_case("far slots", n, hq, hkv, d, p0, win, ring, seed=n + d, p32=p32,
                                 peak_every=2)
    sslot = gu.limit_slot_stride(63, d)
    label = f"prompt far slots n{n} {hq}/{hkv}x{d} p32={p32} slot stride {sslot}"
    gu.log(f"prompt case: {label}")
    k, v = gu.far_slots(case.k, sslot), gu.far_slots(case.v, sslot)
    assert 63 * k.stride(0) * 2 + 2 * d < 2**31 - 1 < 63 * (k.stride(0) + 8) * 2 + 2 * d
    out = api.prompt(gu.dev_bf16(case.q), k, v, p0, win, ring, case.scale, p32=p32)
    torch.cuda.synchronize()
    bits = gu.host_bits(out)
    del k, v, out
    x, S, _ = gu.oracle_prompt(case)
    _, ok = gu.compare(bits, x, S, e_p(p32), label)
    assert ok.all()
    assert np.array_equal(bits, gu.run_prompt(case))


@pytest.mark.parametrize("scale", [-0.8, 0.0])
@pytest.mark.parametrize("d,p32", [(256, True), (256, THREE), (256, False), (128, True)])
def test_negative_and_zero_scale(scale, d, p32):
    """Any finite float32 score scale: negative (the kernels carry its sign on q, exactly) or
    zero (every visible key the same weight)."""
    hi = 300 + np.arange(70)
    hi[5:20] = 300 + 19
    case = workloads.prompt_case("scale", 70, 4, 2, d, 300, 128, 512, seed=d + 5, hi=hi, p32=p32,
                                 scale=scale, peak_every=2)
    _gate(case, f"prompt scale {scale} d{d} p32={p32}")

