"""GPU parity of the split-KV decode (wa_decode) against the float64 oracle.

Gate: every bf16 output inside its tier-G interval (oracle.check) with fp32 probabilities
(e_P = 0). Masks are pinned bit for bit by peaked-edge probes, accumulation by integer sums,
and the row-bit invariants of TensorFold pull request #1123 ("Receipt", exactness bullet)
by byte equality.
"""

import numpy as np
import pytest
import torch

from oracle import attend, check
from sliding_window_gqa_amd import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

E_P = check.E_P_FP32


def _gate(case, label, rows=None):
    gu.log(f"decode case: {label} rows={case.rows} hq={case.hq} hkv={case.hkv} d={case.d} "
           f"win={case.win} ring={case.ring}")
    out = gu.run_decode(case)
    x, S, _ = gu.oracle_decode(case)
    rep, ok = gu.compare(out, x, S, E_P, label)
    assert ok.all()
    return out, rep


def test_tiny_decode():
    _gate(workloads.tiny_decode(), "tiny decode")


def test_decode_12b_three_streams():
    _, rep = _gate(workloads.decode_12b(), "12B decode 64 rows 3 streams")
    assert rep["tier_S_fail"] <= rep["n"] // 1000


def test_decode_12b_64_streams():
    _gate(workloads.decode_12b(streams=64), "12B decode 64 rows 64 streams")


SHAPES = [
    # rows, hq, hkv, d, win, ring, streams
    (5, 2, 1, 256, 1, 40, 1),
    (7, 3, 1, 256, 300, 700, 2),
    (9, 16, 2, 256, 1024, 1536, 3),
    (6, 16, 1, 128, 257, 600, 2),
    (4, 8, 8, 128, 64, 100, 4),
    (3, 4, 2, 256, 0, 1300, 1),
    (8, 32, 16, 256, 1024, 1536, 2),
    (3, 16, 1, 256, 300, 700, 2),         # sixteen query heads on one key head
]


@pytest.mark.parametrize("rows,hq,hkv,d,win,ring,streams", SHAPES)
def test_decode_shapes(rows, hq, hkv, d, win, ring, streams):
    rng = np.random.default_rng(rows * 131 + hq * 7 + d + win)
    hi = ring - 1 if win == 0 else 3000
    pos = rng.integers(0, hi + 1, size=rows)
    pos[0] = 0
    if rows > 2:
        pos[1] = min(hi, 255)
        pos[2] = min(hi, 256)
    case = workloads.decode_case("shape", rows, hq, hkv, d, win, ring, streams, pos,
                                 seed=rows + hq + d, peak_every=2)
    _gate(case, f"decode shape {rows}x{hq}/{hkv}x{d} win{win} ring{ring}")


def test_decode_invariants():
    case = workloads.decode_12b()
    full = gu.run_decode(case)
    # each row alone, in another stream slot, at the same bits
    for r in (0, 5, 17, 63):
        t = int(case.stream[r])
        k1 = case.k[t:t + 1].copy()
        v1 = case.v[t:t + 1].copy()
        one = workloads.DecodeCase("alone", case.q[r:r + 1], np.concatenate([k1 * 0, k1]),
                                   np.concatenate([v1 * 0, v1]), np.array([1], np.int32),
                                   case.pos[r:r + 1], case.win, case.ring)
        assert np.array_equal(gu.run_decode(one)[0], full[r])
    # a smaller call gives the widest call's bits
    sub = workloads.DecodeCase("sub", case.q[10:27], case.k, case.v, case.stream[10:27],
                               case.pos[10:27], case.win, case.ring)
    assert np.array_equal(gu.run_decode(sub), full[10:27])
    # repeat: byte-identical
    for _ in range(4):
        assert np.array_equal(gu.run_decode(case), full)


@pytest.mark.parametrize("rows,hq,hkv,d,win,ring,streams", [
    (32, 32, 8, 256, 1024, 1536, 2),     # four query heads a key head
    (40, 24, 8, 256, 700, 1024, 2),      # three
    (36, 16, 16, 256, 1024, 1536, 2),    # one, d = 256
    (48, 8, 8, 128, 1024, 1536, 3),      # one, d = 128
    (40, 16, 8, 128, 1024, 1536, 3),     # two, d = 128
    (32, 8, 8, 256, 1024, 1536, 32),     # whole rows (a stream a row), one query head a key head
])
def test_large_grid_rows_match_rows_alone(rows, hq, hkv, d, win, ring, streams):
    """Chunk grids of 1,024 workgroups or more (the kernel form with 8-key load units), and
    batches of rows in streams of their own (the whole-row kernel), pass the gate, and a row
    alone (a small grid: the form with 16- or 32-key load units) gets the same bits: neither
    the load unit nor the kernel form changes the arithmetic."""
    rng = np.random.default_rng(rows * 17 + hq + d)
    pos = rng.integers(0, 20001, size=rows)
    pos[:3] = [0, 255, 256]
    case = workloads.decode_case("large grid", rows, hq, hkv, d, win, ring, streams, pos,
                                 seed=rows + 5 * hq + d, peak_every=3)
    full, _ = _gate(case, f"large grid {rows}x{hq}/{hkv}x{d} win{win} ring{ring} streams{streams}")
    for r in (0, 2, rows // 2, rows - 1):
        t = int(case.stream[r])
        one = workloads.DecodeCase("alone", case.q[r:r + 1], case.k[t:t + 1], case.v[t:t + 1],
                                   np.array([0], np.int32), case.pos[r:r + 1], case.win, case.ring)
        assert np.array_equal(gu.run_decode(one)[0], full[r]), r


@pytest.mark.parametrize("rows,hq,hkv,d,ring", [
    (3, 4, 2, 256, 1552),     # ring = 16 mod 32: a 32-key unit of a small grid can wrap
    (40, 16, 8, 256, 1552),   # the same ring under a large grid (8-key units)
    (3, 4, 2, 256, 1544),     # ring = 8 mod 16
    (3, 2, 2, 128, 1040),     # d = 128, ring = 16 mod 32
])
def test_rings_not_a_multiple_of_the_load_unit(rows, hq, hkv, d, ring):
    """Rings whose length is a multiple of 16 but not of 32 (or of 8 but not 16): keys of a
    load unit wrap round the ring end and must come from the ring's first slots; rows whose
    windows cross the wrap pass the gate and match their bits alone."""
    rng = np.random.default_rng(ring + rows)
    pos = rng.integers(ring, 20000, size=rows)
    # positions whose windows hold a load unit that wraps round the ring end (at rings 1552
    # and 1544; at 1040 no unit wraps)
    pos[0] = ring + 48
    if rows > 1:
        pos[1] = ring + 300
    case = workloads.decode_case("wrap", rows, hq, hkv, d, 1024, ring, 2, pos,
                                 seed=ring + hq, peak_every=2)
    full, _ = _gate(case, f"ring {ring} rows {rows} {hq}/{hkv}x{d}")
    for r in (0, rows - 1):
        t = int(case.stream[r])
        one = workloads.DecodeCase("alone", case.q[r:r + 1], case.k[t:t + 1], case.v[t:t + 1],
                                   np.array([0], np.int32), case.pos[r:r + 1], case.win, case.ring)
        assert np.array_equal(gu.run_decode(one)[0], full[r]), r


@pytest.mark.parametrize("rows,hq,hkv,win,ring,streams", [
    (40, 16, 8, 1536, 1536, 2),    # window = ring: a row's chunks c and c + 6 share a slot block
    (33, 4, 4, 0, 1024, 3),        # linear cache, one query head per key head
    (20, 8, 4, 700, 768, 1),       # every row in one stream: groups of 8 rows
    (64, 16, 8, 1024, 1536, 3),    # the 12B shape
])
def test_rows_sharing_streams_match_rows_alone(rows, hq, hkv, win, ring, streams):
    """Many rows on few streams (a row meeting one slot block twice at window = ring, window 0,
    one query head per key head): each row's bits equal those it gets alone in its own call,
    whichever decode kernel each call takes, and pass the gate."""
    rng = np.random.default_rng(rows + win)
    hi = ring - 1 if win == 0 else 20000
    pos = rng.integers(0, hi + 1, size=rows)
    pos[:4] = [0, 255, 256, min(hi, 1535)]
    case = workloads.decode_case("shared", rows, hq, hkv, 256, win, ring, streams, pos,
                                 seed=rows * 3 + hq, peak_every=3)
    full, _ = _gate(case, f"shared streams {rows}x{hq}/{hkv} win{win} ring{ring} streams{streams}")
    for r in range(rows):
        t = int(case.stream[r])
        one = workloads.DecodeCase("alone", case.q[r:r + 1], case.k[t:t + 1], case.v[t:t + 1],
                                   np.array([0], np.int32), case.pos[r:r + 1], case.win, case.ring)
        assert np.array_equal(gu.run_decode(one)[0], full[r]), r


@pytest.mark.parametrize("rows,hq,hkv,d,win,ring,streams", [SHAPES[1], SHAPES[3], (64, 16, 8, 256, 1024, 1536, 3)])
def test_merge_reproduces_decode(rows, hq, hkv, d, win, ring, streams):
    """wa_merge on the partials wa_decode leaves in its workspace (layout of the header:
    m, l, o at float offsets 0, cells, 2 cells with cells rounded up to even) gives
    wa_decode's own bits."""
    from sliding_window_gqa_amd import api
    rng = np.random.default_rng(rows + 3 * d + win)
    pos = rng.integers(0, 3001, size=rows)
    pos[0] = 0
    case = workloads.decode_case("merge", rows, hq, hkv, d, win, ring, streams, pos, seed=rows + d)
    gu.log(f"merge case: {rows}x{hq}/{hkv}x{d} win{win} ring{ring}")
    C = api.lib().wa_decode_chunks(api.window(win, ring), api.INT32_MAX)
    need = api.decode_workspace_bytes(rows, hq, d, win, ring, api.INT32_MAX)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = api.decode(gu.dev_bf16(case.q), gu.dev_bf16(case.k), gu.dev_bf16(case.v),
                     gu.dev_i32(case.stream), gu.dev_i32(case.pos), win, ring, case.scale,
                     workspace=ws)
    cells = rows * hq * C
    cells2 = cells + (cells & 1)
    f = ws.view(torch.float32)
    m = f[:cells].view(rows, hq, C)
    l_ = f[cells2:cells2 + cells].view(rows, hq, C)
    o = f[2 * cells2:2 * cells2 + cells * d].view(rows, hq, C, d)
    merged = api.merge(m, l_, o, gu.dev_i32(case.pos), win, ring)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_bits(merged), gu.host_bits(out))


def test_merge_of_foreign_partials():
    """wa_merge on chunk partials made on the host — per 256-key chunk at absolute positions,
    float64 sums rounded to fp32: m_c the chunk's largest score, l_c and o_c the sums of
    exp(s - m_c) and exp(s - m_c) v — meets the oracle's gate and the literal rule: the merge
    is checked apart from the kernel that usually feeds it."""
    from sliding_window_gqa_amd import api
    rows, hq, hkv, d, win, ring, streams = 9, 4, 2, 256, 700, 1024, 3
    rng = np.random.default_rng(41)
    pos = rng.integers(0, 5000, size=rows)
    pos[:3] = [0, 255, 256]
    case = workloads.decode_case("foreign partials", rows, hq, hkv, d, win, ring, streams, pos,
                                 seed=43, peak_every=2)
    C = api.lib().wa_decode_chunks(api.window(win, ring), api.INT32_MAX)
    G = hq // hkv
    bf = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = np.zeros((rows, hq, C), np.float32)
    l_ = np.zeros((rows, hq, C), np.float32)
    o = np.zeros((rows, hq, C, d), np.float32)
    for r in range(rows):
        p, t = int(case.pos[r]), int(case.stream[r])
        lo = max(0, p - win + 1)
        for h in range(hq):
            qv = bf(case.q[r, h])
            for k in range(p // 256 - lo // 256 + 1):
                c = lo // 256 + k
                js = np.arange(max(lo, 256 * c), min(p, 256 * c + 255) + 1)
                s = float(np.float32(case.scale)) * (bf(case.k[t, js % ring, h // G]) @ qv)
                mc = np.float32(s.max())
                w = np.exp(s - float(mc))
                m[r, h, k], l_[r, h, k] = mc, w.sum()
                o[r, h, k] = w @ bf(case.v[t, js % ring, h // G])
    dev = lambda a: torch.from_numpy(a).cuda()
    merged = api.merge(dev(m), dev(l_), dev(o), gu.dev_i32(case.pos), win, ring)
    torch.cuda.synchronize()
    x, S, _ = gu.oracle_decode(case)
    _, ok = gu.compare(gu.host_bits(merged), x, S, E_P, "merge of host partials")
    assert ok.all()


def test_decode_linear_cache_declared_longer():
    rows = 6
    pos = np.array([0, 100, 255, 256, 700, 999])
    base = workloads.decode_case("linear", rows, 4, 2, 256, 0, 1000, 1, pos, seed=5)
    ref = gu.run_decode(base)
    kl = np.zeros((1, 16000, 2, 256), np.uint16)
    vl = np.zeros_like(kl)
    kl[:, :1000] = base.k
    vl[:, :1000] = base.v
    longer = workloads.DecodeCase("linear x16", base.q, kl, vl, base.stream, base.pos, 0, 16000)
    assert np.array_equal(gu.run_decode(longer), ref)
    x, S, _ = gu.oracle_decode(base)
    assert check.accept(ref, x, S, E_P).all()


def _peak_row(case, r, key, vbits, gap_score=200.0):
    """Make key ``key`` of row r's stream score ~gap_score for every head of the row."""
    t = int(case.stream[r])
    slot = key % case.ring
    G = case.hq // case.hkv
    for g in range(case.hkv):
        qh = (case.q[r, g * G].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        case.k[t, slot, g] = workloads._bf16_bits(qh * (gap_score / (qh @ qh)))
        case.v[t, slot, g] = vbits


def test_decode_mask_edges_bit_exact():
    """Peaked-edge probes: a key at lo and at pos must win outright (out == its v); a key at
    lo - 1 or pos + 1 must not take part at all."""
    win, ring, d = 1024, 1536, 256
    rng = np.random.default_rng(21)
    pos = np.array([1023, 1024, 2047, 5000, 40000, 256 * 57 + 255, 256 * 90, 300])
    rows = len(pos)
    for which in ("lo", "last", "lo-1", "last+1"):
        case = workloads.decode_case("edges", rows, 2, 1, d, win, ring, rows, pos, seed=3,
                                     peak_every=0, stream=np.arange(rows))
        # G = 2 query heads share key head 0: make both heads point the same way
        case.q[:, 1] = case.q[:, 0]
        marks = []
        for r in range(rows):
            lo, last = attend.key_window(int(pos[r]), win)
            key = {"lo": lo, "last": last, "lo-1": lo - 1, "last+1": last + 1}[which]
            if key < 0:
                marks.append(None)
                continue
            vb = workloads._bf16_bits(rng.standard_normal(d) * 4)
            _peak_row(case, r, key, vb)
            marks.append(vb)
        out = gu.run_decode(case)
        x, S, _ = gu.oracle_decode(case)
        assert check.accept(out, x, S, E_P).all(), which
        for r, vb in enumerate(marks):
            if vb is None:
                continue
            hit = np.array_equal(out[r, 0], vb) and np.array_equal(out[r, 1], vb)
            assert hit == (which in ("lo", "last")), (which, r)


def test_decode_integer_sums():
    """Every key alike: every weight is exactly 1, so the output is the exact mean of the
    visible integer values. Values 96..127 make an fp16 running sum overflow and a bf16 one
    drop integers; fp32 holds them exactly."""
    rows, d, win, ring = 3, 256, 1024, 1536
    pos = np.array([1023, 4000, 1500])
    case = workloads.decode_case("sums", rows, 2, 1, d, win, ring, 1, pos, seed=4, peak_every=0)
    case.k[:] = case.k[0, 0, 0]
    slot_vals = 96.0 + (np.arange(ring) * 7) % 32
    case.v[0, :, 0] = workloads._bf16_bits(slot_vals[:, None] * np.ones(d))
    out = gu.run_decode(case)
    for r in range(rows):
        lo, last = attend.key_window(int(pos[r]), win)
        mean = slot_vals[np.arange(lo, last + 1) % ring].sum() / (last - lo + 1)
        want = workloads._bf16_bits(np.array([np.float32(mean)]))[0]
        assert np.all(out[r] == want), r


def _nf_case():
    pos = np.array([100, 300, 301, 600])
    return workloads.decode_case("nonfinite", 4, 4, 2, 256, 256, 700, 1, pos, seed=9, peak_every=0)


def test_decode_nonfinite_classes():
    NAN, PINF, NINF = 0x7FC0, 0x7F80, 0xFF80
    # NaN query: that (row, head) only
    c = _nf_case()
    c.q[1, 2, 7] = NAN
    out = gu.run_decode(c)
    x, S, _ = gu.oracle_decode(c)
    assert check.accept(out, x, S, E_P).all()
    assert np.isnan(x[1, 2]).all()
    # a visible NaN key: the group's heads of the rows that see it
    c = _nf_case()
    c.k[0, 301 % 700, 1, 3] = NAN
    out = gu.run_decode(c)
    x, S, _ = gu.oracle_decode(c)
    assert check.accept(out, x, S, E_P).all()
    # +inf in a value only later rows see
    c = _nf_case()
    c.v[0, 301, 0, 9] = PINF
    out = gu.run_decode(c)
    x, S, _ = gu.oracle_decode(c)
    assert check.accept(out, x, S, E_P).all()
    assert np.isinf(x[2, 0:2, 9]).all() and np.isfinite(x[[0, 1, 3]]).all()
    # opposite infinities sharing one value column
    c = _nf_case()
    c.v[0, 290, 1, 4] = PINF
    c.v[0, 291, 1, 4] = NINF
    out = gu.run_decode(c)
    x, S, _ = gu.oracle_decode(c)
    assert check.accept(out, x, S, E_P).all()


def test_decode_inf_at_negligible_key():
    """fp32's weight e^-200 underflows to 0 and 0 * inf = NaN; float64 keeps e^-200 and gives
    +inf. The float64 re-run of the non-finite (row, head) restores float64's class."""
    c = workloads.decode_case("e-200", 1, 1, 1, 256, 4, 16, 1, [10], seed=2, peak_every=0)
    c.q[0, 0] = workloads._bf16_bits(np.full(256, 1.0))
    c.k[0, 7, 0] = workloads._bf16_bits(np.full(256, 200.0 / 256))
    c.k[0, 8, 0] = workloads._bf16_bits(np.zeros(256))
    c.v[0, 8, 0, 3] = 0x7F80
    out = gu.run_decode(c)
    x, S, _ = gu.oracle_decode(c)
    assert x[0, 0, 3] == np.inf and out[0, 0, 3] == 0x7F80
    assert check.accept(out, x, S, E_P).all()


def test_decode_nonfinite_whole_rows():
    """Non-finite plants in a batch large enough for the whole-row kernel (64 rows x 8 key
    heads, one stream per row): NaN query, visible NaN key, +inf value, opposite infinities in
    the same value column, and an infinite value on a key scoring 200 below the row's peak
    (float64 weight e^-200, fp32 weight 0). Every
    output must be in its interval, with float64's class, and each planted row must have the
    bits it has when computed alone (chunk-partial kernel + merge)."""
    NAN, PINF, NINF = 0x7FC0, 0x7F80, 0xFF80
    case = workloads.decode_12b(streams=64)
    G = case.hq // case.hkv
    lo = lambda r: attend.key_window(int(case.pos[r]), case.win)[0]
    slot = lambda j: j % case.ring
    case.q[3, 5, 11] = NAN
    case.k[9, slot(int(case.pos[9]) - 40), 1, 3] = NAN
    case.v[14, slot(lo(14) + 7), 6, 200] = PINF
    case.v[21, slot(int(case.pos[21])), 2, 4] = PINF
    case.v[21, slot(int(case.pos[21]) - 1), 2, 4] = NINF
    # row 30, key head 4: both query heads all ones; key pos-5 scores 200, key pos-6 scores 0
    r, g = 30, 4
    p = int(case.pos[r])
    case.q[r, g * G:(g + 1) * G] = workloads._bf16_bits(np.full(case.d, 1.0))
    case.k[r, slot(p - 5), g] = workloads._bf16_bits(np.full(case.d, 200.0 / case.d))
    case.k[r, slot(p - 6), g] = workloads._bf16_bits(np.zeros(case.d))
    case.v[r, slot(p - 6), g, 3] = PINF
    gu.log("decode case: whole-row batch with non-finite plants")
    out = gu.run_decode(case)
    x, S, _ = gu.oracle_decode(case)
    assert np.isinf(x[r, g * G, 3]) and x[r, g * G, 3] > 0
    assert check.accept(out, x, S, E_P).all()
    for rr in (3, 9, 14, 21, 30):
        one = workloads.DecodeCase("alone", case.q[rr:rr + 1], case.k[rr:rr + 1], case.v[rr:rr + 1],
                                   np.array([0], np.int32), case.pos[rr:rr + 1], case.win, case.ring)
        assert np.array_equal(gu.run_decode(one)[0], out[rr]), rr


def test_fp32_accumulation_under_cancellation():
    """Decode's fp32 P.V (fma chains in key order, runs summed in run order), measured: q = 0
    gives every key the weight 1, and values in exactly cancelling +/- pairs of magnitudes
    2^-20 .. 2^20 give an exact output of 0 over a 1,024-key window; the output is the
    accumulation error, logged in units of 2^-24 S and held to the strict interval."""
    from tests.test_gpu_prompt import _cancelling_values
    rows, hq, hkv, d, win, ring = 6, 4, 2, 256, 1024, 1024
    rng = np.random.default_rng(43)
    pos = np.array([1023, 1023, 1023, 1023, 1023, 1023])
    case = workloads.decode_case("cancellation", rows, hq, hkv, d, win, ring, rows, pos, seed=43,
                                 peak_every=0)
    case.q[:] = 0
    for t in range(rows):
        case.v[t] = _cancelling_values(rng, ring, hkv, d)
    out = gu.run_decode(case)
    x, S, _ = gu.oracle_decode(case)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    worst = float(np.max(np.abs(got - x) / S))
    gu.log(f"[decode fp32 accumulation] worst |out - x| / S = {worst:.3e} = {worst * 2 ** 24:.1f} x 2^-24")
    assert check.accept(out, x, S, E_P, "S").all()


@pytest.mark.parametrize("rows,win,ring,streams,d", [
    (5, 64, 64, 2, 256),        # small chunk grid
    (5, 64, 64, 2, 128),
    (600, 64, 256, 3, 256),     # large chunk grid (1,200 workgroups), rings shared by rows
    (1100, 64, 256, 3, 128),
    (256, 64, 256, 256, 256),   # whole rows: 256 rows, each in its own stream
])
def test_slot_stride_at_the_31_bit_limit(rows, win, ring, streams, d):
    """K/V slots as far apart as wa_decode accepts (the ring's span a few hundred KB under
    2^31 bytes): the rows match the oracle and the same rings laid out densely, bit for bit."""
    from sliding_window_gqa_amd import api
    rng = np.random.default_rng(rows + ring)
    pos = rng.integers(0, 5000, size=rows)
    pos[0] = 0
    case = workloads.decode_case("far slots", rows, 2, 1, d, win, ring, streams, pos,
                                 seed=rows + 7, peak_every=2)
    sslot = gu.limit_slot_stride(ring - 1, d)
    label = f"decode far slots {rows} rows x{d} ring{ring} streams{streams} slot stride {sslot}"
    gu.log(f"decode case: {label}")
    k, v = gu.far_slots(case.k, sslot), gu.far_slots(case.v, sslot)
    assert (ring - 1) * k.stride(1) * 2 + 2 * d < 2**31 - 1 < (ring - 1) * (k.stride(1) + 8) * 2 + 2 * d
    out = api.decode(gu.dev_bf16(case.q), k, v, gu.dev_i32(case.stream), gu.dev_i32(case.pos),
                     win, ring, case.scale)
    torch.cuda.synchronize()
    bits = gu.host_bits(out)
    del k, v, out
    x, S, _ = gu.oracle_decode(case)
    _, ok = gu.compare(bits, x, S, E_P, label)
    assert ok.all()
    assert np.array_equal(bits, gu.run_decode(case))


@pytest.mark.parametrize("scale", [-0.8, 0.0])
@pytest.mark.parametrize("d", [256, 128])
def test_negative_and_zero_scale(scale, d):
    """The score scale is any finite float32: a negative one turns the peaked keys into the
    least weighted, zero gives every visible key the same weight (the mean of their v)."""
    rng = np.random.default_rng(11 + d)
    pos = rng.integers(0, 3000, size=7)
    case = workloads.decode_case("scale", 7, 4, 2, d, 300, 700, 2, pos, seed=d + 3, scale=scale,
                                 peak_every=2)
    _gate(case, f"decode scale {scale} d{d}")

