"""Pins for the oracle's block-sparse prompt (``attend.sparse_prompt``, ``attend.visible_keys``).

TensorFold pull request #1622, "What this changes": per-row block masks and causal ends over
the union of a row group's selected blocks. The oracle's visibility rule is checked against a
plain enumeration written with Python integers, its values against brute force (exact
rational scores, 60-digit exponentials), and against closed forms and invariants: every
block selected is the dense prompt; a contiguous run of blocks ending at the row is a window;
a row whose only visible key is one key returns that key's v; a NaN or infinity in a block a
row did not select does not reach it, one in a selected block does; a row that sees no key
is NaN.
"""

import numpy as np
import pytest

from oracle import attend
from sliding_window_gqa_amd import workloads
from tests.test_oracle_attend import brute_row_head, mpf_to_bits, rand_bf16, rational_bits

B = 64


def selected(mask, j):
    """Key j's block bit, by Python integers."""
    b = j // B
    w = b // 32
    return w < len(mask) and (int(mask[w]) >> (b % 32)) & 1 == 1


def test_visible_keys_match_enumeration():
    rng = np.random.default_rng(21)
    for _ in range(300):
        words = int(rng.integers(1, 4))
        mask = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
        mask &= rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
        pos = int(rng.integers(0, 64 * 32 * words + 200))
        win = int(rng.choice([0, 1, 63, 64, 65, 500]))
        last = pos + int(rng.integers(0, 100)) if rng.random() < 0.3 else None
        lo, hi = attend.key_window(pos, win, last)
        want = [j for j in range(0, hi + 1) if j >= lo and selected(mask, j)]
        got = attend.visible_keys(pos, win, last, mask).tolist()
        assert got == want


def test_sparse_prompt_matches_brute_force():
    rng = np.random.default_rng(31)
    n, Hq, Hkv, d, p0 = 5, 4, 2, 4, 180
    ring = p0 + n
    q = rand_bf16(rng, (n, Hq, d))
    kr = rand_bf16(rng, (ring, Hkv, d), 0.5)
    vr = rand_bf16(rng, (ring, Hkv, d))
    masks = np.zeros((n, 1), np.uint32)
    masks[:, 0] = [0b1001, 0b0110, 0b1111, 0b1100, 0b0101]   # blocks of keys 0..255
    x, Sx, out = attend.sparse_prompt(q, kr, vr, p0, 0, ring, 0.8, masks)
    for i in range(n):
        keys = [j for j in range(p0 + i + 1) if selected(masks[i], j)]
        for h in range(Hq):
            # brute force over exactly the selected keys: a ring holding only those keys
            kk = kr[keys][None]
            vv = vr[keys][None]
            xs = brute_row_head(q[i], kk, vv, 0, len(keys) - 1, len(keys) - 1, 0, len(keys), h, 0.8)
            for dd in range(d):
                bits, near = rational_bits(mpf_to_bits(xs[dd]))
                assert abs(x[i, h, dd] - float(xs[dd])) <= 1e-13 * max(1.0, Sx[i, h, dd])
                if not near:
                    assert out[i, h, dd] == bits


def test_every_block_selected_is_the_dense_prompt():
    case = workloads.prompt_case("dense", 40, 4, 2, 16, 300, 100, 400, seed=3)
    full = np.full((case.n, 8), 0xFFFFFFFF, np.uint32)
    xs, Ss, _ = attend.sparse_prompt(case.q, case.k, case.v, case.p0, case.win, case.ring, 1.0, full)
    xd, Sd, _ = attend.prompt(case.q, case.k, case.v, case.p0, case.win, case.ring, 1.0)
    assert np.array_equal(xs, xd) and np.array_equal(Ss, Sd)


def test_contiguous_blocks_are_a_window():
    case = workloads.prompt_case("run", 30, 2, 1, 16, 500, 0, 530, seed=4)
    masks = np.zeros((case.n, 1), np.uint32)
    for i in range(case.n):
        own = (case.p0 + i) // B                       # blocks 5..8 (keys 320..575)
        for b in range(own - 2, own + 1):
            masks[i, 0] |= np.uint32(1 << b)
    xs, _, _ = attend.sparse_prompt(case.q, case.k, case.v, case.p0, 0, case.ring, 1.0, masks)
    for i in range(case.n):
        p = case.p0 + i
        win = p - B * ((p // B) - 2) + 1
        xw, _, _ = attend.prompt(case.q, case.k, case.v, case.p0, win, case.ring, 1.0, rows=[i])
        assert np.array_equal(xs[i], xw[0])


def test_one_visible_key_returns_its_v():
    # row at position 64b selecting only its own block sees exactly one key
    case = workloads.prompt_case("one key", 3, 2, 1, 256, 640, 0, 643, seed=5)
    masks = np.zeros((3, 1), np.uint32)
    masks[:, 0] = 1 << 10
    _, _, out = attend.sparse_prompt(case.q, case.k, case.v, case.p0, 0, case.ring, 1.0, masks)
    assert np.array_equal(out[0, 0], case.v[640, 0]) and np.array_equal(out[0, 1], case.v[640, 0])
    assert not np.array_equal(out[1, 0], case.v[640, 0])


def test_nonfinite_only_through_selected_blocks():
    case = workloads.prompt_case("nan", 8, 2, 1, 16, 200, 0, 208, seed=6)
    masks = np.zeros((8, 1), np.uint32)
    masks[:4, 0] = 0b1001          # blocks 0 and 3 (keys 0..63, 192..255)
    masks[4:, 0] = 0b1011          # also block 1
    case.k[70, 0, 3] = 0x7FC0      # NaN key in block 1
    case.v[10, 0, 5] = 0x7F80      # +inf value in block 0, seen by every row
    x, _, _ = attend.sparse_prompt(case.q, case.k, case.v, case.p0, 0, case.ring, 1.0, masks)
    assert np.isfinite(np.delete(x[:4], 5, axis=-1)).all()
    assert np.isposinf(x[:4, :, 5]).all()
    assert np.isnan(x[4:]).all()


def test_row_seeing_no_key_is_nan():
    case = workloads.prompt_case("empty", 4, 2, 1, 16, 100, 0, 104, seed=7)
    masks = np.zeros((4, 1), np.uint32)
    masks[1:, 0] = 0b10            # block 1 = keys 64..127; row 0 selects nothing
    x, S, out = attend.sparse_prompt(case.q, case.k, case.v, case.p0, 0, case.ring, 1.0, masks)
    assert np.isnan(x[0]).all() and np.isfinite(x[1:]).all()


def test_workload_masks():
    rng = np.random.default_rng(1)
    m = workloads.block_masks(rng, 64, 7836, 32)
    counts = np.array([sum(bin(int(w)).count("1") for w in row) for row in m])
    assert (counts == 32).all()
    own = (7836 + np.arange(64)) // B
    assert all(selected(m[i], B * own[i]) for i in range(64))
    assert not any(selected(m[i], B * (own[i] + 1)) for i in range(64))
