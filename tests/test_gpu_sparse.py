"""GPU parity of the block-sparse prompt (wa_prompt_sparse) against the float64 oracle.

TensorFold pull request #1622, "What this changes": per-row block masks over the union of a
row group's selected blocks, causal ends, fp32 online softmax and the parts/merge layout.
Gate: every bf16 output inside its tier-G interval, with e_P by P's representation; P as
three parts (the page's fp32 tile) must also meet the strict interval of fp32 P. Block
visibility is pinned bit for bit by peaked-edge probes; a row's bits must not depend on the
other rows of its call (their selections change the union the workgroup walks) nor on how
the prompt is cut; every block selected reproduces wa_prompt's bits where both take the same
kernel (head dim 128) and meets the oracle's gate where they do not (256).
"""

import numpy as np
import pytest
import torch

from oracle import attend, check
from sliding_window_gqa_amd import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

E_P = {0: check.E_P_BF16, 1: check.E_P_P32, 2: check.E_P_THREE}
B = workloads.SPARSE_BLOCK


def _gate(case, label, p32=None, strict=None):
    p32 = case.p32 if p32 is None else int(p32)
    gu.log(f"sparse case: {label} n={case.n} p0={case.p0} hq={case.hq} hkv={case.hkv} d={case.d} "
           f"win={case.win} ring={case.ring} p32={p32} words={case.masks.shape[1]}")
    out = gu.run_sparse(case, p32=p32)
    x, S, _ = gu.oracle_sparse(case)
    rep, ok = gu.compare(out, x, S, E_P[p32], label)
    assert ok.all()
    if strict if strict is not None else p32 == 2:
        assert rep["tier_S_fail"] == 0, rep
    return out


def test_sparse_prompt_workload():
    _gate(workloads.sparse_prompt(), "sparse 64 rows (24/2)x256, 32 blocks a row, three parts")


@pytest.mark.parametrize("p32", [0, 1])
def test_sparse_prompt_workload_p_modes(p32):
    _gate(workloads.sparse_prompt(), f"sparse workload p32={p32}", p32=p32)


@pytest.mark.parametrize("n,hq,hkv,d,p0,nsel,win", [
    (17, 6, 1, 256, 900, 4, 0),        # the page's 17-row tail, 6/1 heads
    (64, 24, 2, 256, 3000, 48, 0),     # more blocks than half the prefix
    (40, 8, 8, 128, 1500, 6, 0),       # d 128, one query head per key head
    (130, 16, 8, 256, 5000, 10, 1024), # a window narrows the selection
])
def test_sparse_shapes(n, hq, hkv, d, p0, nsel, win):
    case = workloads.sparse_prompt_case("sparse shape", n, hq, hkv, d, p0, nsel, seed=n + p0, win=win)
    if win:
        case.ring = 1536
        case.k, case.v = case.k[p0 + n - 1536:p0 + n], case.v[p0 + n - 1536:p0 + n]
        # ring slot j mod 1536 holds key j: rotate the linear cache into the ring
        shift = (p0 + n - 1536) % 1536
        case.k = np.roll(case.k, shift, axis=0)
        case.v = np.roll(case.v, shift, axis=0)
    _gate(case, f"sparse n{n} {hq}/{hkv}x{d} p0={p0} nsel={nsel} win{win}")


@pytest.mark.parametrize("d", [128, 256])
def test_every_block_selected_gives_wa_prompt(d):
    """Every block selected: at head dim 128 the sparse and the dense windowed prompt take the
    same kernel and chunk layout, so the bits must be equal; at 256 the dense prompt takes
    the quarter-tile kernel (a different fp32 order), so both are held to the oracle."""
    for p32 in (0, 1, 2):
        case = workloads.prompt_case("dense", 200, 16, 8, d, 5000, 1024, 1536, seed=9, p32=p32)
        case.masks = np.full((case.n, 4), 0xFFFFFFFF, np.uint32)   # blocks 0..127
        case.hi = case.p0 + np.arange(case.n)
        case.hi[20:60] = case.p0 + 59
        dense = gu.run_prompt(case)
        sparse = gu.run_sparse(case)
        if d == 128:
            assert np.array_equal(sparse, dense), p32
        else:
            x, S, _ = gu.oracle_sparse(case)
            gu.compare(dense, x, S, E_P[p32], f"dense, every block, p32={p32}")
            gu.compare(sparse, x, S, E_P[p32], f"sparse, every block, p32={p32}")


def test_short_ring_blocks():
    """A ring shorter than one block: keys 53..67 over 15 slots, rows selecting block 0 or
    both blocks, against the oracle."""
    case = workloads.prompt_case("sparse short ring", 8, 2, 1, 256, 60, 8, 15, seed=12, p32=2,
                                 peak_every=2)
    case.masks = np.zeros((case.n, 1), np.uint32)
    case.masks[0::2, 0] = 0x1
    case.masks[1::2, 0] = 0x3
    _gate(case, "sparse short ring")


def test_rows_independent_of_the_other_rows_and_cuts():
    case = workloads.sparse_prompt()
    full = gu.run_sparse(case)
    # other rows' selections change the union their workgroup walks, not row 5's bits
    masks = case.masks.copy()
    masks[np.arange(case.n) != 5] = 0xFFFFFFFF
    assert np.array_equal(gu.run_sparse(case, masks=masks)[5], full[5])
    masks = case.masks.copy()
    masks[np.arange(case.n) != 5] = 0
    masks[np.arange(case.n) != 5, -1] = case.masks[np.arange(case.n) != 5, -1]   # own blocks only
    assert np.array_equal(gu.run_sparse(case, masks=masks)[5], full[5])
    for cut in (1, 5, 6, 31, 63):
        a = gu.run_sparse(case, rows=(0, cut))
        b = gu.run_sparse(case, rows=(cut, case.n))
        assert np.array_equal(np.concatenate([a, b]), full), cut
    for _ in range(3):
        assert np.array_equal(gu.run_sparse(case), full)


def test_block_edges_bit_exact():
    """A key with a score lead of 200 at the first or last key of a selected block wins
    outright; at the last key of the unselected block before it, or the first key of the
    unselected block after it, it takes no part."""
    n, p0, d = 48, 5000, 256
    rng = np.random.default_rng(17)
    for which in ("first", "last", "before", "after"):
        case = workloads.sparse_prompt_case("edges", n, 1, 1, d, p0, 1, seed=23, peak_every=0)
        masks = np.zeros_like(case.masks)
        marks = {}
        for i in range(0, n, 3):
            bsel = 5 + 4 * (i // 3)                  # blocks 5, 9, .., 65: before p0, and
            #                                          no row selects another's neighbours
            masks[i, bsel // 32] |= np.uint32(1 << (bsel % 32))
            own = (p0 + i) // B
            masks[i, own // 32] |= np.uint32(1 << (own % 32))
            key = {"first": B * bsel, "last": B * bsel + B - 1,
                   "before": B * bsel - 1, "after": B * bsel + B}[which]
            qh = (case.q[i, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            case.k[key, 0] = workloads._bf16_bits(qh * (200.0 / (qh @ qh)))
            vb = workloads._bf16_bits(rng.standard_normal(d) * 4)
            case.v[key, 0] = vb
            marks[i] = vb
        case.masks = masks
        out = gu.run_sparse(case)
        x, S, _ = gu.oracle_sparse(case)
        assert check.accept(out, x, S, E_P[2]).all(), which
        for i, vb in marks.items():
            hit = np.array_equal(out[i, 0], vb)
            assert hit == (which in ("first", "last")), (which, i)


def test_nonfinite_only_through_selected_blocks():
    case = workloads.sparse_prompt_case("nonfinite", 40, 4, 2, 256, 1000, 3, seed=29, peak_every=0)
    masks = np.zeros_like(case.masks)
    for i in range(case.n):
        own = (case.p0 + i) // B
        for b in (2, own) if i < 20 else (2, 3, own):
            masks[i, b // 32] |= np.uint32(1 << (b % 32))
    case.masks = masks
    case.k[3 * B + 7, 1, 9] = 0x7FC0        # NaN key in block 3: rows 20..39, key head 1
    case.v[2 * B + 1, 0, 4] = 0x7F80        # +inf value in block 2 (every row), key head 0
    out = gu.run_sparse(case)
    x, S, _ = gu.oracle_sparse(case)
    assert np.isnan(x[20:, 2:4]).all() and np.isfinite(x[:20, 2:4]).all()
    assert np.isposinf(x[:, 0:2, 4]).all()
    assert check.accept(out, x, S, E_P[2]).all()


def test_row_that_sees_no_key_is_nan():
    case = workloads.sparse_prompt_case("empty", 24, 4, 2, 256, 700, 2, seed=31, peak_every=0)
    case.masks[7] = 0
    case.masks[7, 0] = np.uint32(1 << 20)   # block 20 = keys 1280..1343: after row 7's position
    out = gu.run_sparse(case)
    x, S, _ = gu.oracle_sparse(case)
    assert np.isnan(x[7]).all()
    assert check.accept(out, x, S, E_P[2]).all()


def test_sparse_slot_stride_at_the_31_bit_limit():
    """The block-sparse prompt (d = 256) with its slots as far apart as wa_prompt_sparse
    accepts, against the oracle and the dense layout."""
    from sliding_window_gqa_amd import api
    d = 256
    case = workloads.sparse_prompt_case("far slots sparse", 28, 4, 2, d, 100, 2, seed=29)
    sslot = gu.limit_slot_stride(63, d)
    label = f"sparse far slots slot stride {sslot}"
    gu.log(f"prompt case: {label}")
    k, v = gu.far_slots(case.k, sslot), gu.far_slots(case.v, sslot)
    m = torch.from_numpy(np.ascontiguousarray(case.masks).view(np.int32)).cuda()
    out = api.prompt_sparse(gu.dev_bf16(case.q), k, v, case.p0, case.win, case.ring, m, case.scale,
                            p32=case.p32)
    torch.cuda.synchronize()
    bits = gu.host_bits(out)
    del k, v, out
    x, S, _ = gu.oracle_sparse(case)
    _, ok = gu.compare(bits, x, S, E_P[int(case.p32)], label)
    assert ok.all()
    assert np.array_equal(bits, gu.run_sparse(case))


@pytest.mark.parametrize("scale", [-0.8, 0.0])
@pytest.mark.parametrize("d", [256, 128])
def test_negative_and_zero_scale(scale, d):
    """Any finite float32 score scale through the block-sparse walk."""
    case = workloads.sparse_prompt_case("scale", 24, 4, 2, d, 700, 4, seed=d + 9)
    case.scale = scale
    _gate(case, f"sparse scale {scale} d{d}")

