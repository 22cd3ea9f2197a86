"""GPU parity of the q/k row preparation (wa_prepare) against the float64 oracle.

Gate: every bf16 output inside the set of values the oracle's interval propagation allows
at the last rounding point (oracle.prepare), which is one value for all but about 1e-3 of
the outputs. Sources: TensorFold pull request #1257, "What this changes" and "Kernel
contract" (16 query heads over 4 key heads at d = 256, a third of the rows past position
199,800); the "Exact Numerical Contract" page, "Preparation" (d = 128, RMSNorm, RoPE on dims
0-95 with bf16 coefficients).
"""

import numpy as np
import pytest
import torch

from oracle import bf16, prepare as P
from sliding_window_gqa_amd import api, workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MODES = {P.ROPE_L2: api.PREP_ROPE_L2, P.RMS_ROPE: api.PREP_RMS_ROPE}


def _run(case, mode, x_dev=None, **kw):
    x = gu.dev_bf16(case.x) if x_dev is None else x_dev
    qs = None if case.qs is None else torch.from_numpy(case.qs).cuda()
    out = api.prepare(x, gu.dev_i32(case.pos), MODES[mode], case.rope_dims, case.theta, qs=qs, **kw)
    torch.cuda.synchronize()
    return out


def _gate(case, mode, label):
    gu.log(f"prepare case: {label} rows={case.x.shape[0]} heads={case.x.shape[1]} d={case.x.shape[2]} "
           f"R={case.rope_dims} qs={case.qs is not None}")
    out = gu.host_bits(_run(case, mode))
    lo, hi = P.interval(mode, case.x, case.pos, case.rope_dims, case.theta, qs=case.qs)
    ok = P.accept(out, lo, hi)
    pt = P.point(mode, case.x, case.pos, case.rope_dims, case.theta, qs=case.qs)
    gu.log(f"  {label}: {int((~ok).sum())} outside of {ok.size}; equal to the point value: "
           f"{int((out == pt).sum())}; two-value sets: {int((lo != hi).sum())}")
    assert ok.all()
    return out


def test_l2_recipe_q_with_scale_and_k():
    # pull request #1257's shape: 16 query heads over 4 key heads at d = 256
    _gate(workloads.prep_case("q l2", 96, 16, 256, 256, seed=201, with_qs=True), P.ROPE_L2, "q, L2 + scale")
    _gate(workloads.prep_case("k l2", 96, 4, 256, 256, seed=202), P.ROPE_L2, "k, L2")


def test_rms_recipe_partial_rotation():
    # the contract page's shape: d = 128, rotation on dims 0-95 only
    _gate(workloads.prep_case("rms", 64, 56, 128, 96, seed=203), P.RMS_ROPE, "RMS, R = 96")


@pytest.mark.parametrize("mode,d,R", [(P.ROPE_L2, 128, 128), (P.ROPE_L2, 256, 64), (P.RMS_ROPE, 256, 256),
                                      (P.ROPE_L2, 256, 0), (P.RMS_ROPE, 128, 0)])
def test_other_shapes(mode, d, R):
    _gate(workloads.prep_case("shape", 33, 5, d, R, seed=210 + d + R), mode, f"{mode} d={d} R={R}")


def test_position_zero_and_zero_heads():
    c = workloads.prep_case("edge", 8, 3, 256, 256, seed=220, pos=np.zeros(8, np.int64))
    c.x[2, 1] = 0                      # an all-zero head stays zero
    out = _gate(c, P.ROPE_L2, "pos 0, zero head")
    assert np.all(bf16.to_f64(out[2, 1]) == 0.0)


def test_strided_input_view():
    # the interleaved projection buffer of the long prompt: q, k at column offsets 0, heads*d
    c = workloads.prep_case("strided", 40, 6, 128, 96, seed=230)
    rows, heads, d = c.x.shape
    buf = np.zeros((rows, 3 * heads * d), np.uint16)
    buf[:, heads * d:2 * heads * d] = c.x.reshape(rows, -1)
    dev = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).cuda()
    view = dev[:, heads * d:2 * heads * d].view(rows, heads, d)
    out = gu.host_bits(_run(c, P.RMS_ROPE, x_dev=view))
    lo, hi = P.interval(P.RMS_ROPE, c.x, c.pos, 96, c.theta)
    assert P.accept(out, lo, hi).all()


def test_ring_write_and_copy():
    """k prepared straight into its ring slot (pos mod ring of the row's stream), v copied
    as it is; every other slot keeps its sentinel; same bits as the plain-row output."""
    rows, heads, d, ring, streams = 24, 4, 256, 40, 3
    # slots (120 + 5 r) mod 40 repeat every 8 rows, streams r mod 3 every 3: no two rows of
    # a stream share a slot
    c = workloads.prep_case("ring", rows, heads, d, d, seed=240, pos=120 + 5 * np.arange(rows))
    st = np.arange(rows) % streams
    plain = gu.host_bits(_run(c, P.ROPE_L2))
    sentinel = 0x3F80
    cache = torch.full((streams, ring, heads, d), 1.0, dtype=torch.bfloat16, device="cuda")
    vcache = cache.clone()
    x = gu.dev_bf16(c.x)
    api.prepare(x, gu.dev_i32(c.pos), api.PREP_ROPE_L2, d, c.theta, out=cache,
                stream_of_row=gu.dev_i32(st), ring=ring)
    api.prepare(x, gu.dev_i32(c.pos), api.PREP_COPY, out=vcache, stream_of_row=gu.dev_i32(st), ring=ring)
    torch.cuda.synchronize()
    kc, vc = gu.host_bits(cache), gu.host_bits(vcache)
    touched = np.zeros((streams, ring), bool)
    for r in range(rows):
        t, s = st[r], c.pos[r] % ring
        assert not touched[t, s]
        touched[t, s] = True
        assert np.array_equal(kc[t, s], plain[r]) and np.array_equal(vc[t, s], c.x[r])
    assert np.all(kc[~touched] == sentinel) and np.all(vc[~touched] == sentinel)


def test_repeat_is_bit_identical_and_nan_stays_in_its_head():
    c = workloads.prep_case("rep", 16, 8, 256, 256, seed=250, with_qs=True)
    a = gu.host_bits(_run(c, P.ROPE_L2))
    for _ in range(3):
        assert np.array_equal(gu.host_bits(_run(c, P.ROPE_L2)), a)
    c.x[5, 2, 17] = 0x7FC0             # NaN in one head: that head is all NaN, no other moves
    b = gu.host_bits(_run(c, P.ROPE_L2))
    assert bf16.is_nan(b[5, 2]).all()
    mask = np.ones(b.shape[:2], bool)
    mask[5, 2] = False
    assert np.array_equal(b[mask], a[mask])


@pytest.mark.parametrize("mode,d,R", [(P.RMS_ROPE, 128, 40), (P.ROPE_L2, 256, 72)])
def test_rotation_width_not_whole_lanes(mode, d, R):
    # R not a multiple of 16: the partner of a dim is not a whole number of 8-dim lanes away,
    # so the 2- or 4-dims-a-lane form runs; same gate
    _gate(workloads.prep_case("narrow", 21, 7, d, R, seed=260 + R, with_qs=mode == P.ROPE_L2), mode,
          f"{mode} d={d} R={R} (narrow form)")


def test_head_stride_not_16_byte_aligned():
    # heads 132 elements apart (264 bytes): not 16-byte aligned, so the narrow form runs; its
    # bits pass the gate and rows that fit both forms agree with the aligned call's gate too
    c = workloads.prep_case("stride132", 30, 5, 128, 96, seed=270)
    rows, heads, d = c.x.shape
    buf = np.zeros((rows, heads, d + 4), np.uint16)
    buf[:, :, :d] = c.x
    dev = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).cuda()
    view = dev[:, :, :d]
    assert view.stride(1) == d + 4
    out = gu.host_bits(_run(c, P.RMS_ROPE, x_dev=view))
    lo, hi = P.interval(P.RMS_ROPE, c.x, c.pos, 96, c.theta)
    assert P.accept(out, lo, hi).all()
