"""Helpers shared by the GPU tests: move seeded inputs to the device, call the library
through its binding, and compare with the float64 oracle."""

import json
import os
import sys

import numpy as np
import torch

from oracle import attend, check


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a):
    """uint16 numpy array (any strides) -> bf16 CUDA tensor with the same element strides."""
    a = np.asarray(a)
    if a.base is not None and not a.flags.c_contiguous:
        raise ValueError("use dev_view for strided views")
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_view(buf_dev, view, base_np):
    """Strided bf16 CUDA view of ``buf_dev`` matching the numpy view ``view`` of ``base_np``."""
    item = base_np.itemsize
    off = (view.__array_interface__["data"][0] - base_np.__array_interface__["data"][0]) // item
    return torch.as_strided(buf_dev, view.shape, [s // item for s in view.strides], off)


def far_slots(arr, slot_elems):
    """Device copy of a K or V array ([streams, ring, Hkv, d] or [ring, Hkv, d]) whose ring
    slots lie ``slot_elems`` elements apart, the streams and key heads side by side at the
    start of each slot: a layout whose slot span reaches the loads' 2^31-byte offset limit
    with a short ring."""
    a = np.asarray(arr)
    if a.ndim == 3:
        return far_slots(a[None], slot_elems)[0]
    s, ring, hkv, d = a.shape
    assert s * hkv * d <= slot_elems and slot_elems % 8 == 0
    buf = torch.zeros(ring * slot_elems, dtype=torch.bfloat16, device="cuda")
    view = buf.as_strided((s, ring, hkv, d), (hkv * d, slot_elems, d, 1))
    view.copy_(dev_bf16(a))
    return view


def limit_slot_stride(span_slots, d):
    """Largest slot stride (elements, a multiple of 8) for which ``span_slots`` slot strides
    plus one row of d stay under 2^31 bytes: the largest the library accepts."""
    return ((2**31 - 2 - 2 * d) // (2 * span_slots)) // 8 * 8


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_decode(case, **kw):
    from sliding_window_gqa_amd import api
    out = api.decode(dev_bf16(case.q), dev_bf16(case.k), dev_bf16(case.v), dev_i32(case.stream),
                     dev_i32(case.pos), case.win, case.ring, case.scale, **kw)
    torch.cuda.synchronize()
    return host_bits(out)


def run_prompt(case, p32=None, rows=None):
    """Run a prompt case; ``rows`` = (a, b) runs only rows a..b-1 as their own call."""
    from sliding_window_gqa_amd import api
    p32 = case.p32 if p32 is None else p32
    a, b = (0, case.n) if rows is None else rows
    if case.buffer is not None:
        buf = torch.from_numpy(case.buffer.view(np.int16)).view(torch.bfloat16).cuda()
        q = dev_view(buf, case.q, case.buffer)[a:b]
        k = dev_view(buf, case.k, case.buffer)
        v = dev_view(buf, case.v, case.buffer)
    else:
        q = dev_bf16(case.q)[a:b]
        k = dev_bf16(case.k)
        v = dev_bf16(case.v)
    hi = None if case.hi is None else dev_i32(case.hi[a:b])
    out = api.prompt(q, k, v, case.p0 + a, case.win, case.ring, case.scale, hi=hi, p32=p32)
    torch.cuda.synchronize()
    return host_bits(out)


def oracle_decode(case, rows=None):
    return attend.decode(case.q, case.k, case.v, case.stream, case.pos, case.win, case.ring,
                         case.scale, rows=rows)


def oracle_prompt(case, rows=None):
    return attend.prompt(case.q, case.k, case.v, case.p0, case.win, case.ring, case.scale,
                         hi=case.hi, rows=rows)


def _record(label, e_p, rep):
    """Append one case's counts to the JSON-lines file named by WA_PARITY_LOG, if set."""
    path = os.environ.get("WA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, "e_P": e_p, **rep}) + "\n")


def compare(out, x, S, e_p, label):
    """Gate: every output inside its tier-G interval. Where P is fp32 to 2**-16 or better
    (e_P <= 2**-16), also the literal one-ulp rule: every output outside {bf16(x) and its two
    neighbours} must be a cancelling one, |x| / S < check.literal_bound(e_P). The counts
    (equal, within one step, outside, worst |x| / S outside) are logged and recorded."""
    rep = check.report(out, x, S, e_p)
    msg = (f"[{label}] n={rep['n']} equal={rep['equal']} within1ulp={rep['within_1ulp']} "
           f"outside={rep['outside']} worst|x|/S={rep['worst_x_over_S']:.3g} "
           f"tierG_fail={rep['tier_G_fail']} tierS_fail={rep['tier_S_fail']}")
    log(msg)
    _record(label, e_p, rep)
    ok = check.accept(out, x, S, e_p, "G")
    if not ok.all():
        bad = np.argwhere(~ok)[:10]
        for idx in bad:
            t = tuple(idx)
            log(f"  fail at {t}: out=0x{int(out[t]):04x} x={x[t]!r} S={S[t]!r}")
    if e_p <= check.E_P_P32:
        assert rep["worst_x_over_S"] < check.literal_bound(e_p), "literal rule: " + msg
    return rep, ok


def run_sparse(case, p32=None, rows=None, masks=None):
    """Run a block-sparse prompt case (``case.masks``, or ``masks``); ``rows`` = (a, b)
    runs only rows a..b-1 as their own call."""
    from sliding_window_gqa_amd import api
    p32 = case.p32 if p32 is None else p32
    masks = case.masks if masks is None else masks
    a, b = (0, case.n) if rows is None else rows
    q = dev_bf16(case.q)[a:b]
    k = dev_bf16(case.k)
    v = dev_bf16(case.v)
    hi = None if case.hi is None else dev_i32(case.hi[a:b])
    m = torch.from_numpy(np.ascontiguousarray(masks[a:b]).view(np.int32)).cuda()
    out = api.prompt_sparse(q, k, v, case.p0 + a, case.win, case.ring, m, case.scale, hi=hi, p32=p32)
    torch.cuda.synchronize()
    return host_bits(out)


def oracle_sparse(case, rows=None, masks=None):
    return attend.sparse_prompt(case.q, case.k, case.v, case.p0, case.win, case.ring, case.scale,
                                case.masks if masks is None else masks, hi=case.hi, rows=rows)
