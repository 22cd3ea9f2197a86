"""The C-ABI library loads, exports every entry point include/wa.h declares, sizes the decode
workspace, and rejects host-checkable mistakes before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest

from sliding_window_gqa_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="libwa.so not built")

WA_OK, WA_EARG, WA_EUNSUPPORTED, WA_ERANGE, WA_EWORKSPACE, WA_EHIP = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # never dereferenced: every call below returns before a launch


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(wa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared()
    assert set(names) >= {"wa_decode", "wa_prompt", "wa_merge", "wa_decode_workspace",
                          "wa_decode_chunks", "wa_status_string", "wa_version"}
    L = ctypes.CDLL(api.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(api.SIGNATURES)


def test_version_and_status_strings():
    L = api.lib()
    assert b"gfx950" in L.wa_version()
    for s in (WA_OK, WA_EARG, WA_EUNSUPPORTED, WA_ERANGE, WA_EWORKSPACE, WA_EHIP):
        assert L.wa_status_string(s)
    assert L.wa_status_string(12345) == b"unknown status"


def test_chunks_and_workspace():
    L = api.lib()
    w = api.window(1024, 1536)
    assert L.wa_decode_chunks(ctypes.byref(w), 40000) == 5
    w64 = api.window(64, 300)
    assert L.wa_decode_chunks(ctypes.byref(w64), 299) == 2
    w256 = api.window(256, 300)
    assert L.wa_decode_chunks(ctypes.byref(w256), 299) == 2
    w257 = api.window(257, 300)            # keys lo..lo+256 touch at most 2 chunks
    assert L.wa_decode_chunks(ctypes.byref(w257), 299) == 2
    w258 = api.window(258, 300)            # lo = 255: keys 255..512 touch chunks 0, 1, 2
    assert L.wa_decode_chunks(ctypes.byref(w258), 299) == 3
    lin = api.window(0, 300)
    assert L.wa_decode_chunks(ctypes.byref(lin), 299) == 2
    assert L.wa_decode_chunks(ctypes.byref(lin), 255) == 1
    # 64 rows x 16 heads x 5 chunks x (m, l, 256 dims) fp32
    assert L.wa_decode_workspace(64, 16, 256, ctypes.byref(w), 0) == 64 * 16 * 5 * 258 * 4
    assert L.wa_decode_workspace(64, 16, 100, ctypes.byref(w), 0) == 0
    # an odd cell count (7 x 3 x 3): m and l take 64 floats each so that o is 16-byte aligned
    w300 = api.window(300, 700)
    assert L.wa_decode_workspace(7, 3, 256, ctypes.byref(w300), 0) == (2 * 64 + 63 * 256) * 4
    bad = api.window(-1, 10)
    assert L.wa_decode_workspace(1, 1, 256, ctypes.byref(bad), 0) == 0


def _decode(w, rows=2, hq=4, hkv=2, d=256, max_pos=100, ws_bytes=1 << 30, ptr=FAKE,
            streams=1, strides=(1024, 256, 0, 512, 256), ws=None):
    L = api.lib()
    qs, qh, sst, ssl, sh = strides
    ws = ptr if ws is None else ws
    return L.wa_decode(ctypes.byref(w), ptr, qs, qh, ptr, ptr, sst, ssl, sh, streams,
                       ptr, ptr, max_pos, rows, hq, hkv, d, ws, ws_bytes, ptr, qs, qh, None)


def test_decode_rejects_before_launch():
    w = api.window(64, 300)
    assert _decode(w, ptr=None) == WA_EARG
    assert _decode(w, rows=0) == WA_EARG
    assert _decode(w, streams=0) == WA_EARG
    assert _decode(w, d=64) == WA_EUNSUPPORTED
    assert _decode(w, hq=6, hkv=4) == WA_EUNSUPPORTED
    assert _decode(w, hq=34, hkv=2) == WA_EUNSUPPORTED        # group 17 > 16
    assert _decode(api.window(-1, 300)) == WA_EARG
    assert _decode(api.window(64, 0)) == WA_EARG
    assert _decode(api.window(400, 300)) == WA_ERANGE          # window longer than the ring
    assert _decode(api.window(0, 300), max_pos=300) == WA_ERANGE
    assert _decode(w, ws_bytes=16) == WA_EWORKSPACE
    assert _decode(w, strides=(1024, 250, 0, 512, 256)) == WA_EARG   # 16-byte rows
    assert _decode(w, ptr=FAKE + 2) == WA_EARG                       # misaligned
    assert _decode(w, ws=FAKE + 8) == WA_EWORKSPACE                  # workspace not 16-byte aligned


WA_ESCRATCH = -6


def test_noalloc_rejects_before_launch():
    """wa_decode_noalloc refuses a call whose partials exceed its static scratch, and bad
    shapes, before it touches a device."""
    L = api.lib()

    def call(rows, hq, hkv, d, w=api.window(1024, 1536)):
        return L.wa_decode_noalloc(ctypes.byref(w), FAKE, 4096, 256, FAKE, FAKE, 0, 2048, 256, 1,
                                   FAKE, FAKE, api.INT32_MAX, rows, hq, hkv, d, FAKE, 4096, 256,
                                   None)
    w = api.window(1024, 1536)
    need = L.wa_decode_workspace(200, 16, 256, ctypes.byref(w), api.INT32_MAX)
    assert need > 8 << 20
    assert call(200, 16, 8, 256) == WA_ESCRATCH
    assert call(0, 16, 8, 256) == WA_EARG
    assert call(4, 16, 8, 64) == WA_EUNSUPPORTED


def _prompt(w, p0=0, n=10, hq=4, hkv=2, d=256, ptr=FAKE, ws_bytes=1 << 30):
    L = api.lib()
    return L.wa_prompt(ctypes.byref(w), ptr, 1024, 256, ptr, ptr, 512, 256, p0, n, hq, hkv, d,
                       None, ptr, ws_bytes, ptr, 1024, 256, None)


def test_prompt_rejects_before_launch():
    w = api.window(1024, 1536)
    assert _prompt(w, ptr=None) == WA_EARG
    assert _prompt(w, n=0) == WA_EARG
    assert _prompt(w, p0=-1) == WA_EARG
    assert _prompt(w, d=192) == WA_EUNSUPPORTED
    # ring must hold [p0 - window + 1, p0 + n - 1]: 513 + 1023 = 1536 keys fit, 514 do not
    assert _prompt(w, p0=5000, n=514) == WA_ERANGE
    assert _prompt(api.window(0, 100), p0=50, n=51) == WA_ERANGE
    assert _prompt(w, ptr=FAKE + 8) == WA_EARG
    assert _prompt(w, ws_bytes=64) == WA_EWORKSPACE             # windowed: chunk partials
    # P's representation: one bf16, two or three parts; nothing else
    assert _prompt(api.window(1024, 1536, p32=3)) == WA_EUNSUPPORTED
    assert _prompt(api.window(1024, 1536, p32=-1)) == WA_EUNSUPPORTED


def _sparse(w, blocks=FAKE, srow=4, words=4, ws_bytes=1 << 30, p0=0, n=10):
    L = api.lib()
    return L.wa_prompt_sparse(ctypes.byref(w), FAKE, 1024, 256, FAKE, FAKE, 512, 256, p0, n, 4, 2,
                              256, None, blocks, srow, words, FAKE, ws_bytes, FAKE, 1024, 256, None)


def test_prompt_sparse_rejects_before_launch():
    w = api.window(0, 4096)
    assert _sparse(w, blocks=None) == WA_EARG
    assert _sparse(w, words=0) == WA_EARG
    assert _sparse(w, srow=3) == WA_EARG                       # a row's words overlap the next
    assert _sparse(w, blocks=FAKE + 2) == WA_EARG
    assert _sparse(api.window(0, 4096, p32=3)) == WA_EUNSUPPORTED
    assert _sparse(w, p0=4090) == WA_ERANGE                    # keys up to 4099 in a 4096 ring
    need = api.lib().wa_prompt_sparse_workspace(ctypes.byref(w), 0, 10, 4, 256)
    # without a window, chunks of keys 0 .. p0 + n - 1: (10 - 1) / 384 + 1 = 1 per (row, head)
    assert need == 10 * 4 * 1 * 4 * (2 + 256) + 16
    assert _sparse(w, ws_bytes=need - 1) == WA_EWORKSPACE
    w1 = api.window(1024, 1536)
    assert api.lib().wa_prompt_sparse_workspace(ctypes.byref(w1), 5000, 512, 16, 256) == \
        api.lib().wa_prompt_workspace(ctypes.byref(w1), 512, 16, 256)
    big = api.lib().wa_prompt_sparse_workspace(ctypes.byref(api.window(0, 8000)), 7836, 64, 24, 256)
    assert big == 64 * 24 * (7899 // 384 + 1) * 4 * (2 + 256) + 16


def test_prompt_workspace_sizes():
    L = api.lib()
    w = api.window(1024, 1536)
    # 512 rows x 16 heads x ((1023 + 512) / 384 + 2 = 5 chunks) x (m, l, 256 dims) + slack
    assert L.wa_prompt_workspace(ctypes.byref(w), 512, 16, 256) == 512 * 16 * 5 * 258 * 4 + 16
    assert L.wa_prompt_workspace(ctypes.byref(api.window(0, 4096)), 512, 16, 256) == 0
    assert L.wa_prompt_workspace(ctypes.byref(w), 512, 16, 64) == 0


def test_merge_rejects_before_launch():
    L = api.lib()
    w = api.window(64, 300)
    assert L.wa_merge(ctypes.byref(w), None, FAKE, FAKE, FAKE, 1, 1, 1, 256, FAKE, 1, 1, None) == WA_EARG
    assert L.wa_merge(ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 96, FAKE, 1, 1, None) == WA_EUNSUPPORTED
    assert L.wa_merge(ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, 1, 1, 0, 256, FAKE, 1, 1, None) == WA_EARG
    assert L.wa_merge(ctypes.byref(w), FAKE, FAKE, FAKE + 8, FAKE, 1, 1, 1, 256, FAKE, 1, 1, None) == WA_EARG


def _prepare(mode=1, R=256, theta=10000.0, eps=1e-6, x=FAKE, pos=FAKE, qs=None, rows=2, heads=2,
             d=256, st=None, streams=0, ring=0, out=FAKE, o_sstream=0, o_sslot=512, o_shead=256,
             x_srow=512, x_shead=256):
    p = api.Prep(mode, R, theta, eps)
    return api.lib().wa_prepare(ctypes.byref(p), x, x_srow, x_shead, pos, qs, rows, heads, d,
                                st, streams, ring, out, o_sstream, o_sslot, o_shead, None)


def test_prepare_rejects_before_launch():
    assert _prepare(x=None) == WA_EARG
    assert _prepare(pos=None) == WA_EARG
    assert _prepare(rows=0) == WA_EARG
    assert _prepare(d=64) == WA_EUNSUPPORTED
    assert _prepare(mode=7) == WA_EARG
    assert _prepare(R=257) == WA_EARG                      # odd rotated width
    assert _prepare(R=258) == WA_EARG                      # wider than the head
    assert _prepare(theta=0.0) == WA_EARG
    assert _prepare(theta=float("nan")) == WA_EARG
    assert _prepare(mode=2, qs=FAKE) == WA_EARG             # q scale belongs to the L2 recipe
    assert _prepare(ring=16) == WA_EARG                     # ring write without streams
    assert _prepare(x=FAKE + 4) == WA_EARG                  # 8-byte lane loads at d = 256
    assert _prepare(x_srow=514) == WA_EARG
    assert _prepare(ring=-1) == WA_EARG
