"""wa_decode_noalloc (the decode entry point that allocates nothing: its partials live in the
library's static scratch) against wa_decode, bit for bit, through the C ABI: two calls in a
row on one GPU, the second with a smaller input, so the second reads a scratch the first
left full; and a call too large for the scratch is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

from sliding_window_gqa_amd import api, workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

WA_ESCRATCH = -6
SCRATCH = 8 << 20


def _inputs(case):
    return (gu.dev_bf16(case.q), gu.dev_bf16(case.k), gu.dev_bf16(case.v),
            gu.dev_i32(case.stream), gu.dev_i32(case.pos))


def _both(case):
    q, k, v, st, pos = _inputs(case)
    ref = api.decode(q, k, v, st, pos, case.win, case.ring, case.scale)
    out = torch.full_like(ref, float("nan"))
    api.decode_noalloc(q, k, v, st, pos, case.win, case.ring, case.scale, out=out)
    torch.cuda.synchronize()
    return gu.host_bits(ref), gu.host_bits(out)


def test_noalloc_matches_decode_twice_second_smaller():
    big = workloads.decode_12b()                       # 64 rows x 16 heads x 5 chunks: 5.3 MB
    need = api.decode_workspace_bytes(big.rows, big.hq, big.d, big.win, big.ring, api.INT32_MAX)
    assert 0 < need <= SCRATCH
    gu.log(f"noalloc: 12B decode, {need} scratch bytes")
    ref, out = _both(big)
    assert np.array_equal(ref, out)
    small = workloads.decode_case("small after big", 5, 4, 2, 256, 300, 700, 2,
                                  [10, 699, 300, 255, 256], seed=31)
    gu.log("noalloc: 5-row decode after the 12B decode")
    ref, out = _both(small)
    assert np.array_equal(ref, out)
    tiny = workloads.tiny_decode()
    gu.log("noalloc: tiny decode")
    ref, out = _both(tiny)
    assert np.array_equal(ref, out)


def test_noalloc_refuses_more_than_its_scratch():
    L = api.lib()
    w = api.window(1024, 1536)
    rows = 102                                          # 102 x 16 x 5 x (256 + 2) fp32 > 8 MiB
    assert L.wa_decode_workspace(rows, 16, 256, ctypes.byref(w), api.INT32_MAX) > SCRATCH
    q = torch.zeros((rows, 16, 256), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1536, 8, 256), dtype=torch.bfloat16, device="cuda")
    ix = torch.zeros(rows, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    st = L.wa_decode_noalloc(ctypes.byref(w), q.data_ptr(), q.stride(0), q.stride(1),
                             kv.data_ptr(), kv.data_ptr(), kv.stride(0), kv.stride(1), kv.stride(2),
                             1, ix.data_ptr(), ix.data_ptr(), api.INT32_MAX, rows, 16, 8, 256,
                             out.data_ptr(), out.stride(0), out.stride(1),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == WA_ESCRATCH
    assert b"scratch" in L.wa_status_string(WA_ESCRATCH)
