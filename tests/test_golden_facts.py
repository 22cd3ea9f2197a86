"""Workload shapes and byte accounting pinned to numbers the pages print (tests/golden)."""

import json
import os

import numpy as np

from oracle import attend
from sliding_window_gqa_amd import workloads

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def fact(k):
    return FACTS[k]["value"]


def test_decode_row_bytes_match_the_page():
    c = workloads.decode_12b(rows=4)
    lo, last = attend.key_window(20000, c.win)
    keys = last - lo + 1
    assert keys == fact("gemma4_window_ring")[0]
    assert keys * c.hkv * c.d * 2 * 2 == fact("kv_bytes_per_12b_decode_row")


def test_gemma_shapes():
    c2 = workloads.decode_12b(rows=4)
    assert [c2.hq, c2.hkv] == fact("gemma4_12b_heads")
    assert [c2.win, c2.ring] == fact("gemma4_window_ring")
    c4 = workloads.prompt_31b()
    assert [c4.hq, c4.hkv] == fact("gemma4_31b_heads")
    c3 = workloads.prompt_12b()
    assert [c3.hq, c3.hkv] == fact("gemma4_12b_heads") and c3.p32


def test_long_prompt_layout_matches_the_contract_page():
    n = 300                                          # same layout, fewer tokens
    c = workloads.long_prompt(n=n)
    shape = fact("long_prompt_shape")
    assert c.q.shape == (n, shape[2], shape[3])
    width = fact("long_prompt_qkv_row_width")
    assert c.buffer.shape == (n, width)
    item = c.buffer.itemsize
    base = c.buffer.__array_interface__["data"][0]
    offs = [(a.__array_interface__["data"][0] - base) // item for a in (c.q, c.k, c.v)]
    assert offs == fact("long_prompt_qkv_offsets")
    st = fact("long_prompt_strides")
    assert [s // item for s in c.q.strides] == st[1:]
    assert st[0] == 37810 * width
    # per-head RMS is 1 up to bf16 rounding and the eps
    z = (c.k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt((z * z).mean(-1))
    assert np.all(np.abs(rms - 1) < 0.01)
    tail = fact("long_prompt_tail_rows")
    assert 37810 % tail["q_tile"] == tail["valid"] and 37810 % tail["k_tile"] == tail["valid"]
