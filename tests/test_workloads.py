"""The seeded generators produce the receipt's distributions and are reproducible."""

import numpy as np

from sliding_window_gqa_amd import workloads


def f(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms(x):
    return np.sqrt((x * x).mean(-1))


def test_distributions_and_peaks():
    c = workloads.decode_12b()
    assert c.rows == 64 and c.q.shape == (64, 16, 256) and c.k.shape == (3, 1536, 8, 256)
    assert np.all((rms(f(c.q)) > 0.94) & (rms(f(c.q)) < 1.06))
    kr = rms(f(c.k))
    assert np.all((kr > 0.059) & (kr < 0.131))
    assert np.all(np.abs(rms(f(c.v)) - 1) < 0.01)
    assert list(c.stream[:4]) == [0, 1, 2, 0] and c.pos.min() >= 0 and c.pos.max() < 40000
    assert len(c.peaks) == 8 * 8                     # rows 0, 8, ..., 56 x 8 key heads
    for r, h, j in c.peaks:
        s = f(c.q[r, h]) @ f(c.k[c.stream[r], j % c.ring, h // 2])
        assert 24 < s < 32
        assert c.pos[r] - c.win < j <= c.pos[r]


def test_reproducible():
    a = workloads.prompt_31b()
    b = workloads.prompt_31b()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert a.hi is None and not a.p32


def test_tiny_and_image_prompt():
    c = workloads.tiny_decode()
    assert c.pos.tolist() == [299] and c.ring == 300 and c.win == 64 and len(c.peaks) == 1
    p = workloads.prompt_12b()
    assert p.hi[39] == 5039 and p.hi[40] == 5300 and p.hi[300] == 5300 and p.hi[301] == 5301


def test_sample_rows():
    r = workloads.long_prompt_sample_rows(37810)
    assert len(r) == 256 and r[0] == 0 and r[-1] == 37809 and len(set(r.tolist())) == 256
