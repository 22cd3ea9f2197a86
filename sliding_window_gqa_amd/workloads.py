"""Seeded synthetic inputs for windowed GQA attention (input generation only, no attention math).

Both the oracle's tests and the HIP path's tests and bench draw their inputs from here; the
module computes nothing of the method itself. Shapes and value distributions follow the
Gemma-4-shaped receipt of TensorFold pull request #1123 ("Receipt", environment bullet):
q rows at RMS 0.95-1.05, k at 0.06-0.13, v at unit RMS, and every few rows one key set to a
query head's direction at k's RMS so that its score is near 30. The long non-windowed
prompt takes its shape and strided layout from the "Exact Numerical Contract" page
("Canonical Boundary": 37,810 tokens, 56 heads of 128, one interleaved QKV buffer of row
width 21,504 with Q/K/V at column offsets 0, 7,168 and 14,336) and its per-head RMS
normalisation (eps 1e-5) from that page's "Preparation" section.

Random generator: numpy PCG64 with a per-workload seed. bf16 values are produced by
rounding float32 draws with torch's float32 -> bfloat16 conversion (round to nearest even)
and are handed out as uint16 bit patterns.
"""

import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


def _directions(rng, shape, d, rho):
    """bf16 bits of vectors ``rho * z / rms(z)``, z ~ N(0, I_d); rho broadcasts over shape."""
    z = rng.standard_normal(tuple(shape) + (d,))
    z = z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True))
    return _bf16_bits(np.asarray(rho)[..., None] * z)


@dataclass
class DecodeCase:
    """Decode inputs: row r of stream stream[r] at position pos[r]."""
    name: str
    q: np.ndarray                 # uint16 [rows, Hq, d]
    k: np.ndarray                 # uint16 [streams, ring, Hkv, d]
    v: np.ndarray
    stream: np.ndarray            # int32 [rows]
    pos: np.ndarray               # int32 [rows]
    win: int
    ring: int
    scale: float = 1.0
    seed: int = 0
    peaks: list = field(default_factory=list)   # (row, q head, key position)

    @property
    def rows(self):
        return self.q.shape[0]

    @property
    def hq(self):
        return self.q.shape[1]

    @property
    def hkv(self):
        return self.k.shape[2]

    @property
    def d(self):
        return self.q.shape[2]


@dataclass
class PromptCase:
    """Prompt inputs: row i at position p0 + i of one stream, last key hi[i] (or its own)."""
    name: str
    q: np.ndarray                 # uint16 [n, Hq, d] (may be a strided view)
    k: np.ndarray                 # uint16 [ring, Hkv, d] (may be a strided view)
    v: np.ndarray
    p0: int
    win: int
    ring: int
    hi: Optional[np.ndarray] = None   # int32 [n] or None
    scale: float = 1.0
    p32: bool = False
    seed: int = 0
    buffer: Optional[np.ndarray] = None  # the interleaved buffer q/k/v view, if any
    peaks: list = field(default_factory=list)
    masks: Optional[np.ndarray] = None   # uint32 [n, words] block masks (sparse prompts)

    @property
    def n(self):
        return self.q.shape[0]

    @property
    def hq(self):
        return self.q.shape[1]

    @property
    def hkv(self):
        return self.k.shape[1]

    @property
    def d(self):
        return self.q.shape[2]


def _window(pos, win, last):
    lo = max(0, pos - win + 1) if win > 0 else 0
    return lo, last


def _plant_peaks(rng, q, k, rows, key_range_of_row, stream_of_row, ring, every=8):
    """Give row r (r % every == 0) one key per key head aligned with one of its query heads.

    k_j = bf16(rho_pk * q_h / rms(q_h)), rho_pk ~ U[0.100, 0.117], so q_h . k_j is about
    rho_pk * d * rms(q_h), i.e. 25-31 at d = 256. A slot is peaked at most once.
    """
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[2]
    G = hq // hkv
    used = set()
    peaks = []
    for r in rows:
        if r % every:
            continue
        lo, last = key_range_of_row(r)
        t = int(stream_of_row[r])
        for g in range(hkv):
            h = g * G + int(rng.integers(0, G))
            for _ in range(64):
                j = int(rng.integers(lo, last + 1))
                if (t, j % ring, g) not in used:
                    break
            else:
                continue
            used.add((t, j % ring, g))
            qh = _bits_to_f32(q[r, h]).astype(np.float64)
            rho = rng.uniform(0.100, 0.117)
            k[t, j % ring, g] = _bf16_bits(rho * qh / np.sqrt(np.mean(qh * qh)))
            peaks.append((int(r), int(h), j))
    return peaks


def decode_case(name, rows, hq, hkv, d, win, ring, streams, pos, seed, scale=1.0,
                peak_every=8, stream=None):
    """Generic decode inputs with the receipt's distributions. ``pos`` int array [rows]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = np.asarray(pos, dtype=np.int32)
    stream = (np.arange(rows) % streams if stream is None else np.asarray(stream)).astype(np.int32)
    q = _directions(rng, (rows, hq), d, rng.uniform(0.95, 1.05, size=(rows, hq)))
    k = _directions(rng, (streams, ring, hkv), d, rng.uniform(0.06, 0.13, size=(streams, ring, hkv)))
    v = _directions(rng, (streams, ring, hkv), d, np.ones((streams, ring, hkv)))
    peaks = []
    if peak_every:
        peaks = _plant_peaks(rng, q, k, range(rows), lambda r: _window(int(pos[r]), win, int(pos[r])),
                             stream, ring, peak_every)
    return DecodeCase(name, q, k, v, stream, pos, win, ring, float(np.float32(scale)), seed, peaks)


def prompt_case(name, n, hq, hkv, d, p0, win, ring, seed, hi=None, p32=False, scale=1.0,
                peak_every=8):
    """Generic prompt inputs (one stream). ``hi`` int array [n] or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _directions(rng, (n, hq), d, rng.uniform(0.95, 1.05, size=(n, hq)))
    k = _directions(rng, (ring, hkv), d, rng.uniform(0.06, 0.13, size=(ring, hkv)))
    v = _directions(rng, (ring, hkv), d, np.ones((ring, hkv)))
    hi = None if hi is None else np.asarray(hi, dtype=np.int32)
    peaks = []
    if peak_every:
        last = (lambda i: int(hi[i])) if hi is not None else (lambda i: p0 + i)
        k4, v4 = k[None], v[None]
        peaks = _plant_peaks(rng, q, k4, range(n), lambda i: _window(p0 + i, win, last(i)),
                             np.zeros(n, dtype=np.int32), ring, peak_every)
    return PromptCase(name, q, k, v, p0, win, ring, hi, float(np.float32(scale)), p32, seed,
                      None, peaks)


# ---- the five workloads -------------------------------------------------------------

def tiny_decode(seed=1001):
    """1 row, 2 query heads over 1 key head, d 256, window 64, linear cache of 300 keys,
    query at position 299, scale 1.0, one peaked key."""
    return decode_case("tiny decode 1x(2/1)x256 win64 linear300", 1, 2, 1, 256, 64, 300, 1,
                       [299], seed, peak_every=1)


def decode_12b(seed=1002, streams=3, rows=64):
    """64 rows over ``streams`` streams (row r -> stream r mod streams), 16/8 heads, d 256,
    window 1024 over a ring of 1536, positions uniform in 0..39,999, peaked key every 8th row."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    pos = rng.integers(0, 40000, size=rows)
    name = f"12B sliding decode {rows} rows (16/8)x256 win1024 ring1536 {streams} streams"
    return decode_case(name, rows, 16, 8, 256, 1024, 1536, streams, pos, seed)


def prompt_12b(seed=1003):
    """512 rows at p0 5,000, 16/8 heads, d 256, window 1024, ring 1536 (wraps), p32 on,
    hi[i] = p0 + i except the image span rows 40..300 which end at p0 + 300."""
    n, p0 = 512, 5000
    hi = p0 + np.arange(n)
    hi[40:301] = p0 + 300
    return prompt_case("12B sliding prompt 512 rows p0=5000 (16/8)x256 win1024 p32 image-hi",
                       n, 16, 8, 256, p0, 1024, 1536, seed, hi=hi, p32=True)


def prompt_31b(seed=1004):
    """333 rows at p0 1,300, 32/16 heads, d 256, window 1024, ring 1536, bf16 P, causal."""
    return prompt_case("31B sliding prompt 333 rows p0=1300 (32/16)x256 win1024 bf16P",
                       333, 32, 16, 256, 1300, 1024, 1536, seed)


def long_prompt(seed=1005, n=37810, heads=56, d=128, p32=False, block=1024):
    """Non-windowed, non-causal prompt over a linear cache: n tokens, ``heads`` heads of d,
    scale fl32(1/sqrt(d)). Q/K/V are N(0,1) draws normalised to unit RMS per (token, head)
    with eps 1e-5, in one interleaved [n, 3*heads*d] buffer (Q, K, V column blocks).
    Every row's last key is n - 1. Token block b (``block`` tokens) draws from its own
    PCG64 stream, spawned from ``seed``, so blocks can be generated in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    width = 3 * heads * d
    buf = np.empty((n, width), dtype=np.uint16)
    starts = list(range(0, n, block))
    seqs = np.random.SeedSequence(seed).spawn(len(starts))

    def fill(i):
        a = starts[i]
        b = min(n, a + block)
        rng = np.random.Generator(np.random.PCG64(seqs[i]))
        z = rng.standard_normal((b - a, 3 * heads, d), dtype=np.float32)
        z /= np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + np.float32(1e-5))
        buf[a:b] = _bf16_bits(z).reshape(b - a, width)

    workers = min(16, max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(len(starts))))
    hd = heads * d
    q = buf[:, 0:hd].reshape(n, heads, d)
    k = buf[:, hd:2 * hd].reshape(n, heads, d)
    v = buf[:, 2 * hd:3 * hd].reshape(n, heads, d)
    hi = np.full(n, n - 1, dtype=np.int32)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    return PromptCase(f"long non-windowed prompt {n}x{heads}x{d} non-causal", q, k, v, 0, 0, n,
                      hi, scale, p32, seed, buf, [])


SPARSE_BLOCK = 64      # keys per selectable block of a sparse prompt


def block_masks(rng, n, p0, nsel, words=None, block=SPARSE_BLOCK):
    """uint32 [n, words] masks: row i (position p0 + i) selects its own block and up to
    nsel - 1 other blocks drawn without replacement from the blocks before it (bit b % 32 of
    word b // 32 for block b)."""
    own = (p0 + np.arange(n)) // block
    words = int(own.max()) // 32 + 1 if words is None else words
    m = np.zeros((n, words), dtype=np.uint32)
    for i in range(n):
        b = int(own[i])
        others = rng.choice(b, size=min(nsel - 1, b), replace=False) if b > 0 else np.zeros(0, int)
        for x in [b, *others.tolist()]:
            m[i, x // 32] |= np.uint32(1) << np.uint32(x % 32)
    return m


def sparse_prompt_case(name, n, hq, hkv, d, p0, nsel, seed, win=0, p32=2, peak_every=8):
    """Block-sparse prompt over a linear cache holding keys 0 .. p0 + n - 1: each row selects
    ``nsel`` 64-key blocks (its own and nsel - 1 earlier ones), causal ends, the receipt's
    distributions; peaked keys are planted in selected blocks."""
    ring = p0 + n
    case = prompt_case(name, n, hq, hkv, d, p0, win, ring, seed, p32=p32, peak_every=0)
    rng = np.random.Generator(np.random.PCG64(seed + 15485863))
    case.masks = block_masks(rng, n, p0, nsel)
    if peak_every:
        def sel_range(i):
            own = (p0 + i) // SPARSE_BLOCK
            return own * SPARSE_BLOCK, p0 + i       # the own block's visible keys
        case.peaks = _plant_peaks(rng, case.q, case.k[None], range(n), sel_range,
                                  np.zeros(n, dtype=np.int32), ring, peak_every)
    return case


def sparse_prompt(seed=1007):
    """The sparse prompt slice of TensorFold pull request #1622's receipts: 64 rows of a
    7,900-token prompt (p0 7,836), 24 query heads over 2 key heads, d 256, 32 selected
    64-key blocks a row (2,048 keys; the own block is cut at the row's position), causal,
    P as three bf16 parts (the page's fp32 tile)."""
    return sparse_prompt_case("sparse prompt 64 rows p0=7836 (24/2)x256 32 blocks of 64",
                              64, 24, 2, 256, 7836, 32, seed)


def long_prompt_sample_rows(n, per_head=256, seed=1005):
    """Seeded sample of ``per_head`` row indices, always holding rows 0 and n - 1."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    inner = rng.choice(np.arange(1, n - 1), size=min(per_head, n) - 2, replace=False)
    return np.sort(np.concatenate([[0], inner, [n - 1]])).astype(np.int64)


@dataclass
class PrepCase:
    """Projection rows for the q/k preparation: x [rows, heads, d] bf16 bits at positions
    pos [rows]; qs float32 [d] or None (the L2 recipe's q scale)."""
    name: str
    x: np.ndarray
    pos: np.ndarray
    rope_dims: int
    theta: float = 10000.0
    qs: Optional[np.ndarray] = None


def prep_case(name, rows, heads, d, rope_dims, seed, pos=None, with_qs=False, theta=10000.0):
    """Projection rows with a per-(row, head) scale drawn log-uniform in [0.25, 4] (heads of
    very different sizes), Gaussian directions, and positions a third of which lie past
    199,800 (TensorFold pull request #1257, "Kernel contract": a third of the rows past
    position 199,800); the q scale, when asked, is a positive fp32 vector in [0.5, 3]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if pos is None:
        pos = np.concatenate([rng.integers(0, 8192, rows - rows // 3),
                              rng.integers(199_801, 262_144, rows // 3)])
        rng.shuffle(pos)
    scale = np.exp(rng.uniform(np.log(0.25), np.log(4.0), size=(rows, heads)))
    x = _bf16_bits(scale[..., None] * rng.standard_normal((rows, heads, d)))
    qs = rng.uniform(0.5, 3.0, d).astype(np.float32) if with_qs else None
    return PrepCase(name, x, np.asarray(pos, np.int32), rope_dims, theta, qs)
