"""Windowed grouped-query softmax attention in float64 (test infrastructure; see the package header).

Source: TensorFold pull request #1123, "window_attention at head dim 256", section
"What this changes":
  * Decode bullet: chunked decode with an ordered merge is an exact rewrite, in real
    arithmetic, of softmax attention over the row's visible keys; so is the prompt's tiled
    online softmax (Prompt bullet). The oracle is therefore the plain definition.
  * promptRows(..., hi) bullet: prompt row i (position p0 + i) sees keys from
    p0 + i - win + 1 up to hi[i]; without hi the last key is the row's own position.
  * Scale/Window 0 bullet: the score is scale * (q . k); window 0 means no window, the
    cache is linear (a ring as long as the cache).
  * first paragraph: any number of query heads per key head.

Readings taken where the page is silent (each also listed in the design doc):
  * key j lives in ring slot j mod ring of the row's stream;
  * query head h reads key head h // G, with G = Hq / Hkv (contiguous groups);
  * the window's low end is clamped at key 0 and anchored on the row's own position, also
    when hi[i] is larger; decode's last key is the row's own position;
  * scale is the float32 value the caller passes, widened exactly;
  * keys outside the window are excluded from every sum (never multiplied by zero);
  * sums start at +0.0, so a column of signed zeros gives +0.

Block-sparse prompts (TensorFold pull request #1622, "What this changes": per-row block
masks over the union of a row group's selected blocks, causal ends, the parts/merge layout)
narrow a prompt row's keys further: with a mask, row i sees only the keys of [lo_i, last_i]
whose block is selected. Readings: a block is 64 consecutive keys at absolute positions
(block b = keys 64b .. 64b + 63; the page does not give the size); the mask of a row is
32-bit words, bit b % 32 of word b // 32 for block b, and blocks past the last word are not
selected; a row that sees no key at all has no softmax and its output is NaN (0 / 0).

Everything here is float64 with one rounding, to bf16 at the output (``bf16.to_bf16_bits``).
Alongside the value x the oracle records S = sum_j p_j |v_j| / l, the conditioning scale the
acceptance interval uses (S >= |x|).
"""

import numpy as np

from . import bf16


def key_window(pos, win, last=None):
    """First and last visible key of a row at position ``pos`` (window ``win``, 0 = none)."""
    lo = max(0, int(pos) - int(win) + 1) if win > 0 else 0
    return lo, int(pos) if last is None else int(last)


SPARSE_BLOCK = 64


def visible_keys(pos, win, last=None, mask=None, block=SPARSE_BLOCK):
    """Sorted absolute positions of the keys a row sees: [lo, last] of ``key_window``, and,
    with a block mask (uint32 words), only those whose block's bit is set."""
    lo, hi = key_window(pos, win, last)
    keys = np.arange(lo, hi + 1, dtype=np.int64)
    if mask is None:
        return keys
    mask = np.asarray(mask, dtype=np.uint32)
    b = keys // block
    word = b // 32
    inside = word < mask.size
    bits = (mask[np.minimum(word, max(mask.size - 1, 0))] >> (b % 32).astype(np.uint32)) & 1
    return keys[inside & (bits == 1)]


def chunk_range(pos, win, last=None, chunk=256):
    """Decode chunks (``chunk`` keys at absolute positions) holding at least one visible key."""
    lo, hi = key_window(pos, win, last)
    return lo // chunk, hi // chunk


def _head_group(qg, K, V, c):
    """Softmax attention of the query heads ``qg`` [G, d] over keys K, V [n, d] (all float64).

    Returns x [G, d] and S [G, d].
    """
    finite = np.isfinite(qg).all() and np.isfinite(K).all() and np.isfinite(V).all()
    if finite:
        dots = qg @ K.T
    else:
        # elementwise form: a BLAS kernel may skip zero multiplicands, which would hide
        # the NaN that 0 * inf makes under IEEE arithmetic
        dots = (qg[:, None, :] * K[None, :, :]).sum(axis=-1)
    s = c * dots                                   # [G, n]
    m = s.max(axis=1, keepdims=True)               # NaN propagates
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    if finite:
        num = 0.0 + p @ V
        num_abs = 0.0 + p @ np.abs(V)
    else:
        num = 0.0 + (p[:, :, None] * V[None, :, :]).sum(axis=1)
        num_abs = 0.0 + (p[:, :, None] * np.abs(V)[None, :, :]).sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return num / l, num_abs / l


def attention(q, k_cache, v_cache, stream_of_row, pos_of_row, win, ring, scale,
              last_of_row=None, rows=None, masks=None):
    """Float64 windowed GQA attention for the rows ``rows`` (default: all).

    q        uint16 bf16 bits [R, Hq, d]
    k_cache  uint16 bf16 bits [S, ring, Hkv, d] (stream, slot, key head, dim); v_cache alike
    stream_of_row, pos_of_row   int [R]
    last_of_row  int [R] or None (None: each row's last key is its own position)
    win      window (0 = none); ring: slots per stream; scale: float32 score scale
    masks    uint32 [R, W] block masks (``visible_keys``) or None (every key of the range)

    Returns (x, S, out): x and S float64 [len(rows), Hq, d], out uint16 bf16 bits of x.
    """
    q = np.asarray(q)
    R, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    c = float(np.float32(scale))
    rows = np.arange(R) if rows is None else np.asarray(rows)
    x = np.empty((len(rows), Hq, d), dtype=np.float64)
    S = np.empty_like(x)
    # rows with the same stream and visible key set are evaluated together (same definition)
    groups = {}
    for n, i in enumerate(rows):
        last = None if last_of_row is None else last_of_row[i]
        keys = visible_keys(pos_of_row[i], win, last, None if masks is None else masks[i])
        groups.setdefault((int(stream_of_row[i]), keys.tobytes()), (keys, []))[1].append((n, int(i)))
    for (t, _), (keys, members) in groups.items():
        slots = keys % ring
        ns = [m[0] for m in members]
        idx = [m[1] for m in members]
        if keys.size == 0:                         # no key: 0 / 0
            x[ns] = np.nan
            S[ns] = 0.0
            continue
        for g in range(Hkv):
            K = bf16.to_f64(k_cache[t, slots, g, :])
            V = bf16.to_f64(v_cache[t, slots, g, :])
            qg = bf16.to_f64(q[idx, g * G:(g + 1) * G, :]).reshape(len(idx) * G, d)
            xg, Sg = _head_group(qg, K, V, c)
            x[ns, g * G:(g + 1) * G, :] = xg.reshape(len(idx), G, d)
            S[ns, g * G:(g + 1) * G, :] = Sg.reshape(len(idx), G, d)
    return x, S, bf16.to_bf16_bits(x)


def decode(q, k_cache, v_cache, stream_of_row, pos_of_row, win, ring, scale, rows=None):
    """Decode form: row r at position pos_of_row[r] of stream stream_of_row[r]."""
    return attention(q, k_cache, v_cache, stream_of_row, pos_of_row, win, ring, scale,
                     None, rows)


def prompt(q, k_ring, v_ring, p0, win, ring, scale, hi=None, rows=None):
    """Prompt form: row i at position p0 + i of one stream, last key hi[i] (or p0 + i).

    k_ring, v_ring: uint16 [ring, Hkv, d]. The p32 flag changes only how the kernel
    represents P, not the value it approximates, so the oracle takes no p32 argument.
    """
    n = q.shape[0]
    pos = p0 + np.arange(n, dtype=np.int64)
    return attention(q, k_ring[None], v_ring[None], np.zeros(n, dtype=np.int64), pos,
                     win, ring, scale, None if hi is None else np.asarray(hi), rows)


def sparse_prompt(q, k_ring, v_ring, p0, win, ring, scale, masks, hi=None, rows=None):
    """Block-sparse prompt: row i at position p0 + i sees the keys of its range [lo_i, last_i]
    whose 64-key block is selected in masks[i] (uint32 words, bit b % 32 of word b // 32)."""
    n = q.shape[0]
    pos = p0 + np.arange(n, dtype=np.int64)
    return attention(q, k_ring[None], v_ring[None], np.zeros(n, dtype=np.int64), pos,
                     win, ring, scale, None if hi is None else np.asarray(hi), rows,
                     np.asarray(masks, dtype=np.uint32))
