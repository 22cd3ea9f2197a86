"""Thin ctypes binding of ``libwa.so`` (C ABI in include/wa.h).

Argument marshalling only: tensors supply device pointers and strides, torch's current
stream supplies the HIP stream, and every step of the computation runs in the library's
HIP kernels. There is no fallback: if ``libwa.so`` is missing or a GPU is absent, the
calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwa.so")
INT32_MAX = 2**31 - 1

_lib = None


class Window(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("ring", ctypes.c_int32),
                ("scale", ctypes.c_float), ("p32", ctypes.c_int32)]


# Window.p32 values: P enters P.V as one bf16, two bf16 parts, or three parts summing to P
P_BF16, P_TWO, P_THREE = 0, 1, 2


def _p_mode(p32):
    # a bool maps onto the page's flag: False -> one bf16, True -> two parts
    return P_BF16 if p32 is None else int(p32)


def window(window, ring, scale=1.0, p32=False):
    """p32: False/0 (one bf16 P), True/1 (two parts) or 2 (three parts, P exactly)."""
    return Window(int(window), int(ring), float(scale), _p_mode(p32))


class Prep(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
                ("theta", ctypes.c_float), ("eps", ctypes.c_float)]


PREP_COPY, PREP_ROPE_L2, PREP_RMS_ROPE = 0, 1, 2
# the pages' epsilons: on the sum of squares (L2), on their mean (RMSNorm)
PREP_EPS = {PREP_ROPE_L2: 1e-6, PREP_RMS_ROPE: 1e-5, PREP_COPY: 0.0}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_WP = ctypes.POINTER(Window)

SIGNATURES = {
    "wa_decode_chunks": (_I32, [_WP, _I32]),
    "wa_decode_workspace": (_SZ, [_I32, _I32, _I32, _WP, _I32]),
    "wa_decode": (ctypes.c_int, [_WP, _P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I32,
                                 _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _SZ,
                                 _P, _I64, _I64, _P]),
    "wa_decode_noalloc": (ctypes.c_int, [_WP, _P, _I64, _I64, _P, _P, _I64, _I64, _I64, _I32,
                                         _P, _P, _I32, _I32, _I32, _I32, _I32,
                                         _P, _I64, _I64, _P]),
    "wa_merge": (ctypes.c_int, [_WP, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                _P, _I64, _I64, _P]),
    "wa_prompt_workspace": (_SZ, [_WP, _I32, _I32, _I32]),
    "wa_prompt": (ctypes.c_int, [_WP, _P, _I64, _I64, _P, _P, _I64, _I64,
                                 _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P, _I64, _I64, _P]),
    "wa_prompt_sparse_workspace": (_SZ, [_WP, _I32, _I32, _I32, _I32]),
    "wa_prompt_sparse": (ctypes.c_int, [_WP, _P, _I64, _I64, _P, _P, _I64, _I64,
                                        _I32, _I32, _I32, _I32, _I32, _P, _P, _I64, _I32,
                                        _P, _SZ, _P, _I64, _I64, _P]),
    "wa_prepare": (ctypes.c_int, [ctypes.POINTER(Prep), _P, _I64, _I64, _P, _P, _I32, _I32, _I32,
                                  _P, _I32, _I32, _P, _I64, _I64, _I64, _P]),
    "wa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "wa_version": (ctypes.c_char_p, []),
}


def load_library(path):
    """Load a build of the library at ``path`` with the C signatures set (the product library,
    or another build of the same sources)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m sliding_window_gqa_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """Load libwa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


class using:
    """Context in which the binding's calls go to another build of the library (``L`` from
    load_library), e.g. a build with a planted mistake that a test must see fail."""

    def __init__(self, L):
        self.L = L

    def __enter__(self):
        global _lib
        self.prev, _lib = _lib, self.L
        return self.L

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev


def _check(status):
    if status != 0:
        raise RuntimeError(f"wa: {lib().wa_status_string(status).decode()} (status {status})")


def _bf16(t, name):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 CUDA tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the innermost (dim) stride must be 1")
    return t


def _i32(t, name):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 CUDA tensor")
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def decode_workspace_bytes(rows, hq, d, win, ring, max_pos):
    w = window(win, ring)
    return lib().wa_decode_workspace(rows, hq, d, ctypes.byref(w), max_pos)


def decode(q, k, v, stream_of_row, pos_of_row, win, ring, scale=1.0, max_pos=None,
           out=None, workspace=None):
    """Decode rows. q [rows, Hq, d]; k, v [streams, ring, Hkv, d] (bf16, CUDA);
    stream_of_row, pos_of_row int32 [rows] (CUDA). Returns out [rows, Hq, d] bf16."""
    _bf16(q, "q"); _bf16(k, "k"); _bf16(v, "v")
    _i32(stream_of_row, "stream_of_row"); _i32(pos_of_row, "pos_of_row")
    if k.shape != v.shape or k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must share one [streams, ring, Hkv, d] layout")
    rows, hq, d = q.shape
    streams, ring_k, hkv, dk = k.shape
    if dk != d or ring_k != ring:
        raise ValueError("k/v shape does not match q or the ring length")
    if max_pos is None:
        max_pos = INT32_MAX if win > 0 else ring - 1
    w = window(win, ring, scale)
    need = lib().wa_decode_workspace(rows, hq, d, ctypes.byref(w), max_pos)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=q.device)
    _check(lib().wa_decode(ctypes.byref(w), q.data_ptr(), q.stride(0), q.stride(1),
                           k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
                           streams, stream_of_row.data_ptr(), pos_of_row.data_ptr(), max_pos,
                           rows, hq, hkv, d, workspace.data_ptr(), workspace.numel(),
                           out.data_ptr(), out.stride(0), out.stride(1), _stream()))
    return out



def decode_noalloc(q, k, v, stream_of_row, pos_of_row, win, ring, scale=1.0, max_pos=None,
                   out=None):
    """decode() through wa_decode_noalloc: the library's static scratch instead of a
    workspace (pass ``out`` to allocate nothing at all). Same arguments and result."""
    _bf16(q, "q"); _bf16(k, "k"); _bf16(v, "v")
    _i32(stream_of_row, "stream_of_row"); _i32(pos_of_row, "pos_of_row")
    if k.shape != v.shape or k.stride() != v.stride() or k.dim() != 4:
        raise ValueError("k and v must share one [streams, ring, Hkv, d] layout")
    rows, hq, d = q.shape
    streams, ring_k, hkv, dk = k.shape
    if dk != d or ring_k != ring:
        raise ValueError("k/v shape does not match q or the ring length")
    if max_pos is None:
        max_pos = INT32_MAX if win > 0 else ring - 1
    w = window(win, ring, scale)
    if out is None:
        out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=q.device)
    _check(lib().wa_decode_noalloc(ctypes.byref(w), q.data_ptr(), q.stride(0), q.stride(1),
                                   k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1),
                                   k.stride(2), streams, stream_of_row.data_ptr(),
                                   pos_of_row.data_ptr(), max_pos, rows, hq, hkv, d,
                                   out.data_ptr(), out.stride(0), out.stride(1), _stream()))
    return out

def merge(m, l, o, pos_of_row, win, ring, out=None):
    """Merge decode partials m, l [rows, Hq, C] and o [rows, Hq, C, d] (fp32, CUDA)."""
    for t, nm in ((m, "m"), (l, "l"), (o, "o")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous float32 CUDA tensor")
    _i32(pos_of_row, "pos_of_row")
    rows, hq, C, d = o.shape
    if out is None:
        out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=o.device)
    w = window(win, ring)
    _check(lib().wa_merge(ctypes.byref(w), m.data_ptr(), l.data_ptr(), o.data_ptr(),
                          pos_of_row.data_ptr(), rows, hq, C, d, out.data_ptr(),
                          out.stride(0), out.stride(1), _stream()))
    return out


def prompt_workspace_bytes(n, hq, d, win, ring):
    w = window(win, ring)
    return lib().wa_prompt_workspace(ctypes.byref(w), n, hq, d)


def prompt(q, k, v, p0, win, ring, scale=1.0, hi=None, p32=False, out=None, workspace=None):
    """Prompt rows p0 .. p0+n-1. q [n, Hq, d]; k, v [ring, Hkv, d] (bf16, CUDA, any
    strides with a unit dim stride); hi int32 [n] (CUDA) or None."""
    _bf16(q, "q"); _bf16(k, "k"); _bf16(v, "v")
    if k.shape != v.shape or k.stride() != v.stride() or k.dim() != 3:
        raise ValueError("k and v must share one [ring, Hkv, d] layout")
    n, hq, d = q.shape
    ring_k, hkv, dk = k.shape
    if dk != d or ring_k < ring:
        raise ValueError("k/v shape does not match q or the ring length")
    hp = None
    if hi is not None:
        _i32(hi, "hi")
        hp = hi.data_ptr()
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.bfloat16, device=q.device)
    w = window(win, ring, scale, p32)
    need = lib().wa_prompt_workspace(ctypes.byref(w), n, hq, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp = workspace.data_ptr() if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    _check(lib().wa_prompt(ctypes.byref(w), q.data_ptr(), q.stride(0), q.stride(1),
                           k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1),
                           int(p0), n, hq, hkv, d, hp, wp, wn, out.data_ptr(), out.stride(0),
                           out.stride(1), _stream()))
    return out


def prompt_sparse(q, k, v, p0, win, ring, masks, scale=1.0, hi=None, p32=False, out=None,
                  workspace=None):
    """Block-sparse prompt rows p0 .. p0+n-1 (wa_prompt_sparse): as ``prompt``, and row i sees
    only the keys whose 64-key block is selected in masks[i] (int32/uint32 words as an int32
    CUDA tensor [n, words], unit word stride)."""
    _bf16(q, "q"); _bf16(k, "k"); _bf16(v, "v")
    if k.shape != v.shape or k.stride() != v.stride() or k.dim() != 3:
        raise ValueError("k and v must share one [ring, Hkv, d] layout")
    if masks.dtype != torch.int32 or not masks.is_cuda or masks.dim() != 2 or masks.stride(1) != 1:
        raise TypeError("masks must be an int32 CUDA tensor [n, words] with unit word stride")
    n, hq, d = q.shape
    ring_k, hkv, dk = k.shape
    if dk != d or ring_k < ring or masks.shape[0] != n:
        raise ValueError("k/v/masks shape does not match q or the ring length")
    hp = None
    if hi is not None:
        _i32(hi, "hi")
        hp = hi.data_ptr()
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.bfloat16, device=q.device)
    w = window(win, ring, scale, p32)
    need = lib().wa_prompt_sparse_workspace(ctypes.byref(w), int(p0), n, hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().wa_prompt_sparse(ctypes.byref(w), q.data_ptr(), q.stride(0), q.stride(1),
                                  k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1),
                                  int(p0), n, hq, hkv, d, hp, masks.data_ptr(), masks.stride(0),
                                  masks.shape[1], workspace.data_ptr(), workspace.numel(),
                                  out.data_ptr(), out.stride(0), out.stride(1), _stream()))
    return out


def prepare(x, pos_of_row, mode, rope_dims=0, theta=10000.0, qs=None, eps=None, out=None,
            stream_of_row=None, ring=0):
    """q/k row preparation (wa_prepare). x [rows, heads, d] bf16 (CUDA, unit dim stride);
    pos_of_row int32 [rows]; qs float32 [d] or None. With ring == 0 the result is a new (or
    the given) [rows, heads, d] tensor; with ring > 0, ``out`` is the cache
    [streams, ring, heads, d] and row r goes to slot pos mod ring of stream_of_row[r]."""
    _bf16(x, "x"); _i32(pos_of_row, "pos_of_row")
    rows, heads, d = x.shape
    p = Prep(int(mode), int(rope_dims), float(theta), float(PREP_EPS[mode] if eps is None else eps))
    qp = None
    if qs is not None:
        if qs.dtype != torch.float32 or not qs.is_cuda or not qs.is_contiguous() or qs.numel() != d:
            raise TypeError("qs must be a contiguous float32 CUDA tensor of d values")
        qp = qs.data_ptr()
    if ring > 0:
        if out is None or stream_of_row is None:
            raise ValueError("a ring write needs the cache tensor and stream_of_row")
        _bf16(out, "out"); _i32(stream_of_row, "stream_of_row")
        if out.dim() != 4 or out.shape[1] != ring or out.shape[2] != heads or out.shape[3] != d:
            raise ValueError("out must be [streams, ring, heads, d]")
        streams, sst, ssl, sh = out.shape[0], out.stride(0), out.stride(1), out.stride(2)
        sp = stream_of_row.data_ptr()
    else:
        if out is None:
            out = torch.empty((rows, heads, d), dtype=torch.bfloat16, device=x.device)
        _bf16(out, "out")
        streams, sst, ssl, sh, sp = 0, 0, out.stride(0), out.stride(1), None
    _check(lib().wa_prepare(ctypes.byref(p), x.data_ptr(), x.stride(0), x.stride(1),
                            pos_of_row.data_ptr(), qp, rows, heads, d, sp, streams, int(ring),
                            out.data_ptr(), sst, ssl, sh, _stream()))
    return out
