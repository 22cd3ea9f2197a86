"""Throughput of windowed GQA attention on one MI355X: decode KV GB/s and prefill TFLOP/s.

One step is one pass of the whole hot path of a Gemma-4-12B-shaped sliding layer:
  * decode: 64 rows over 3 streams, 16/8 heads x 256, window 1024 over a ring of 1536,
    positions up to 40,000 (split-KV chunk partials + ordered merge), and
  * prompt: a 512-row chunk at p0 5,000 with p32 and an image span (MFMA online softmax).
``value`` is the decode's rate in HBM terms: the distinct K/V ring bytes the call must read
(each (stream, slot, key head) once) plus q and out, over the call's time, with L2 and MALL
flushed (by reading 512 MiB) before every timed call. The 64 rows share three rings, so the
rows' own K/V reads (the pull request's per-row accounting, 8 MiB a full 12B row) are mostly
served from the caches; that figure is reported beside it under its own name.

Also timed in the same run, each with its own roofline object: the tiny decode (absolute
time), the 31B prompt chunk, the 64-stream decode (no shared keys: the clean HBM shape), the
long non-windowed prompt (37,810 x 56 x 128, the MFMA-bound shape; P as one bf16, and on the
same inputs as two halves (p32) and as three parts), the 12B chunk with P as three parts, the
block-sparse slice and the long prompt's q/k preparation.

The float64 oracle runs on the host cores first (a process pool forked before the GPU is
touched, one BLAS thread a process): its time per workload is ``cpu_baseline`` and its
values give the ``parity`` object (every output against its interval, and the literal
one-ulp counts), computed from the timed calls' own outputs.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--long-iters 3] [--no-cpu]
                    [--no-long] [--no-prep]

Prints one JSON line.
"""

import argparse
import ctypes
import json
import multiprocessing
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sliding_window_gqa_amd import api, workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# The decode's fp32 arithmetic on the vector ALUs: q.k as v_dot2_f32_bf16 (2 multiply-adds a
# lane, 4 flops) and p.v as v_fma_f32 (2 flops), one instruction a lane-slot; 2d flops of each
# per (key, query head): 4d flops in 1.5d lane-instructions. 16 lanes x 4 SIMDs x 256 CUs at
# 2.4 GHz issue 39.3 T lane-instructions/s -> 4/1.5 x 39.3 = 104.9 TFLOP/s for this mix
# (packed fp32, which the 157.3 TFLOP/s figure counts, is not used).
DECODE_VALU_PEAK_TFS = 16 * 4 * 256 * 2.4e9 * (4 / 1.5) / 1e12
CPU_SHARE = 16               # host cores this box gives one GPU


def key_span(pos, win, last=None):
    lo = max(0, pos - win + 1) if win > 0 else 0
    return lo, pos if last is None else last


def decode_units(case):
    """Bytes and flops of a decode call: per-row K/V bytes (every row's visible keys, the
    receipt's accounting), unique bytes (distinct ring slots per stream and key head, plus q
    and out) and the fp32 work (2d for q.k and 2d for p.v per visible (row, query head, key))."""
    per_row = 0
    slots = {}
    for r in range(case.rows):
        lo, last = key_span(int(case.pos[r]), case.win)
        per_row += (last - lo + 1) * case.hkv * case.d * 2 * 2
        s = slots.setdefault(int(case.stream[r]), np.zeros(case.ring, bool))
        s[np.arange(lo, last + 1) % case.ring] = True
    unique = sum(int(s.sum()) for s in slots.values()) * case.hkv * case.d * 2 * 2
    qo = 2 * case.rows * case.hq * case.d * 2
    flops = 0
    for r in range(case.rows):
        lo, last = key_span(int(case.pos[r]), case.win)
        flops += (last - lo + 1) * case.hq * case.d * 2 * 2
    return {"kv_bytes": per_row, "unique_bytes": unique + qo, "row_bytes": per_row + qo,
            "flops_fp32": flops}


def prompt_units(case):
    """MFMA flops the method performs: 2d for S and 2d per P.V product per visible
    (row, head, key); P.V runs once per bf16 part of P (one, two with p32, or three).
    Bytes: q and out once, and the K/V of every ring slot the rows reach."""
    pv = 1 + api._p_mode(case.p32)
    triples = 0
    for i in range(case.n):
        last = None if case.hi is None else int(case.hi[i])
        lo, hi = key_span(case.p0 + i, case.win, last)
        triples += (hi - lo + 1)
    triples *= case.hq
    flops = triples * (2 + 2 * pv) * case.d
    first = key_span(case.p0, case.win)[0]
    keys = min(case.ring, case.p0 + case.n - first)
    byts = (2 * case.q.shape[0] * case.hq * case.d + 2 * keys * case.hkv * case.d) * 2
    return {"triples": triples, "flops": flops, "bytes": byts}


def sparse_units(case):
    """MFMA flops of a block-sparse prompt: (2 + 2 * parts) * d per visible (row, head, key),
    visible = the selected blocks' keys inside the row's range."""
    pv = 1 + api._p_mode(case.p32)
    triples = 0
    for i in range(case.n):
        last = None if case.hi is None else int(case.hi[i])
        lo, hi = key_span(case.p0 + i, case.win, last)
        keys = np.arange(lo, hi + 1)
        blk = keys // workloads.SPARSE_BLOCK
        words = case.masks[i][np.minimum(blk // 32, case.masks.shape[1] - 1)]
        sel = (blk // 32 < case.masks.shape[1]) & (((words >> (blk % 32)) & 1) == 1)
        triples += int(sel.sum())
    triples *= case.hq
    return {"triples": triples, "flops": triples * (2 + 2 * pv) * case.d}


# ---- the float64 oracle on the host cores ---------------------------------------------------

_CASES = {}     # name -> case, set before the pool forks (the workers read them copy-on-write)


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _oracle_part(job):
    from oracle import attend
    name, rows = job
    c = _CASES[name]
    if isinstance(c, workloads.DecodeCase):
        x, S, _ = attend.decode(c.q, c.k, c.v, c.stream, c.pos, c.win, c.ring, c.scale, rows=rows)
    else:
        x, S, _ = attend.prompt(c.q, c.k, c.v, c.p0, c.win, c.ring, c.scale, hi=c.hi, rows=rows)
    return rows, x, S


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def run_oracle(cases, sample_rows):
    """The oracle over every row of each workload (the long prompt: its sample rows), split
    by rows over a pool of one process per core; returns per-workload x, S and seconds."""
    _CASES.clear()
    _CASES.update(cases)
    cores = min(CPU_SHARE, len(os.sched_getaffinity(0)))
    ctx = multiprocessing.get_context("fork")
    res = {}
    with ctx.Pool(cores, initializer=_worker_init) as pool:
        for name, c in cases.items():
            rows = sample_rows.get(name)
            if rows is None:
                rows = np.arange(c.rows if isinstance(c, workloads.DecodeCase) else c.n)
            parts = [p for p in np.array_split(rows, min(len(rows), 2 * cores)) if len(p)]
            t0 = time.perf_counter()
            outs = pool.map(_oracle_part, [(name, p) for p in parts])
            dt = time.perf_counter() - t0
            x = np.concatenate([o[1] for o in outs])
            S = np.concatenate([o[2] for o in outs])
            res[name] = {"x": x, "S": S, "rows": rows, "seconds": dt}
            print(f"oracle {name}: {len(rows)} rows in {dt:.2f} s", file=sys.stderr, flush=True)
    _CASES.clear()
    return res, cores


# ---- device-side callers --------------------------------------------------------------------

def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Timed:
    """HIP events on the current stream (the one every C-ABI call is queued on) around each
    call."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def ms(self):
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.pairs]


class Decoder:
    """Decode inputs resident on the device and the C-ABI call prepared once (so the timed
    region holds no Python marshalling)."""

    def __init__(self, case):
        self.c = case
        self.q = to_dev(case.q)
        self.k = to_dev(case.k)
        self.v = to_dev(case.v)
        self.st = torch.from_numpy(case.stream.astype(np.int32)).cuda()
        self.pos = torch.from_numpy(case.pos.astype(np.int32)).cuda()
        n = api.decode_workspace_bytes(case.rows, case.hq, case.d, case.win, case.ring, api.INT32_MAX)
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.out = torch.empty((case.rows, case.hq, case.d), dtype=torch.bfloat16, device="cuda")
        # one checked call through the binding, then the raw call with the same arguments
        api.decode(self.q, self.k, self.v, self.st, self.pos, case.win, case.ring, case.scale,
                   out=self.out, workspace=self.ws)
        self.w = api.window(case.win, case.ring, case.scale)
        k = self.k
        self.args = (ctypes.byref(self.w), self.q.data_ptr(), self.q.stride(0), self.q.stride(1),
                     k.data_ptr(), self.v.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
                     k.shape[0], self.st.data_ptr(), self.pos.data_ptr(), api.INT32_MAX,
                     case.rows, case.hq, case.hkv, case.d, self.ws.data_ptr(), self.ws.numel(),
                     self.out.data_ptr(), self.out.stride(0), self.out.stride(1),
                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self.fn = api.lib().wa_decode

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"wa_decode status {st}")

    def bits(self, rows=None):
        return host_bits(self.out)


class Prompter:
    def __init__(self, case):
        self.c = case
        if case.buffer is not None:
            buf = to_dev(case.buffer)
            n, heads, d = case.q.shape
            hd = heads * d
            self.q = buf[:, 0:hd].view(n, heads, d)
            self.k = buf[:, hd:2 * hd].view(n, heads, d)
            self.v = buf[:, 2 * hd:3 * hd].view(n, heads, d)
        else:
            self.q, self.k, self.v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
        self.hi = None if case.hi is None else torch.from_numpy(case.hi.astype(np.int32)).cuda()
        self.out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
        api.prompt(self.q, self.k, self.v, case.p0, case.win, case.ring, case.scale, hi=self.hi,
                   p32=case.p32, out=self.out)
        torch.cuda.synchronize()
        self.w = api.window(case.win, case.ring, case.scale, case.p32)
        need = api.prompt_workspace_bytes(case.n, case.hq, case.d, case.win, case.ring)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        q, k = self.q, self.k
        self.args = (ctypes.byref(self.w), q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(),
                     self.v.data_ptr(), k.stride(0), k.stride(1), case.p0, case.n, case.hq,
                     case.hkv, case.d, None if self.hi is None else self.hi.data_ptr(),
                     self.ws.data_ptr(), self.ws.numel(),
                     self.out.data_ptr(), self.out.stride(0), self.out.stride(1),
                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self.fn = api.lib().wa_prompt

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"wa_prompt status {st}")

    def bits(self, rows=None):
        o = self.out if rows is None else self.out[torch.as_tensor(rows, device="cuda")]
        return host_bits(o)


class SparsePrompter:
    def __init__(self, case):
        self.c = case
        self.q, self.k, self.v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
        self.m = torch.from_numpy(np.ascontiguousarray(case.masks).view(np.int32)).cuda()
        self.out = torch.empty(case.q.shape, dtype=torch.bfloat16, device="cuda")
        api.prompt_sparse(self.q, self.k, self.v, case.p0, case.win, case.ring, self.m, case.scale,
                          p32=case.p32, out=self.out)
        torch.cuda.synchronize()
        self.w = api.window(case.win, case.ring, case.scale, case.p32)
        need = api.lib().wa_prompt_sparse_workspace(ctypes.byref(self.w), case.p0, case.n, case.hq, case.d)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        q, k = self.q, self.k
        self.args = (ctypes.byref(self.w), q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(),
                     self.v.data_ptr(), k.stride(0), k.stride(1), case.p0, case.n, case.hq,
                     case.hkv, case.d, None, self.m.data_ptr(), self.m.stride(0), self.m.shape[1],
                     self.ws.data_ptr(), self.ws.numel(), self.out.data_ptr(), self.out.stride(0),
                     self.out.stride(1), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self.fn = api.lib().wa_prompt_sparse

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"wa_prompt_sparse status {st}")


class Preparer:
    """The long prompt's q and k preparation (contract recipe: per-head RMSNorm, RoPE on dims
    0-95 with bf16 coefficients): 37,810 rows x 112 heads (56 q + 56 k) x 128, read from the
    interleaved projection buffer (row stride 21,504), written as contiguous rows."""

    def __init__(self):
        n, heads, d = 37810, 56, 128
        g = torch.Generator(device="cuda").manual_seed(1006)
        self.buf = torch.randn((n, 3 * heads * d), generator=g, device="cuda").to(torch.bfloat16)
        self.x = self.buf[:, 0:2 * heads * d].view(n, 2 * heads, d)
        self.pos = torch.arange(n, dtype=torch.int32, device="cuda")
        self.out = torch.empty((n, 2 * heads, d), dtype=torch.bfloat16, device="cuda")
        self.p = api.Prep(api.PREP_RMS_ROPE, 96, 10000.0, api.PREP_EPS[api.PREP_RMS_ROPE])
        x = self.x
        self.args = (ctypes.byref(self.p), x.data_ptr(), x.stride(0), x.stride(1), self.pos.data_ptr(),
                     None, n, 2 * heads, d, None, 0, 0, self.out.data_ptr(), 0, self.out.stride(0),
                     self.out.stride(1), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        self.bytes = 2 * n * 2 * heads * d * 2          # bf16 read + written
        self.fn = api.lib().wa_prepare

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"wa_prepare status {st}")


def source_hash():
    import hashlib
    import glob
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sliding_window_gqa_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_bytes(workload, kernels):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) recorded in
    profiles/traffic.txt for these kernels, or None if the kernel sources changed since."""
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.txt")))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    tot, found = 0, False
    for name, v in t.get("workloads", {}).get(workload, {}).items():
        if any(k in name for k in kernels):
            tot += v.get("fetch", 0) + v.get("write", 0)
            found = True
    return tot if found else None


def roofline(bound, achieved, peak, unit, traffic=None, kernel=None):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": round(peak, 2), "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
    return r


def _three(case):
    case.p32 = api.P_THREE
    return case


def _with_p(case, p32):
    """The same inputs (arrays shared, not copied) with P carried as ``p32``."""
    import copy
    c = copy.copy(case)
    c.p32 = p32
    return c


def profile_driver(names, iters):
    """Run the workloads for profiler passes, after a plain copy of known size."""
    a = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)                     # 256 MiB read + 256 MiB written: counter calibration
    torch.cuda.synchronize()
    del a, b
    make = {"decode1": lambda: Decoder(workloads.tiny_decode()),
            "decode12b": lambda: Decoder(workloads.decode_12b()),
            "decode12b64": lambda: Decoder(workloads.decode_12b(streams=64)),
            "prompt12b": lambda: Prompter(workloads.prompt_12b()),
            "prompt31b": lambda: Prompter(workloads.prompt_31b()),
            "long": lambda: Prompter(workloads.long_prompt()),
            "long2": lambda: Prompter(workloads.long_prompt(p32=api.P_TWO)),
            "long3": lambda: Prompter(workloads.long_prompt(p32=api.P_THREE)),
            "prompt12b3": lambda: Prompter(_three(workloads.prompt_12b())),
            "sparse": lambda: SparsePrompter(workloads.sparse_prompt()),
            "prepare_long": lambda: Preparer()}
    for n in names:
        f = make[n]()
        torch.cuda.synchronize()
        for _ in range(iters):
            f()
        torch.cuda.synchronize()
        print("done", n, flush=True)
        del f


def parity_entry(out, ref, e_p):
    """Every output against its interval (tier G, the gate; tier S, strict) and the literal
    one-ulp counts; where P is fp32 to 2**-16 or better, whether every output outside the
    one-step set is a cancelling one (|x| / S below the derived bound)."""
    from oracle import check
    rep = check.report(out, ref["x"], ref["S"], e_p)
    rep["e_P"] = e_p
    if e_p <= check.E_P_P32:
        rep["literal_bound_x_over_S"] = check.literal_bound(e_p)
        rep["literal_ok"] = bool(rep["worst_x_over_S"] < rep["literal_bound_x_over_S"])
    return rep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--long-iters", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the host oracle (and parity)")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-prep", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiler driver: run a 256 MiB device copy (counter calibration), then "
                         "each listed workload (decode1, decode12b, decode12b64, prompt12b, "
                         "prompt12b3, prompt31b, sparse, long, long2, long3, prepare_long) --steps "
                         "times; no timing, no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards without exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.only:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        api.lib()
        profile_driver(args.only.split(","), args.steps)
        return

    # seeded inputs (host), then the oracle on the host cores before the GPU is touched
    cases = {"C1": workloads.tiny_decode(), "C2": workloads.decode_12b(),
             "C2-D": workloads.decode_12b(streams=64), "C3": workloads.prompt_12b(),
             "C4": workloads.prompt_31b()}
    if not args.no_long:
        cases["C5"] = workloads.long_prompt()
    sample = {}
    if "C5" in cases:
        sample["C5"] = workloads.long_prompt_sample_rows(cases["C5"].n)
    oracle, cores = (None, 0) if args.no_cpu else run_oracle(cases, sample)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    api.lib()
    dcase, pcase = cases["C2"], cases["C3"]
    dec, pro = Decoder(dcase), Prompter(pcase)
    du, pu = decode_units(dcase), prompt_units(pcase)
    # cache flush between timed calls: READ a 512 MiB buffer (> 256 MB MALL, > L2), which
    # evicts the working set without leaving dirty lines whose write-back would land in the
    # timed call
    flush_buf = torch.ones(64 * 2**20, dtype=torch.int64, device="cuda")
    flush_out = torch.empty(1, dtype=torch.int64, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

    def time_cold(fn, n):
        for _ in range(args.warmup):
            fn()
        t = Timed()
        for _ in range(n):
            flush()
            with t:
                fn()
        return float(np.mean(t.ms()))

    for _ in range(args.warmup):
        dec(); pro()
    torch.cuda.synchronize()
    td, tp = Timed(), Timed()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        flush()
        with td:
            dec()
        with tp:
            pro()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dms = float(np.mean(td.ms()))
    pms = float(np.mean(tp.ms()))
    gpu_bits = {"C2": dec.bits(), "C3": pro.bits()}
    tw = Timed()
    for _ in range(args.steps):
        with tw:
            dec()
    dms_warm = float(np.mean(tw.ms()))

    uniq_gbs = du["unique_bytes"] / (dms * 1e-3) / 1e9
    row_gbs = du["kv_bytes"] / (dms * 1e-3) / 1e9
    pre_tfs = pu["flops"] / (pms * 1e-3) / 1e12
    dec_tfs = du["flops_fp32"] / (dms * 1e-3) / 1e12
    res = {
        "metric": "decode KV GB/s + prefill TFLOP/s, hd256 GQA window attn, % of roofline",
        "value": round(uniq_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dms + pms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded; receipt distributions)",
        "config": {"workload": "Gemma-4-12B-shaped sliding layer step: decode 64 rows over 3 "
                               "streams (16/8 x 256, window 1024, ring 1536, pos < 40,000) + "
                               "prompt chunk 512 rows at p0 5,000 (p32, image rows 40..300)",
                   "decode_rows": 64, "prompt_rows": 512, "window": 1024, "ring": 1536},
        "value_accounting": "decode: distinct ring bytes (K and V of each stream, slot and key "
                            "head the rows reach, once) + q + out, per second of the call, "
                            "caches flushed before each call",
        "decode": {"ms": round(dms, 5), "ms_warm_cache": round(dms_warm, 5),
                   "unique_bytes_per_call": du["unique_bytes"], "unique_gbs": round(uniq_gbs, 2),
                   "per_row_kv_bytes_per_call": du["kv_bytes"],
                   "per_row_kv_gbs_cache_served": round(row_gbs, 2),
                   "per_row_kv_gbs_cache_served_warm": round(du["kv_bytes"] / (dms_warm * 1e-3) / 1e9, 2),
                   "fp32_tflops": round(dec_tfs, 2)},
        "prefill": {"ms": round(pms, 5), "tflops": round(pre_tfs, 2), "flops_per_call": pu["flops"],
                    "flop_accounting": "(2 + 2*2) * d per visible (row, head, key), p32"},
        "wall_s_timed_loop": round(wall, 3),
    }
    dec_traffic = traffic_bytes("decode12b", ["decode_kernel", "merge_kernel"])
    rl_decode = roofline("hbm", uniq_gbs, HBM_PEAK_GBS, "GB/s", dec_traffic,
                         "decode_kernel<256,2,chunks> + merge_kernel, one call (distinct ring bytes)")
    rl_decode_alu = roofline("alu", dec_tfs, DECODE_VALU_PEAK_TFS, "TFLOP/s", dec_traffic,
                             "decode_kernel<256,2,chunks> + merge_kernel (fp32 q.k dot2 + p.v fma)")
    rl_prompt = roofline("mfma", pre_tfs, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                         traffic_bytes("prompt12b", ["prompt_quarter_kernel"]),
                         "prompt_quarter_kernel<p32>, one call (12B prompt chunk: the whole call "
                         "is this one kernel)")
    res["roofline"] = rl_prompt if pms >= dms else rl_decode
    res["roofline_decode"] = rl_decode
    res["roofline_decode_alu"] = rl_decode_alu
    res["roofline_prefill"] = rl_prompt

    # tiny decode: latency only
    tcase = cases["C1"]
    tdec = Decoder(tcase)
    t1 = time_cold(tdec, args.steps)
    tw1 = Timed()
    for _ in range(args.steps):
        with tw1:
            tdec()
    res["decode_tiny"] = {"workload": tcase.name, "us": round(t1 * 1e3, 2),
                          "us_warm_cache": round(float(np.mean(tw1.ms())) * 1e3, 2),
                          "bound": "launch latency (64 keys x 2 heads)"}
    gpu_bits["C1"] = tdec.bits()
    del tdec

    # the same decode shape with 64 streams (one row each): no keys shared between rows, so
    # every per-row byte is an HBM byte -- the clean HBM-roofline shape
    hcase = cases["C2-D"]
    hdec, hu = Decoder(hcase), decode_units(hcase)
    hms = time_cold(hdec, args.steps)
    gpu_bits["C2-D"] = hdec.bits()
    del hdec
    hgbs = hu["row_bytes"] / (hms * 1e-3) / 1e9
    res["decode_64_streams"] = {"workload": "12B decode shape, 64 rows in 64 streams (no shared keys)",
                                "ms": round(hms, 5), "bytes_per_call": hu["row_bytes"],
                                "gbs": round(hgbs, 2)}
    res["roofline_decode_64_streams"] = roofline(
        "hbm", hgbs, HBM_PEAK_GBS, "GB/s", traffic_bytes("decode12b64", ["decode_kernel", "merge_kernel"]),
        "decode_kernel<256,2,whole rows> (64 streams, no shared keys)")

    # 31B prompt chunk, P as one bf16
    ccase = cases["C4"]
    cp, cu_ = Prompter(ccase), prompt_units(ccase)
    cms = time_cold(cp, args.steps)
    gpu_bits["C4"] = cp.bits()
    del cp
    ctf = cu_["flops"] / (cms * 1e-3) / 1e12
    res["prefill_31b"] = {"workload": ccase.name, "ms": round(cms, 5), "tflops": round(ctf, 2),
                          "flops_per_call": cu_["flops"], "bytes_per_call": cu_["bytes"],
                          "flop_accounting": "(2 + 2*1) * d per visible (row, head, key), bf16 P"}
    res["roofline_prefill_31b"] = roofline(
        "mfma", ctf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
        traffic_bytes("prompt31b", ["prompt_quarter_kernel"]),
        "prompt_quarter_kernel<bf16P>, one call (31B prompt chunk: the whole call is this one "
        "kernel)")

    def time_long(case):
        """Mean warm time of the long prompt (a call is ~40-65 ms: caches hold no part of its
        2 GB working set between calls) and its sampled rows' bits."""
        lp = Prompter(case)
        lp(); torch.cuda.synchronize()
        tl = Timed()
        for _ in range(args.long_iters):
            with tl:
                lp()
        bits = lp.bits(sample["C5"])
        del lp
        return float(np.mean(tl.ms())), bits

    if not args.no_long:
        lcase = cases["C5"]
        lu = prompt_units(lcase)
        lms, gpu_bits["C5"] = time_long(lcase)
        ltf = lu["flops"] / (lms * 1e-3) / 1e12
        res["prefill_long"] = {"workload": "long non-windowed prompt 37,810 x 56 x 128, non-causal, bf16 P",
                               "ms": round(lms, 3), "tflops": round(ltf, 2),
                               "flops_per_call": lu["flops"]}
        res["roofline_prefill_long"] = roofline("mfma", ltf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                                                traffic_bytes("long", ["prompt_kernel"]),
                                                "prompt_kernel<128,bf16P> (long prompt)")
        # the same inputs with p32 on (P as two bf16 halves), the long prompt's variant
        lcase2 = _with_p(lcase, api.P_TWO)
        lu2 = prompt_units(lcase2)
        l2ms, gpu_bits["C5-p32"] = time_long(lcase2)
        l2tf = lu2["flops"] / (l2ms * 1e-3) / 1e12
        res["prefill_long_p32"] = {"workload": "long prompt 37,810 x 56 x 128, non-causal, p32 (P as two bf16 halves)",
                                   "ms": round(l2ms, 3), "tflops": round(l2tf, 2),
                                   "flops_per_call": lu2["flops"],
                                   "flop_accounting": "(2 + 2*2) * d per visible (row, head, key)"}
        res["roofline_prefill_long_p32"] = roofline(
            "mfma", l2tf, MFMA_BF16_PEAK_TFS, "TFLOP/s", traffic_bytes("long2", ["prompt_kernel"]),
            "prompt_kernel<128,p32> (long prompt)")

    # P as three bf16 parts (fp32-accurate P.V): the 12B prompt chunk and the long prompt
    tcase3 = _three(workloads.prompt_12b())
    tp3 = Prompter(tcase3)
    tu = prompt_units(tcase3)
    t3ms = time_cold(tp3, args.steps)
    del tp3
    res["prefill_three_parts"] = {"workload": "12B prompt chunk with P as three bf16 parts",
                                  "ms": round(t3ms, 5),
                                  "tflops": round(tu["flops"] / (t3ms * 1e-3) / 1e12, 2),
                                  "flops_per_call": tu["flops"],
                                  "flop_accounting": "(2 + 2*3) * d per visible (row, head, key)"}
    if not args.no_long:
        lcase3 = _with_p(cases["C5"], api.P_THREE)
        lu3 = prompt_units(lcase3)
        l3ms, gpu_bits["C5-3"] = time_long(lcase3)
        l3tf = lu3["flops"] / (l3ms * 1e-3) / 1e12
        res["prefill_long_three_parts"] = {"workload": "long prompt 37,810 x 56 x 128, non-causal, P as three bf16 parts",
                                           "ms": round(l3ms, 3), "tflops": round(l3tf, 2),
                                           "flops_per_call": lu3["flops"]}
        res["roofline_prefill_long_three_parts"] = roofline(
            "mfma", l3tf, MFMA_BF16_PEAK_TFS, "TFLOP/s", traffic_bytes("long3", ["prompt_kernel"]),
            "prompt_kernel<128,3 parts> (long prompt)")

    # block-sparse prompt slice: 64 rows of a 7,900-token prompt, 32 selected 64-key blocks a
    # row, 24/2 heads x 256, P as three parts
    scase = workloads.sparse_prompt()
    sp = SparsePrompter(scase)
    su = sparse_units(scase)
    sms = time_cold(sp, args.steps)
    del sp
    stf = su["flops"] / (sms * 1e-3) / 1e12
    res["prefill_sparse"] = {"workload": "block-sparse prompt slice: 64 rows at p0 7,836, 24/2 x 256, "
                                         "32 selected 64-key blocks a row, causal, P as three parts",
                             "ms": round(sms, 5), "tflops": round(stf, 2), "triples": su["triples"],
                             "flops_per_call": su["flops"],
                             "flop_accounting": "(2 + 2*3) * d per selected visible (row, head, key)"}
    res["roofline_prefill_sparse"] = roofline(
        "mfma", stf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
        traffic_bytes("sparse", ["prompt_rows_kernel", "prompt_merge_kernel"]),
        "prompt_rows_kernel<3 parts> + prompt_merge_kernel (sparse slice)")

    if not args.no_long and not args.no_prep:
        pr = Preparer()
        pr(); torch.cuda.synchronize()
        t = Timed()
        for _ in range(max(args.long_iters, 3)):
            with t:
                pr()
        ms = float(np.median(t.ms()))
        gbs = pr.bytes / (ms * 1e-3) / 1e9
        res["prepare_long"] = {"workload": "q/k preparation of the long prompt: 37,810 x 112 heads x 128, "
                                           "RMSNorm eps 1e-5 + split-half RoPE on dims 0-95, from the "
                                           "interleaved projection buffer",
                               "ms": round(ms, 4), "bytes_per_call": pr.bytes, "gbs": round(gbs, 2)}
        res["roofline_prepare_long"] = roofline(
            "hbm", gbs, HBM_PEAK_GBS, "GB/s", traffic_bytes("prepare_long", ["prepare_wide_kernel", "prepare_kernel"]),
            "prepare_wide_kernel<128> (RMSNorm + RoPE 96 dims, bf16 coefficients, 8 dims a lane)")
        del pr

    if oracle is not None:
        from oracle import check
        e_p = {"C1": check.E_P_FP32, "C2": check.E_P_FP32, "C2-D": check.E_P_FP32,
               "C3": check.E_P_P32, "C4": check.E_P_BF16, "C5": check.E_P_BF16}
        res["parity"] = {name: parity_entry(gpu_bits[name], oracle[name], e_p[name])
                         for name in oracle if name in gpu_bits}
        # the long prompt's P variants against the same float64 values (P's carrying changes
        # only the allowance e_P)
        for name, ep in (("C5-p32", check.E_P_P32), ("C5-3", check.E_P_THREE)):
            if "C5" in oracle and name in gpu_bits:
                res["parity"][name] = parity_entry(gpu_bits[name], oracle["C5"], ep)
        res["parity"]["note"] = ("outputs of the timed calls against the float64 oracle; C5: its "
                                 "seeded sample of 256 rows x 56 heads, with P as one bf16 (C5), "
                                 "two halves (C5-p32) and three parts (C5-3)")
        secs = {name: round(o["seconds"], 3) for name, o in oracle.items()}
        c2s = oracle["C2"]["seconds"]
        cb = {"value": round(du["unique_bytes"] / c2s / 1e9, 4), "unit": "GB/s", "cores": cores,
              "kind": "oracle",
              "sample": "every row of C1-C4 and the 64-stream decode, and the long prompt's "
                        "seeded 256 rows x 56 heads (14,336 (row, head) pairs); value = the 12B "
                        "decode's distinct ring bytes over its oracle time",
              "cpu_model": cpu_model(), "seconds_per_workload": secs,
              "parallelism": f"{cores} processes (os.sched_getaffinity, at most {CPU_SHARE}), "
                             "one BLAS thread each, rows split evenly"}
        if "C5" in oracle:
            n = cases["C5"].n
            cb["C5_full_extrapolated_s"] = round(oracle["C5"]["seconds"] * n / len(sample["C5"]), 1)
            cb["C5_extrapolation"] = f"sample seconds x {n}/{len(sample['C5'])} rows (linear)"
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
