"""Throughput of windowed GQA attention on one MI355X: decode KV GB/s and prefill TFLOP/s.

One step is one pass of the whole hot path of a Gemma-4-12B-shaped sliding layer:
  * decode: 64 rows over 3 streams, 16/8 heads x 256, window 1024 over a ring of 1536,
    positions up to 40,000 (split-KV chunk partials + ordered merge), and
  * prompt: a 512-row chunk at p0 5,000 with p32 and an image span (MFMA online softmax).
``value`` is the decode's key/value bytes per second in the accounting of TensorFold pull
request #1123's receipt (each row reads its visible keys' K and V: 8 MiB for a full 12B
row), with L2/MALL flushed (by reading 512 MiB) before every timed decode call. Prefill throughput
is reported beside it, and the long non-windowed prompt (37,810 x 56 x 128, non-causal) is
timed on its own as the MFMA-bound shape, followed by that prompt's q/k preparation
(RMSNorm + RoPE, the HBM-bound step on the input side).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--long-iters 3] [--no-cpu]
                    [--no-long] [--no-prep]

Prints one JSON line.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sliding_window_gqa_amd import api, workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
VALU_FP32_PEAK_TFS = 157.3   # MI355X fp32 vector (256 CUs x 2.4 GHz x 256 flop/clk, packed)
CHUNK = 256


def key_span(pos, win, last=None):
    lo = max(0, pos - win + 1) if win > 0 else 0
    return lo, pos if last is None else last


def decode_units(case):
    """Per the receipt's accounting: K and V bytes of every visible key of every row, plus q
    and out; and the unique K/V bytes (distinct ring slots touched per stream and head)."""
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
    G = case.hq // case.hkv
    for r in range(case.rows):
        lo, last = key_span(int(case.pos[r]), case.win)
        flops += (last - lo + 1) * case.hkv * G * case.d * 2 * 2
    return {"kv_bytes": per_row, "unique_bytes": unique + qo, "row_bytes": per_row + qo,
            "flops_fp32": flops}


def prompt_units(case):
    """MFMA flops the method performs: 2d for S and 2d per P.V product per visible
    (row, head, key); P.V runs once per bf16 part of P (one, two with p32, or three)."""
    pv = 1 + api._p_mode(case.p32)
    triples = 0
    for i in range(case.n):
        last = None if case.hi is None else int(case.hi[i])
        lo, hi = key_span(case.p0 + i, case.win, last)
        triples += (hi - lo + 1)
    triples *= case.hq
    flops = triples * (2 + 2 * pv) * case.d
    byts = (case.q.size + case.q.size + 2 * case.k.shape[0] * case.k.shape[1] * case.d) * 2
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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


class Timed:
    """HIP events on the current stream around each call."""

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


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def cpu_baseline(case, budget_s=10.0):
    """The float64 oracle on the decode workload's rows, on the host cores."""
    from oracle import attend
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    units = decode_units(case)
    t0 = time.perf_counter()
    reps = 0
    while True:
        attend.decode(case.q, case.k, case.v, case.stream, case.pos, case.win, case.ring, case.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(units["kv_bytes"] * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"all {case.rows} rows of the decode workload, {reps} pass(es) in {dt:.1f} s "
                      f"(numpy float64, BLAS threads as shown)"}


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


def prepare_long_leg(iters):
    pr = Preparer()
    pr(); torch.cuda.synchronize()
    t = Timed()
    for _ in range(max(iters, 3)):
        with t:
            pr()
    ms = float(np.median(t.ms()))
    gbs = pr.bytes / (ms * 1e-3) / 1e9
    rl = roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", traffic_bytes("prepare_long", ["prepare_kernel"]))
    rl["kernel"] = "prepare_kernel<128> (RMSNorm + RoPE 96 dims, bf16 coefficients)"
    out = {"prepare_long": {"workload": "q/k preparation of the long prompt: 37,810 x 112 heads x 128, "
                                        "RMSNorm eps 1e-5 + split-half RoPE on dims 0-95, from the "
                                        "interleaved projection buffer",
                            "ms": round(ms, 4), "bytes_per_call": pr.bytes, "gbs": round(gbs, 2)},
           "roofline_prepare_long": rl}
    del pr
    return out


def _three(case):
    case.p32 = api.P_THREE
    return case


def profile_driver(names, iters):
    """Run the workloads for profiler passes, after a plain copy of known size."""
    a = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)                     # 256 MiB read + 256 MiB written: counter calibration
    torch.cuda.synchronize()
    del a, b
    make = {"decode12b": lambda: Decoder(workloads.decode_12b()),
            "decode12b64": lambda: Decoder(workloads.decode_12b(streams=64)),
            "prompt12b": lambda: Prompter(workloads.prompt_12b()),
            "prompt31b": lambda: Prompter(workloads.prompt_31b()),
            "long": lambda: Prompter(workloads.long_prompt()),
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--long-iters", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-prep", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiler driver: run a 256 MiB device copy (counter calibration), then "
                         "each listed workload (decode12b, decode12b64, prompt12b, prompt12b3, "
                         "prompt31b, sparse, long, long3, prepare_long) --steps times; no timing, "
                         "no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards without exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    api.lib()
    if args.only:
        profile_driver(args.only.split(","), args.steps)
        return

    dcase = workloads.decode_12b()
    pcase = workloads.prompt_12b()
    dec, pro = Decoder(dcase), Prompter(pcase)
    du, pu = decode_units(dcase), prompt_units(pcase)
    # cache flush between timed calls: READ a 512 MiB buffer (> 256 MB MALL, > L2), which
    # evicts the working set without leaving dirty lines whose write-back would land in the
    # timed call
    flush_buf = torch.ones(64 * 2**20, dtype=torch.int64, device="cuda")
    flush_out = torch.empty(1, dtype=torch.int64, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

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
    # warm-cache decode, for reference
    tw = Timed()
    for _ in range(args.steps):
        with tw:
            dec()
    dms_warm = float(np.mean(tw.ms()))

    # the same decode shape with 64 streams (one row each): no keys shared between rows, so
    # every per-row byte is an HBM byte -- the clean HBM-roofline shape
    hcase = workloads.decode_12b(streams=64)
    hdec, hu = Decoder(hcase), decode_units(hcase)
    for _ in range(args.warmup):
        hdec()
    th = Timed()
    for _ in range(args.steps):
        flush()
        with th:
            hdec()
    hms = float(np.mean(th.ms()))
    del hdec

    kv_gbs = du["kv_bytes"] / (dms * 1e-3) / 1e9
    pre_tfs = pu["flops"] / (pms * 1e-3) / 1e12
    res = {
        "metric": "decode KV GB/s + prefill TFLOP/s, hd256 GQA window attn, % of roofline",
        "value": round(kv_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dms + pms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded; receipt distributions)",
        "config": {"workload": "Gemma-4-12B-shaped sliding layer step: decode 64 rows over 3 "
                               "streams (16/8 x 256, window 1024, ring 1536, pos < 40,000) + "
                               "prompt chunk 512 rows at p0 5,000 (p32, image rows 40..300)",
                   "decode_rows": 64, "prompt_rows": 512, "window": 1024, "ring": 1536},
        "decode": {"ms": round(dms, 5), "ms_warm_cache": round(dms_warm, 5),
                   "kv_bytes_per_call": du["kv_bytes"], "unique_bytes_per_call": du["unique_bytes"],
                   "kv_gbs_warm": round(du["kv_bytes"] / (dms_warm * 1e-3) / 1e9, 2),
                   "unique_gbs": round(du["unique_bytes"] / (dms * 1e-3) / 1e9, 2)},
        "prefill": {"ms": round(pms, 5), "tflops": round(pre_tfs, 2), "flops_per_call": pu["flops"],
                    "flop_accounting": "(2 + 2*2) * d per visible (row, head, key), p32"},
        "wall_s_timed_loop": round(wall, 3),
    }
    rl_prompt = roofline("mfma", pre_tfs, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                         traffic_bytes("prompt12b", ["prompt_kernel", "prompt_merge_kernel"]))
    rl_prompt["kernel"] = "prompt_kernel<256,p32> + prompt_merge_kernel (12B prompt chunk)"
    # The rows share three rings: the per-row K/V reads come from L2/MALL and the call is
    # bound by its fp32 VALU work (q.k and p.v fmas), not by HBM bytes; both views are given.
    dec_tfs = du["flops_fp32"] / (dms * 1e-3) / 1e12
    dec_traffic = traffic_bytes("decode12b", ["decode_kernel", "merge_kernel"])
    rl_decode = roofline("alu", dec_tfs, VALU_FP32_PEAK_TFS, "TFLOP/s", dec_traffic)
    rl_decode["kernel"] = "decode_kernel<256,2,chunks> + merge_kernel (fp32 q.k and p.v work)"
    rl_decode_hbm = roofline("hbm", du["unique_bytes"] / (dms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                             dec_traffic)
    rl_decode_hbm["kernel"] = "decode_kernel<256,2,chunks> + merge_kernel (unique K/V bytes)"
    res["roofline"] = rl_prompt if pms >= dms else rl_decode
    res["roofline_decode"] = rl_decode
    res["roofline_decode_unique_bytes"] = rl_decode_hbm
    res["roofline_prefill"] = rl_prompt
    hgbs = hu["row_bytes"] / (hms * 1e-3) / 1e9
    res["decode_64_streams"] = {"workload": "12B decode shape, 64 rows in 64 streams (no shared keys)",
                                "ms": round(hms, 5), "bytes_per_call": hu["row_bytes"],
                                "gbs": round(hgbs, 2)}
    rl_h = roofline("hbm", hgbs, HBM_PEAK_GBS, "GB/s",
                    traffic_bytes("decode12b64", ["decode_kernel", "merge_kernel"]))
    rl_h["kernel"] = "decode_kernel<256,2,whole rows> (64 streams, no shared keys)"
    res["roofline_decode_64_streams"] = rl_h

    if not args.no_long:
        lcase = workloads.long_prompt()
        lp = Prompter(lcase)
        lu = prompt_units(lcase)
        lp(); torch.cuda.synchronize()
        tl = Timed()
        for _ in range(args.long_iters):
            with tl:
                lp()
        lms = float(np.mean(tl.ms()))
        ltf = lu["flops"] / (lms * 1e-3) / 1e12
        res["prefill_long"] = {"workload": "long non-windowed prompt 37,810 x 56 x 128, non-causal, bf16 P",
                               "ms": round(lms, 3), "tflops": round(ltf, 2),
                               "flops_per_call": lu["flops"]}
        rl = roofline("mfma", ltf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                      traffic_bytes("long", ["prompt_kernel"]))
        rl["kernel"] = "prompt_kernel<128,bf16P> (long prompt)"
        res["roofline_prefill_long"] = rl
        del lp

    # P as three bf16 parts (fp32-accurate P.V): the 12B prompt chunk and the long prompt
    tcase = workloads.prompt_12b()
    tcase.p32 = api.P_THREE
    tp3 = Prompter(tcase)
    tu = prompt_units(tcase)
    for _ in range(args.warmup):
        tp3()
    t3 = Timed()
    for _ in range(args.steps):
        flush()
        with t3:
            tp3()
    t3ms = float(np.mean(t3.ms()))
    res["prefill_three_parts"] = {"workload": "12B prompt chunk with P as three bf16 parts",
                                  "ms": round(t3ms, 5),
                                  "tflops": round(tu["flops"] / (t3ms * 1e-3) / 1e12, 2),
                                  "flops_per_call": tu["flops"],
                                  "flop_accounting": "(2 + 2*3) * d per visible (row, head, key)"}
    del tp3
    if not args.no_long:
        lcase3 = workloads.long_prompt(p32=api.P_THREE)
        lp3 = Prompter(lcase3)
        lu3 = prompt_units(lcase3)
        lp3(); torch.cuda.synchronize()
        tl3 = Timed()
        for _ in range(args.long_iters):
            with tl3:
                lp3()
        l3ms = float(np.mean(tl3.ms()))
        l3tf = lu3["flops"] / (l3ms * 1e-3) / 1e12
        res["prefill_long_three_parts"] = {"workload": "long prompt 37,810 x 56 x 128, non-causal, P as three bf16 parts",
                                           "ms": round(l3ms, 3), "tflops": round(l3tf, 2),
                                           "flops_per_call": lu3["flops"]}
        rl3 = roofline("mfma", l3tf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                       traffic_bytes("long3", ["prompt_kernel"]))
        rl3["kernel"] = "prompt_kernel<128,3 parts> (long prompt)"
        res["roofline_prefill_long_three_parts"] = rl3
        del lp3

    # block-sparse prompt slice: 64 rows of a 7,900-token prompt, 32 selected 64-key blocks a
    # row, 24/2 heads x 256, P as three parts
    scase = workloads.sparse_prompt()
    sp = SparsePrompter(scase)
    su = sparse_units(scase)
    for _ in range(args.warmup):
        sp()
    tsp = Timed()
    for _ in range(args.steps):
        flush()
        with tsp:
            sp()
    sms = float(np.mean(tsp.ms()))
    stf = su["flops"] / (sms * 1e-3) / 1e12
    res["prefill_sparse"] = {"workload": "block-sparse prompt slice: 64 rows at p0 7,836, 24/2 x 256, "
                                         "32 selected 64-key blocks a row, causal, P as three parts",
                             "ms": round(sms, 5), "tflops": round(stf, 2), "triples": su["triples"],
                             "flops_per_call": su["flops"],
                             "flop_accounting": "(2 + 2*3) * d per selected visible (row, head, key)"}
    rls = roofline("mfma", stf, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                   traffic_bytes("sparse", ["prompt_kernel", "prompt_merge_kernel"]))
    rls["kernel"] = "prompt_kernel<256,3 parts> sparse + prompt_merge_kernel"
    res["roofline_prefill_sparse"] = rls
    del sp

    if not args.no_long and not args.no_prep:
        res.update(prepare_long_leg(args.long_iters))

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(dcase)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
