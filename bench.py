#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step runs the five benchmark workloads once each, every input resident in
HBM before timing starts:
  C1 tiny non-causal MHA (B1, Hq=Hkv=2, S256, D64),
  C2 causal GQA prefill (B1, Hq32/Hkv4, S4096, D128),
  C3 long causal GQA prefill (B1, Hq16/Hkv2, S16384, D256),
  C4 varlen causal sliding-window prefill (8 packed sequences, Hq32/Hkv8, D128,
     window 1024 left / 0 right),
  C5 paged split-KV decode (B16, Hq32/Hkv4, D128, Sk32768, 256-token pages in
     a random page table, 16 splits, then the LSE combine).

Prints ONE JSON line on stdout. `value` is C3's (the largest prefill that fits
one GPU) algorithmic throughput: 4*D*(visible query-key pairs)*Hq flops per
launch (causal pairs only) over the launch's duration, measured with HIP events
recorded on the launch stream around every launch of the timed steps. Every
workload has its own entry under "workloads" (average launch time, throughput,
roofline fraction, HBM counter traffic); the decode's K/V bytes per second is
also under "decode". Outside the step, "backward" holds the same figures for
the backward of C2 and C3 (one mi_attn_bwd call: all its launches). Progress
goes to stderr.

Flags: --gpus N (only 1 is supported: the path is single-GPU), --steps K,
--warmup W, --warmup-gpu-ms T, --no-cpu-baseline, --cpu-seconds S (oracle
sample budget), --no-backward (skip the backward entries), --all-configs (also
time further workloads: head dims 96/192, paged prefill, softcap, a multi-token
decode step, fp8 decode), --zero-inputs (prefill workloads
on all-zero inputs; a clock measurement, never the reported value's data).

Warm-up: W untimed steps, then more untimed steps until at least T ms (default
1000) of GPU time has passed since the first. The core clock climbs only under
sustained matrix-core load; a step-count warm-up of a few steps times the
prefill kernels ~20% slower than they run in steady state. The line states
both (`warmup`, `warmup_gpu_ms`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (causal-adjusted) + decode KV GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "exact_attention_45_amd", "csrc")
PROFILES = os.path.join(HERE, "profiles")
# sources whose compiled code the counted kernels consist of
KERNEL_SOURCES = {
    "fwd_pp_kernel<64>": ["fwd_pp_kernel.hip", "attn_common.hpp", "kernels.hpp"],
    "fwd_pp_kernel<128>": ["fwd_pp_kernel.hip", "attn_common.hpp", "kernels.hpp"],
    "fwd_sp_kernel<256,1>": ["fwd_sp_kernel.hip", "attn_common.hpp", "kernels.hpp"],
    "decode_stream_kernel<128>": ["decode_stream_kernel.hip", "attn_common.hpp", "kernels.hpp"],
    "combine_kernel<128>": ["decode_kernel.hip", "attn_common.hpp", "kernels.hpp"],
}
for _d in (128, 256):
    for _k in ("bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dkdv_pair_kernel",
               "bwd_dkv_reduce_kernel"):
        KERNEL_SOURCES[f"{_k}<{_d}>"] = ["bwd_kernel.hip", "bwd.hpp", "attn_common.hpp"]
# the backward's launches per call, by head dim (the reduce runs when the dK/dV
# walk is split, which the two measured workloads' shapes decide)
BWD_KERNELS = {128: ["bwd_pre_kernel<128>", "bwd_dq_kernel<128>", "bwd_dkdv_kernel<128>",
                     "bwd_dkv_reduce_kernel<128>"],
               256: ["bwd_pre_kernel<256>", "bwd_dq_kernel<256>", "bwd_dkdv_pair_kernel<256>"]}


def _code_text(src: str) -> str:
    """The source with comments, trailing blanks and empty lines removed: an
    edit to a comment leaves the compiled kernel, and so its counters, as they
    were. (The sources hold no string literal containing a comment marker.)"""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (ln.split("//", 1)[0].rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_digest(kernel: str) -> str:
    """Digest of the code (not the comments) of the sources a kernel is
    compiled from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def _traffic_lines():
    """`traffic:` lines of the committed counter summaries under profiles/."""
    found = {}
    try:
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return found
    for n in names:
        if not n.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, n)) as fh:
            for ln in fh.read().splitlines():
                if ln.startswith("traffic: "):
                    kv = dict(t.split("=", 1) for t in ln[len("traffic: "):].split())
                    found[(kv.get("kernel"), kv.get("workload"))] = kv
    return found


def counter_traffic(workload: str, *kernels: str):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of `workload`, summed
    over `kernels`, read from the committed counter summaries; None when a
    summary has no line for one of them or the kernel's sources changed since
    the counters were taken."""
    found = _traffic_lines()
    total = 0
    for k in kernels:
        kv = found.get((k, workload))
        if kv is None or kv.get("source_sha256") != source_digest(k):
            return None
        total += int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return total


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-gpu-ms", type=float, default=1000.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--all-configs", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="prefill workloads on all-zero Q/K/V (the same kernels and cycle "
                         "counts; the matrix cores then draw less power and the core clock "
                         "runs higher): shows how much of a launch's duration is clock")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the "
                         "reference kernel for scaling HBM byte counters), then exit")
    return ap.parse_args()


def copy_calibration(torch):
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 copies of {n} bytes")


def prefill_flops(w) -> float:
    if w.kind == "varlen":
        pairs = 0
        for b in range(len(w.cu_seqlens_q) - 1):
            lq = int(w.cu_seqlens_q[b + 1] - w.cu_seqlens_q[b])
            lk = int(w.cu_seqlens_k[b + 1] - w.cu_seqlens_k[b])
            pairs += _pairs(lq, lk, w.causal, w.window_left, w.window_right)
    elif w.kind == "paged_prefill":
        cap = w.page_table.shape[1] * w.page_size
        pairs = 0
        for b in range(w.batch):
            lk = cap if w.seqused_k is None else int(w.seqused_k[b])
            lq = (int(w.cu_seqlens_q[b + 1] - w.cu_seqlens_q[b]) if w.cu_seqlens_q is not None
                  else w.seqlen_q)
            pairs += _pairs(lq, lk, w.causal, w.window_left, w.window_right)
    else:
        pairs = w.batch * _pairs(w.seqlen_q, w.seqlen_k, w.causal, w.window_left, w.window_right)
    return 4.0 * w.head_dim * w.num_heads_q * pairs


def _pairs(sq, sk, causal, wl, wr) -> int:
    """Visible (query, key) pairs of one head, closed form per row."""
    right = 0 if causal else (None if wr is None or wr < 0 else wr)
    left = None if wl is None or wl < 0 else wl
    tot = 0
    off = sk - sq
    for i in range(sq):
        lo = 0 if left is None else max(0, i + off - left)
        hi = sk - 1 if right is None else min(sk - 1, i + off + right)
        tot += max(0, hi - lo + 1)
    return tot


def decode_bytes(w) -> int:
    elem = 1 if w.kv_dtype.startswith("fp8") else 2
    kv = 2 * int(w.seqused_k.sum()) * w.num_heads_kv * w.head_dim * elem
    q = w.batch * w.num_heads_q * w.head_dim * 2
    o = q
    lse = w.batch * w.num_heads_q * 4
    table = sum(-(-int(s) // w.page_size) for s in w.seqused_k) * 4
    descale = 0 if w.k_descale is None else 2 * w.batch * w.num_heads_kv * 4
    return kv + q + o + lse + table + descale


class Prefill:
    def __init__(self, mi, w, torch, softcap: float = 0.0, zero: bool = False):
        from tests.gpu_util import dev_bf16, dev_i32
        self.mi, self.w = mi, w
        self.q, self.k, self.v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
        if zero:
            for t in (self.q, self.k, self.v):
                t.zero_()
        self.kw = dict(softmax_scale=w.softmax_scale, causal=w.causal,
                       window_left=w.window_left, window_right=w.window_right, softcap=softcap)
        if w.kind == "varlen":
            self.kw.update(cu_seqlens_q=dev_i32(w.cu_seqlens_q), cu_seqlens_k=dev_i32(w.cu_seqlens_k),
                           max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k)
        if w.kind == "paged_prefill":
            self.kw.update(page_table=dev_i32(w.page_table),
                           seqused_k=None if w.seqused_k is None else dev_i32(w.seqused_k))
        self.out, self.lse = mi.mi_attn_fwd(self.q, self.k, self.v, **self.kw)

    def __call__(self):
        self.mi.mi_attn_fwd(self.q, self.k, self.v, out=self.out, lse=self.lse, **self.kw)


class Decode:
    def __init__(self, mi, w, torch):
        from tests.gpu_util import dev_bf16, dev_i32
        self.mi, self.w = mi, w
        self.q = dev_bf16(w.q)
        self.kd = self.vd = None
        if w.kv_dtype.startswith("fp8"):
            dt = {"fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2}[w.kv_dtype]
            self.kc = torch.from_numpy(w.k).to("cuda").view(dt)
            self.vc = torch.from_numpy(w.v).to("cuda").view(dt)
            if w.k_descale is not None:
                self.kd = torch.from_numpy(w.k_descale).to("cuda")
                self.vd = torch.from_numpy(w.v_descale).to("cuda")
        else:
            self.kc, self.vc = dev_bf16(w.k), dev_bf16(w.v)
        self.pt, self.su = dev_i32(w.page_table), dev_i32(w.seqused_k)
        nb = mi.mi_attn_decode_workspace_bytes(self.q, self.kc, self.vc, self.pt, w.num_splits)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.out, self.lse = mi.mi_attn_decode_splitkv(
            self.q, self.kc, self.vc, self.pt, seqused_k=self.su, softmax_scale=w.softmax_scale,
            num_splits=w.num_splits, workspace=self.ws, k_descale=self.kd, v_descale=self.vd)

    def __call__(self):
        self.mi.mi_attn_decode_splitkv(self.q, self.kc, self.vc, self.pt, seqused_k=self.su,
                                       out=self.out, lse=self.lse,
                                       softmax_scale=self.w.softmax_scale,
                                       num_splits=self.w.num_splits, workspace=self.ws,
                                       k_descale=self.kd, v_descale=self.vd)


class VarlenDecode:
    """mi_attn_decode_splitkv with several query tokens per sequence (packed
    by cu_seqlens_q, causal), split heuristic."""

    def __init__(self, mi, w, torch):
        from tests.gpu_util import dev_bf16, dev_i32
        self.mi, self.w = mi, w
        self.q, self.kc, self.vc = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
        self.pt, self.su = dev_i32(w.page_table), dev_i32(w.seqused_k)
        self.cu = dev_i32(w.cu_seqlens_q)
        self.kw = dict(seqused_k=self.su, cu_seqlens_q=self.cu, max_seqlen_q=w.max_seqlen_q,
                       causal=True, softmax_scale=w.softmax_scale, num_splits=0)
        nb = mi.mi_attn_decode_workspace_bytes(self.q, self.kc, self.vc, self.pt, 0, self.cu,
                                               w.max_seqlen_q)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.out, self.lse = mi.mi_attn_decode_splitkv(self.q, self.kc, self.vc, self.pt,
                                                       workspace=self.ws, **self.kw)

    def __call__(self):
        self.mi.mi_attn_decode_splitkv(self.q, self.kc, self.vc, self.pt, out=self.out,
                                       lse=self.lse, workspace=self.ws, **self.kw)


def varlen_decode_bytes(w) -> int:
    kv = 2 * int(w.seqused_k.sum()) * w.num_heads_kv * w.head_dim * 2
    tq = int(w.cu_seqlens_q[-1])
    qo = 2 * tq * w.num_heads_q * w.head_dim * 2
    lse = tq * w.num_heads_q * 4
    table = sum(-(-int(s) // w.page_size) for s in w.seqused_k) * 4
    return kv + qo + lse + table + 4 * (len(w.seqused_k) + 1)


class Backward:
    """mi_attn_bwd on a dense workload: the forward's out and LSE are made
    once, outside the timed calls; each call runs the backward's launches
    (row sums of O dO and LSE log2 e, dQ, dK/dV, and the reduce of split dK/dV
    partials). `dev` reuses the device q, k, v of a Prefill of the same
    workload."""

    def __init__(self, mi, w, torch, dev=None):
        import workloads as W
        from tests.gpu_util import dev_bf16
        self.mi, self.w = mi, w
        if dev is not None:
            self.q, self.k, self.v = dev.q, dev.k, dev.v
        else:
            self.q, self.k, self.v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
        self.kw = dict(softmax_scale=w.softmax_scale, causal=w.causal,
                       window_left=w.window_left, window_right=w.window_right)
        self.out, self.lse = mi.mi_attn_fwd(self.q, self.k, self.v, **self.kw)
        self.g = dev_bf16(W.grad_output(w.seed, tuple(self.q.shape)))
        self.dq, self.dk, self.dv = (torch.empty_like(self.q), torch.empty_like(self.k),
                                     torch.empty_like(self.v))
        nb = mi.mi_attn_bwd_workspace_bytes(self.q, self.k, self.v, self.out, self.g, self.lse)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def __call__(self):
        self.mi.mi_attn_bwd(self.q, self.k, self.v, self.out, self.g, self.lse, dq=self.dq,
                            dk=self.dk, dv=self.dv, workspace=self.ws, **self.kw)


def time_launches(torch, fn, n):
    """Per-launch durations (ms) from HIP events on the launch stream."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def warm_up(torch, fn, gpu_ms: float = 40.0):
    """Runs fn until about gpu_ms of GPU time has passed: the core clock drops
    while the host prepares a workload and climbs back only under sustained
    load, so short kernels need many launches before they are timed."""
    fn()
    torch.cuda.synchronize()
    per = max(min(time_launches(torch, fn, 3)), 1e-3)
    for _ in range(int(min(5000, max(3, gpu_ms / per)))):
        fn()
    torch.cuda.synchronize()


def cpu_baseline(w, budget_s: float):
    """The float64 oracle on a bounded sample of a dense causal prefill
    workload: blocks of 512 query rows (full fp64 score rows against every
    key, masked as the definition says), taken from the last rows backwards,
    query head 0 first, then head 1, ..., until the budget is spent.
    Throughput uses the same causal-adjusted flop count (visible pairs of the
    sampled rows)."""
    import numpy as np
    import oracle.attention as OA
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    S, r = w.seqlen_q, w.num_heads_q // w.num_heads_kv
    blk = 512
    t0 = time.perf_counter()
    pairs = rows = 0
    heads = set()
    done = False
    for h in range(w.num_heads_q):
        g = h // r
        k = W.bf16_bits_to_f64(w.k[0, :, g])
        v = W.bf16_bits_to_f64(w.v[0, :, g])
        for hi in range(S, 0, -blk):
            pos = np.arange(max(0, hi - blk), hi)
            q = W.bf16_bits_to_f64(w.q[0, pos, h])
            OA.attention_rows(q, pos, k, v, w.softmax_scale, S, w.causal, w.window_left,
                              w.window_right)
            pairs += int(OA.visible_mask(S, w.seqlen_k, w.causal, w.window_left,
                                         w.window_right, rows=pos).sum())
            rows += len(pos)
            heads.add(h)
            if time.perf_counter() - t0 >= budget_s:
                done = True
                break
        if done:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.head_dim * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} query rows ({pairs} visible pairs) of {len(heads)} of "
                      f"{w.num_heads_q} query heads of the {w.name} workload, full fp64 "
                      f"score rows, {dt:.1f} s wall"}


# (workload id, label, kernel(s) the counters and the roofline refer to)
STEP = (
    (1, "C1 tiny non-causal MHA B1 Hq2 Hkv2 S256 D64", ("fwd_pp_kernel<64>",)),
    (2, "C2 causal GQA prefill B1 Hq32 Hkv4 S4096 D128", ("fwd_pp_kernel<128>",)),
    (3, "C3 long causal GQA prefill B1 Hq16 Hkv2 S16384 D256", ("fwd_sp_kernel<256,1>",)),
    (4, "C4 varlen causal window prefill 8 seqs Hq32 Hkv8 D128 wl1024 wr0",
     ("fwd_pp_kernel<128>",)),
    (5, "C5 paged split-KV decode B16 Hq32 Hkv4 D128 Sk32768 page256 16 splits",
     ("decode_stream_kernel<128>", "combine_kernel<128>")),
)
HEADLINE = 3


def timed_extra(torch, fn, n):
    """Median per-launch duration (ms) of fn after a 40 ms GPU-time warm-up."""
    warm_up(torch, fn)
    ms = sorted(time_launches(torch, fn, n))
    return ms[len(ms) // 2]


def backward_workloads(mi, W, torch, args, runs, ws):
    """The backward of the causal GQA S4096 D128 and S16384 D256 prefill
    workloads (median of event-timed calls after a GPU-time warm-up). The
    algorithmic flops are 2.5x the forward's: five tile products per score
    tile (S, dP, dV, dK, dQ) against two."""
    res = {}
    n = max(5, args.steps // 2)
    for i in (2, 3):
        w = ws[i]
        bw = Backward(mi, w, torch, dev=runs[i])
        med = timed_extra(torch, bw, n)
        f = 2.5 * prefill_flops(w)
        tf = f / (med * 1e-3) / 1e12
        d = w.head_dim
        res[w.name] = {"label": f"backward of {w.name}", "kernel": " + ".join(BWD_KERNELS[d]),
                       "avg_call_us": round(med * 1e3, 2), "bound": "mfma",
                       "achieved": round(tf, 2), "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
                       "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_call": f,
                       "traffic": counter_traffic("backward_" + w.name, *BWD_KERNELS[d])}
        log(f"[bench] backward {w.name}: {med * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        del bw
        torch.cuda.empty_cache()
    return res


def extra_workloads(mi, W, torch, args, extra):
    """--all-configs: head dims 96/192, paged prefill, softcap, the multi-token
    decode step, fp8 decode and the decode at D96/D192/D256 (median of
    event-timed launches, stderr and "other_workloads")."""
    n = max(5, args.steps)
    paged = W.paged_prefill_case(1002, 1, 32, 4, 128, 256, 16, None, seqlen_q=4096,
                                 causal=True, name="paged256_causal_gqa32x4_s4096_d128")
    d96 = W.dense_case(1006, 1, 4096, 4096, 32, 4, 96, causal=True,
                       name="causal_gqa32x4_s4096_d96")
    d192 = W.dense_case(1007, 1, 8192, 8192, 16, 2, 192, causal=True,
                        name="causal_gqa16x2_s8192_d192")
    for wi in (paged, d96, d192):
        p = Prefill(mi, wi, torch)
        med = timed_extra(torch, p, n)
        f = prefill_flops(wi)
        extra[wi.name] = {"median_us": med * 1e3, "tflops": f / (med * 1e-3) / 1e12,
                          "frac": f / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        log(f"[bench] {wi.name}: {med * 1e3:.1f} us, {extra[wi.name]['tflops']:.1f} TFLOP/s")
        del p
        torch.cuda.empty_cache()
    wc = W.standard_config(2)
    pc = Prefill(mi, wc, torch, softcap=30.0)
    med = timed_extra(torch, pc, n)
    f = prefill_flops(wc)
    name = "softcap30_" + wc.name
    extra[name] = {"median_us": med * 1e3, "tflops": f / (med * 1e-3) / 1e12,
                   "frac": f / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    log(f"[bench] {name}: {med * 1e3:.1f} us, {extra[name]['tflops']:.1f} TFLOP/s")
    del pc
    torch.cuda.empty_cache()
    # speculative decoding step: the paged decode workload's cache with 4
    # causal query tokens per sequence
    wv = W.paged_prefill_case(1005, 16, 32, 4, 128, 256, 128, [32768] * 16, seqlens_q=[4] * 16,
                              causal=True, name="paged_decode_4tok_b16_gqa32x4_sk32768_d128")
    vd = VarlenDecode(mi, wv, torch)
    med = timed_extra(torch, vd, n)
    gb = varlen_decode_bytes(wv) / (med * 1e-3) / 1e9
    extra[wv.name] = {"median_us": med * 1e3, "gbs": gb, "frac": gb / PEAK_HBM_GBS,
                      "bytes_per_launch": varlen_decode_bytes(wv)}
    log(f"[bench] {wv.name}: {med * 1e3:.1f} us, {gb:.0f} GB/s")
    del vd, wv
    torch.cuda.empty_cache()
    for fmt, wname in (("e4m3", "paged_decode_fp8_b16_sk32768"),
                       ("e5m2", "paged_decode_fp8_e5m2_b16_sk32768")):
        w8 = W.paged_decode_fp8_case(1005, 16, 32, 4, 128, 256, 128, num_splits=16,
                                     name=wname, fmt=fmt)
        d8 = Decode(mi, w8, torch)
        med = timed_extra(torch, d8, n)
        gb = decode_bytes(w8) / (med * 1e-3) / 1e9
        extra[w8.name] = {"median_us": med * 1e3, "gbs": gb, "frac": gb / PEAK_HBM_GBS,
                          "bytes_per_launch": decode_bytes(w8)}
        log(f"[bench] {w8.name}: {med * 1e3:.1f} us, {gb:.0f} GB/s")
        del d8, w8
        torch.cuda.empty_cache()
    # the decode at head dims 96, 192, 256: B8 Hq32 Hkv4 Sk16384 with 256-token
    # pages, the heuristic's split count
    for wd in (W.paged_decode_case(1008, 8, 32, 4, 256, 256, 64,
                                   name="paged_decode_b8_gqa32x4_sk16384_d256"),
               W.paged_decode_case(1009, 8, 32, 4, 192, 256, 64,
                                   name="paged_decode_b8_gqa32x4_sk16384_d192"),
               W.paged_decode_case(1012, 8, 32, 4, 96, 256, 64,
                                   name="paged_decode_b8_gqa32x4_sk16384_d96"),
               W.paged_decode_fp8_case(1010, 8, 32, 4, 256, 256, 64,
                                       name="paged_decode_fp8_b8_sk16384_d256", fmt="e4m3")):
        dd = Decode(mi, wd, torch)
        med = timed_extra(torch, dd, n)
        gb = decode_bytes(wd) / (med * 1e-3) / 1e9
        extra[wd.name] = {"median_us": med * 1e3, "gbs": gb, "frac": gb / PEAK_HBM_GBS,
                          "bytes_per_launch": decode_bytes(wd)}
        log(f"[bench] {wd.name}: {med * 1e3:.1f} us, {gb:.0f} GB/s")
        del dd, wd
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention "
              "path here is single-GPU, see the sharding notes in the design document",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import exact_attention_45_amd as mi
    import workloads as W

    if args.copy_calibration:
        torch.cuda.init()
        copy_calibration(torch)
        return
    mi.load()  # raises if the HIP library is missing
    torch.cuda.init()
    log("[bench] generating inputs")
    ws, runs, work = {}, {}, {}
    for i, label, _ in STEP:
        ws[i] = W.standard_config(i)
        if ws[i].kind == "paged":
            runs[i] = Decode(mi, ws[i], torch)
            work[i] = decode_bytes(ws[i])
        else:
            runs[i] = Prefill(mi, ws[i], torch, zero=args.zero_inputs)
            work[i] = prefill_flops(ws[i])
        if i not in (HEADLINE,):
            ws[i].q = ws[i].k = ws[i].v = None  # host copies no longer needed
    torch.cuda.synchronize()

    def step():
        for i, _, _ in STEP:
            runs[i]()

    stream = torch.cuda.current_stream()
    log(f"[bench] warmup: {args.warmup} steps, then until {args.warmup_gpu_ms:.0f} ms of GPU time")
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    t0 = time.perf_counter()
    nw = 0
    while nw < args.warmup or (time.perf_counter() - t0) * 1e3 < args.warmup_gpu_ms:
        step()
        nw += 1
        if nw % 8 == 0:
            torch.cuda.synchronize()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_gpu_ms = w0.elapsed_time(w1)

    log(f"[bench] timing {args.steps} steps")
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in STEP] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        for (i, _, _), (a, b) in zip(STEP, e):
            a.record(stream)
            runs[i]()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {}
    for j, (i, label, kernels) in enumerate(STEP):
        ms = [e[j][0].elapsed_time(e[j][1]) for e in ev]
        avg = sum(ms) / len(ms)
        rec = {"label": label, "kernel": " + ".join(kernels), "avg_launch_us": round(avg * 1e3, 2),
               "min_launch_us": round(min(ms) * 1e3, 2)}
        if ws[i].kind == "paged":
            gbs = work[i] / (avg * 1e-3) / 1e9
            rec.update({"bound": "hbm", "achieved": round(gbs, 1), "unit": "GB/s",
                        "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "bytes_per_launch": work[i]})
            log(f"[bench] {label}: {avg * 1e3:.1f} us, {gbs:.0f} GB/s")
        else:
            tf = work[i] / (avg * 1e-3) / 1e12
            rec.update({"bound": "mfma", "achieved": round(tf, 2), "unit": "TFLOP/s",
                        "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "flops_per_launch": work[i]})
            log(f"[bench] {label}: {avg * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        rec["traffic"] = counter_traffic(ws[i].name, *kernels)
        per[ws[i].name] = rec

    bwd = None if args.no_backward else backward_workloads(mi, W, torch, args, runs, ws)

    extra = {}
    if args.all_configs:
        del runs
        torch.cuda.empty_cache()
        extra_workloads(mi, W, torch, args, extra)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(ws[HEADLINE], args.cpu_seconds)
        log(f"[bench] oracle {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    head = per[ws[HEADLINE].name]
    dec = per[ws[5].name]
    rec = {
        "metric": METRIC,
        "value": head["achieved"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": nw,
        "warmup_gpu_ms": round(warm_gpu_ms, 1),
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, all-zero prefill inputs" if args.zero_inputs else "synthetic",
        "config": {
            "workload": "long causal GQA prefill B1 Hq16 Hkv2 S16384 D256 (value); every step "
                        "also runs the tiny MHA, causal GQA S4096 D128, varlen window and paged "
                        "split-KV decode workloads (each under workloads)",
            "prefill_flops_per_launch": work[HEADLINE],
            "decode_bytes_per_launch": work[5],
        },
        "roofline": {
            "bound": "mfma", "achieved": head["achieved"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": head["frac"], "traffic": head["traffic"],
            "kernel": head["kernel"], "avg_launch_us": head["avg_launch_us"],
        },
        "cpu_baseline": cpu,
        "decode": {
            "value": dec["achieved"], "unit": "GB/s", "avg_launch_us": dec["avg_launch_us"],
            "roofline": {"bound": "hbm", "achieved": dec["achieved"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": dec["frac"], "traffic": dec["traffic"],
                         "kernel": dec["kernel"]},
        },
        "workloads": per,
    }
    if bwd is not None:
        rec["backward"] = bwd
    if extra:
        rec["other_workloads"] = extra
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
