#!/usr/bin/env python3
"""Benchmark of the fused exact-attention forward on one MI355X.

A step is one forward call (attn_fwd, or attn_fwd_gqa for grouped-query and
cross-attention shapes; their split-key forms when the shape has too few
work items to fill the GPU) over one batch of seeded synthetic inputs that
are already resident in device memory.  The launches cycle through several
copies of the inputs, enough that each launch reads them from HBM rather
than from the last-level cache.  The K timed steps are recorded into one HIP
graph and replayed, so no host time separates the launches; the graph is
replayed untimed for at least --warmup-seconds first, so that the clocks
have settled, and again after the timed replay for a median and a minimum
per launch.  The default workload is the causal decoder prefill B=1 H=32
N=4096 d=128 fp16 (scale 1/sqrt(128)), the configuration whose throughput
is reported as TFLOP/s and as a fraction of the dense fp16 matrix-core peak;
the other four configurations are measured in the same run under
``configs``.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--no-naive] [--no-graph] [--no-rotate] [--no-configs]
                  [--splitkv auto|on|off] [--kv-splits S]
  python bench.py --copy-probe       # a plain device copy of known size, for
                                     # scaling rocprofv3 FETCH_SIZE/WRITE_SIZE
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (4·B·H·N²·d, causal ×½) + % of MI355X MFMA peak"
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense matrix-core peak
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "exact_self_attention_amd", "csrc", f)
                  for f in ("cdna4.h", "dispatch.cpp", "fwd_body.h", "fwd_decode.hip", "fwd_deep.hip",
                            "fwd_fused.hip", "fwd_masked.hip", "fwd_short.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
COPY_PROBE_BYTES = 1 << 30
# dense fp16/bf16 matrix-core flops per clock per compute unit: four SIMDs,
# each finishing a 32x32x16 MFMA (32768 flops) every 32 clocks
MFMA_FLOPS_PER_CLK_CU = 4096
HIP_ATTR_CLOCK_RATE = 5   # hipDeviceAttributeClockRate (peak clock, kHz)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up until this much wall time has passed")
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU seconds of the oracle sample")
    ap.add_argument("--splitkv", choices=["auto", "on", "off"], default="auto",
                    help="time the split-key entry point: auto = when the library's "
                         "default split count for the shape is above 1")
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="split count for the split-key entry point instead of the default")
    ap.add_argument("--no-graph", action="store_true",
                    help="time K plain launches instead of one replay of a graph of K launches")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip timing the unfused attn_fwd_naive baseline")
    ap.add_argument("--no-rotate", action="store_true",
                    help="time every launch on one input set (warm caches) instead of "
                         "rotating through enough copies that each launch reads from HBM")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip measuring the other configurations in the same run")
    ap.add_argument("--stats-seconds", type=float, default=0.25,
                    help="GPU time of the extra timed repeats behind the median and minimum")
    ap.add_argument("--copy-probe", action="store_true")
    return ap.parse_args()


def key_lengths(w, key_len=None) -> np.ndarray:
    """Valid keys per sequence, clamped to [0, N]."""
    if key_len is None:
        return np.full(w.B, w.N, dtype=np.int64)
    return np.clip(np.asarray(key_len, np.int64), 0, w.N)


def visible_per_query(w, L: int) -> np.ndarray:
    """Visible keys of each query row of a sequence with L valid keys: under
    causal masking query i sees keys j <= i + N - Nq (aligned at the end)."""
    i = np.arange(w.q_len, dtype=np.int64)
    if not w.causal:
        return np.full(w.q_len, L, dtype=np.int64)
    return np.clip(np.minimum(L, i + w.N - w.q_len + 1), 0, None)


def visible_pairs(w, key_len=None) -> int:
    """Visible (query, key) pairs: the algorithmic unit of work (4d flops each)."""
    return int(sum(int(visible_per_query(w, int(L)).sum()) * w.H for L in key_lengths(w, key_len)))


def metric_flops(w) -> float:
    """The metric's FLOP count: 4 B H N^2 d, halved when causal, for
    self-attention; 4 d per visible (query, key) pair for the other shapes."""
    if w.general:
        return 4.0 * w.d * visible_pairs(w, None)
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2 if w.causal else f


def algorithmic_bytes(w, key_len=None) -> int:
    """Q and O once, each key/value head's visible K and V rows once, LSE once
    (4 B per query row), and a shared additive mask's elements that some
    query sees once (4 B each)."""
    elem = 2
    qo = 2 * w.B * w.H * w.q_len * w.d * elem
    kv = 0
    for L in key_lengths(w, key_len):
        seen = int(visible_per_query(w, int(L)).max()) if w.q_len > 0 else 0
        kv += 2 * w.kv_heads * seen * w.d * elem
    mask = 0
    if w.mask_sigma is not None:  # one [Nq, N] mask shared by all (b, h)
        mask = 4 * int(visible_per_query(w, int(key_lengths(w, key_len).max())).sum())
    return qo + kv + w.B * w.H * w.q_len * 4 + mask


def code_only(text: str) -> str:
    """A C/C++ source without its comments, trailing blanks and empty lines
    (string and character literals kept), so that a change to comments
    alone leaves the digest below as it was."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def source_digest() -> str:
    """sha256 (first 16 hex digits) of the fused-kernel sources' code (no
    comments), file after file."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = source_digest()
    for line in open(TRAFFIC_FILE):
        m = re.match(r"\s*traffic\s+(.*)$", line)
        if not m:
            continue
        kv = dict(x.split("=", 1) for x in m.group(1).split())
        if kv.get("kernel") == kernel and kv.get("workload") == workload \
                and kv.get("source_sha256_16") == digest:
            return int(float(kv["hbm_bytes_per_launch"]))
    return None


def copy_probe():
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES,
                      "copy_probe_bytes_written": COPY_PROBE_BYTES, "launches": 5}))


def device_mfma_peak(torch):
    """The matrix-core peak of the device in this process from its compute
    units and peak clock (hipDeviceGetAttribute), beside the nominal figure;
    None where the runtime cannot be asked."""
    import ctypes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = None
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            hip = ctypes.CDLL(name)
        except OSError:
            continue
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_CLOCK_RATE, 0) == 0 \
                and 1e5 <= v.value <= 1e7:
            khz = v.value
            break
    if khz is None:
        return {"cus": cus, "clock_mhz": None, "tflops": None}
    return {"cus": cus, "clock_mhz": khz / 1e3,
            "tflops": cus * khz * 1e3 * MFMA_FLOPS_PER_CLK_CU / 1e12}


def copy_roof(torch):
    """The practical memory roof in this run: a 1 GiB device-to-device copy
    (bytes read + written over the median of 10 timed copies)."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(10)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    secs = float(np.median([a.elapsed_time(b) / 1e3 for a, b in evs]))
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": 2 * COPY_PROBE_BYTES / secs / 1e9, "bytes_read": COPY_PROBE_BYTES,
            "bytes_written": COPY_PROBE_BYTES, "kind": "torch copy_, median of 10"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def naive_baseline(attn, torch, w, q, k, v, kl, scale, stream, F):
    """Time the unfused attn_fwd_naive (scores and probabilities through HBM)
    on the same inputs; its workspace holds at most 8 GiB of heads at once."""
    per_head = attn.attn_fwd_naive_workspace_bytes(1, 1, w.N)
    heads = max(1, min(w.B * w.H, (8 << 30) // per_head))
    ws = torch.empty(heads * per_head // 4, dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)

    def run():
        attn.attn_fwd_naive(q, k, v, o, lse, workspace=ws, scale=scale, causal=w.causal,
                            key_len=kl, stream=stream)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    once = time.perf_counter() - t0
    reps = int(max(1, min(50, 1.0 / max(once, 1e-6))))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    secs = ev0.elapsed_time(ev1) / 1e3 / reps
    del ws
    return {"value": F / secs / 1e12, "unit": "TFLOP/s", "ms_per_step": secs * 1e3,
            "steps": reps, "kind": "attn_fwd_naive",
            "workspace_heads_per_launch": heads}


def cpu_baseline(w, case, target_s: float):
    """Time the fp64 oracle on a bounded sample of the workload's query rows."""
    import attn_inputs as ai
    import oracle
    dt = case["dtype"]
    Q = ai.bits_to_f32(case["Q"], dt)
    K = ai.bits_to_f32(case["K"], dt)
    V = ai.bits_to_f32(case["V"], dt)
    kl = case["key_len"]
    Ls = key_lengths(w, kl)
    vis = {int(L): visible_per_query(w, int(L)) for L in set(Ls.tolist())}
    rng = np.random.Generator(np.random.PCG64(w.seed + 31))

    def rows_flops(sel):
        return sum(4 * w.d * int(vis[int(Ls[b])][i]) for b, h, i in sel)

    def pick(per_head):
        out = []
        for b in range(w.B):
            for h in range(w.H):
                for i in rng.choice(w.q_len, size=per_head, replace=False):
                    out.append((b, h, int(i)))
        return np.asarray(out, np.int64)

    sel = pick(min(2, w.q_len))
    t0 = time.perf_counter()
    oracle.attn_rows(Q, K, V, float(case["scale"]), w.causal, kl, sel, mask=case.get("mask"))
    rate = rows_flops(sel) / max(time.perf_counter() - t0, 1e-6)
    per_row = max(1.0, 4 * w.d * float(np.mean([v.mean() for v in vis.values()])))
    per_head = int(max(1, min(w.q_len, target_s * rate / per_row / (w.B * w.H))))
    sel = pick(per_head)
    flops = rows_flops(sel)
    t0 = time.perf_counter()
    oracle.attn_rows(Q, K, V, float(case["scale"]), w.causal, kl, sel, mask=case.get("mask"))
    secs = time.perf_counter() - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{per_head} seeded random query rows per (b,h) of all {w.B * w.H} heads, "
                      f"each over its full visible key range; {flops:.3e} flops in {secs:.1f} s"}


# Input sets cycled through by the timed launches: enough that, between two
# uses of a set, the other sets have moved more bytes than the 256 MB
# last-level cache (MALL) and the L2s hold, so every launch reads its inputs
# from HBM; at least 16 for the small shapes, and at most 4096 (for sets
# under 128 KB, such as the 64-row single head, the other sets then move
# less than the MALL holds and a launch may read its inputs from there).
ROTATE_EVICT_BYTES = 512 << 20
ROTATE_MIN_SETS_SMALL = 16
ROTATE_SMALL_SET_BYTES = 64 << 20
ROTATE_MAX_SETS = 4096


def input_sets(set_bytes: int) -> int:
    n = 1 + -(-ROTATE_EVICT_BYTES // max(set_bytes, 1))
    if set_bytes <= ROTATE_SMALL_SET_BYTES:
        n = max(n, ROTATE_MIN_SETS_SMALL)
    return int(min(n, ROTATE_MAX_SETS))


class Runner:
    """One workload on the device: R copies of its inputs and outputs and a
    step function that launches the chosen entry point on copy i."""

    def __init__(self, attn, torch, w, case, splitkv="auto", kv_splits=0, rotate=True):
        import attn_inputs as ai
        self.attn, self.torch, self.w, self.case = attn, torch, w, case
        dev = torch.device("cuda:0")
        self.dev = dev
        tdt = torch.float16 if w.dtype == ai.F16 else torch.bfloat16

        def to_dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

        q, k, v = to_dev(case["Q"]), to_dev(case["K"]), to_dev(case["V"])
        self.kl = None if case["key_len"] is None else torch.from_numpy(case["key_len"]).to(dev)
        self.scale = float(w.scale)
        self.code = attn.ATTN_F16 if w.dtype == ai.F16 else attn.ATTN_BF16
        default_splits = attn.attn_fwd_gqa_splitkv_default_splits(
            self.code, w.B, w.H, w.kv_heads, w.q_len, w.N, w.d, w.causal)
        use_split = splitkv == "on" or (splitkv == "auto" and (kv_splits > 1 or default_splits > 1))
        self.n_splits = None
        self.ws = None
        if use_split:
            self.n_splits = kv_splits if kv_splits > 0 else default_splits
            self.ws = torch.empty(attn.attn_fwd_splitkv_workspace_bytes(
                w.B, w.H, w.q_len, w.d, self.n_splits) // 4, dtype=torch.float32, device=dev)
        self.mask = None
        if w.mask_sigma is not None:
            self.mask = torch.from_numpy(case["mask"]).to(dev)
            self.entry = "attn_fwd_masked_splitkv" if use_split else "attn_fwd_masked"
        elif w.general:
            self.entry = "attn_fwd_gqa_splitkv" if use_split else "attn_fwd_gqa"
        else:
            self.entry = "attn_fwd_splitkv" if use_split else "attn_fwd"
        set_bytes = 2 * (q.numel() + k.numel() + v.numel() + q.numel()) + 4 * q.numel() // w.d
        self.n_sets = input_sets(set_bytes) if rotate else 1
        self.sets = []
        for i in range(self.n_sets):
            qi, ki, vi = (q, k, v) if i == 0 else (q.clone(), k.clone(), v.clone())
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            self.sets.append((qi, ki, vi, o, lse))
        self.kernel = attn.attn_fwd_gqa_kernel_name(self.code, w.d, w.H, w.kv_heads, w.q_len, w.N,
                                                    w.causal, self.mask is not None,
                                                    self.n_splits or 0)

    def step(self, i=0):
        """Launch on the current stream (the capture stream while a graph records)."""
        attn, w = self.attn, self.w
        q, k, v, o, lse = self.sets[i % self.n_sets]
        kl, scale, ws, S = self.kl, self.scale, self.ws, self.n_splits
        e = self.entry
        if e == "attn_fwd_splitkv":
            attn.attn_fwd_splitkv(q, k, v, o, lse, workspace=ws, n_splits=S, scale=scale,
                                  causal=w.causal, key_len=kl)
        elif e == "attn_fwd_gqa_splitkv":
            attn.attn_fwd_gqa_splitkv(q, k, v, o, lse, workspace=ws, n_splits=S, scale=scale,
                                      causal=w.causal, key_len=kl)
        elif e == "attn_fwd_gqa":
            attn.attn_fwd_gqa(q, k, v, o, lse, scale=scale, causal=w.causal, key_len=kl)
        elif e == "attn_fwd_masked":
            attn.attn_fwd_masked(q, k, v, o, lse, mask=self.mask, scale=scale, causal=w.causal,
                                 key_len=kl)
        elif e == "attn_fwd_masked_splitkv":
            attn.attn_fwd_masked_splitkv(q, k, v, o, lse, mask=self.mask, workspace=ws,
                                         n_splits=S, scale=scale, causal=w.causal, key_len=kl)
        else:
            attn.attn_fwd(q, k, v, o, lse, scale=scale, causal=w.causal, key_len=kl)

    def timed(self, steps, warmup, warmup_seconds, stats_seconds, graph=True):
        """W untimed steps and at least warmup_seconds of back-to-back GPU work,
        then exactly ``steps`` launches timed (wall clock between two device
        synchronisations, HIP events on the stream around them), then more
        timed repeats of the same launches for the median and minimum.  With
        ``graph`` the launches are recorded once into a HIP graph and
        replayed, so no host time separates them."""
        torch = self.torch
        stream = torch.cuda.current_stream(self.dev)
        g = None
        if graph:
            # capture after a first launch of each set (library state, if any,
            # is initialised outside the capture)
            for i in range(min(self.n_sets, steps)):
                self.step(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    self.step(i)
            torch.cuda.synchronize()

        def run():
            if g is not None:
                g.replay()
            else:
                for i in range(steps):
                    self.step(i)

        # warmup: one replay stays queued behind the one the host waits for,
        # so the GPU does not idle between them
        t_w = time.perf_counter()
        n_warm = 0
        prev = None
        while n_warm < warmup or time.perf_counter() - t_w < warmup_seconds:
            run()
            n_warm += steps
            e = torch.cuda.Event()
            e.record(stream)
            if prev is not None:
                prev.synchronize()
            prev = e
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        run()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch_s = ev0.elapsed_time(ev1) / 1e3 / steps
        # repeats for the median and minimum, queued back to back
        n_rep = int(min(500, max(5, stats_seconds / max(launch_s * steps, 1e-7))))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_rep)]
        for a, b in evs:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        reps = [a.elapsed_time(b) / 1e3 / steps for a, b in evs]
        return {"wall_s": wall, "launch_s": launch_s, "warmup_steps_run": n_warm,
                "median_launch_s": float(np.median(reps)), "min_launch_s": float(np.min(reps)),
                "repeats": n_rep}


def roofline(w, key_len, launch_s):
    """The bound and the achieved fraction of it: HBM when the flops per
    algorithmic byte are below the machine balance (matrix-core peak / HBM
    bandwidth), else the matrix cores."""
    pairs = visible_pairs(w, key_len)
    F_alg = 4.0 * w.d * pairs
    nbytes = algorithmic_bytes(w, key_len)
    if F_alg / nbytes < MFMA_PEAK_TFLOPS[w.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = nbytes / launch_s / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}
    achieved = F_alg / launch_s / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    return {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "algorithmic_flops": F_alg}


def config_entry(w, r, t, device_peak=None):
    roof = roofline(w, r.case["key_len"], t["launch_s"])
    achieved_med = roof["achieved"] * t["launch_s"] / t["median_launch_s"]
    out = {"kernel": r.kernel, "entry": r.entry, "bound": roof["bound"], "unit": roof["unit"],
           "achieved": roof["achieved"], "frac": roof["frac"],
           "frac_median": achieved_med / roof["peak"],
           "avg_launch_us": t["launch_s"] * 1e6, "median_launch_us": t["median_launch_s"] * 1e6,
           "min_launch_us": t["min_launch_s"] * 1e6, "input_sets": r.n_sets}
    if roof["bound"] == "mfma" and device_peak:
        out["frac_device_peak"] = roof["achieved"] / device_peak
    if roof["bound"] == "hbm":
        # beside the algorithmic bytes: the bytes with every padded key row
        # read, and the flops of the visible pairs per second
        F_alg = 4.0 * w.d * visible_pairs(w, r.case["key_len"])
        out["algorithmic_bytes"] = roof["algorithmic_bytes"]
        out["dense_bytes"] = algorithmic_bytes(w, None)
        out["tflops_alg"] = F_alg / t["launch_s"] / 1e12
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); attention heads "
              "shard across GPUs without any exchange, so the multi-GPU figure is N "
              "times this one-GPU throughput and is not measured here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import torch
    import attn_inputs as ai
    import exact_self_attention_amd as attn

    w = ai.WORKLOADS[args.workload]
    case = ai.generate(w)
    r = Runner(attn, torch, w, case, args.splitkv, args.kv_splits, rotate=not args.no_rotate)
    t = r.timed(args.steps, args.warmup, args.warmup_seconds, args.stats_seconds,
                graph=not args.no_graph)
    ms_per_step = t["wall_s"] * 1e3 / args.steps
    launch_s = t["launch_s"]

    F = metric_flops(w)
    roof = roofline(w, case["key_len"], launch_s)
    roof.pop("algorithmic_bytes", None)
    roof.pop("algorithmic_flops", None)
    roof["traffic"] = read_traffic(r.kernel, w.name)
    dev_peak = device_mfma_peak(torch)
    if roof["bound"] == "mfma":
        # the same against CUs x peak clock x 4096 flops/clock of this device
        roof["peak_device"] = dev_peak["tflops"]
        roof["frac_device_peak"] = (roof["achieved"] / dev_peak["tflops"]
                                    if dev_peak["tflops"] else None)
        roof["device"] = {"cus": dev_peak["cus"], "clock_mhz": dev_peak["clock_mhz"]}
    roof["kernel"] = r.kernel
    roof["avg_launch_us"] = launch_s * 1e6
    roof["median_launch_us"] = t["median_launch_s"] * 1e6
    roof["min_launch_us"] = t["min_launch_s"] * 1e6

    value = F / (ms_per_step / 1e3) / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": t["warmup_steps_run"],
        "launch": "plain" if args.no_graph else "hip_graph",
        "entry": r.entry, "input_sets": r.n_sets,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "Hkv": w.kv_heads, "Nq": w.q_len,
                   "mask": None if r.mask is None else f"fp32 [{w.q_len}, {w.N}] shared, N(0, {w.mask_sigma}^2)",
                   "causal": w.causal, "key_padding": w.key_padding, "seed": w.seed,
                   "kv_splits": r.n_splits,
                   "global_batch": w.B, "seq_len": w.N},
        "pct_mfma_peak": 100.0 * value / MFMA_PEAK_TFLOPS[w.dtype],
        "roofline": roof,
    }
    # the unfused baseline takes self-attention shapes without a mask only
    if not args.no_naive and not w.general and r.mask is None:
        stream = torch.cuda.current_stream(r.dev)
        q, k, v = r.sets[0][:3]
        nb = naive_baseline(attn, torch, w, q, k, v, r.kl, r.scale, stream, F)
        nb["fused_speedup"] = nb["ms_per_step"] / ms_per_step
        out["naive_baseline"] = nb
    # the practical memory roof on this machine, for the bandwidth-bound shapes
    out["copy_roof"] = copy_roof(torch)
    if not args.no_configs:
        # every configuration of the scope, measured in this run the same way
        # (the headline's own entry is the measurement above)
        configs = {}
        for name in ai.WORKLOAD_ORDER:
            if name == w.name:
                configs[name] = config_entry(w, r, t, dev_peak["tflops"])
                continue
            wc = ai.WORKLOADS[name]
            rc = Runner(attn, torch, wc, ai.generate(wc), rotate=not args.no_rotate)
            # at least 20 launches per replay, and enough that a replay is
            # >= 2 ms of work
            t_est = rc.timed(8, 0, 0.05, 0.0, graph=False)["median_launch_s"]
            n = int(min(2000, max(20, np.ceil(2e-3 / max(t_est, 1e-7)))))
            tc = rc.timed(n, 0, args.warmup_seconds, args.stats_seconds, graph=not args.no_graph)
            configs[name] = config_entry(wc, rc, tc, dev_peak["tflops"])
            configs[name]["steps"] = n
            if configs[name]["bound"] == "hbm" and rc.n_sets > 1:
                # labelled warm-cache figure: every launch on one input set
                del rc
                torch.cuda.empty_cache()
                rc = Runner(attn, torch, wc, ai.generate(wc), rotate=False)
                tw = rc.timed(n, 0, args.warmup_seconds, args.stats_seconds,
                              graph=not args.no_graph)
                configs[name]["warm_avg_launch_us"] = tw["launch_s"] * 1e6
                configs[name]["warm_median_launch_us"] = tw["median_launch_s"] * 1e6
            del rc
            torch.cuda.empty_cache()
        out["configs"] = configs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, case, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
