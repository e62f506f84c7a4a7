#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

One step = one fa_fwd call (the whole hot path: validation, launch, GQA
packing, K/V streaming, QK^T, masking, online softmax, PV, epilogue, and the
split-KV merge where the shape takes that path) over one batch of seeded
synthetic inputs that are already resident in HBM.

After the W eager warm-up calls, the K steps are captured back to back in
one HIP graph, which is replayed untimed (its upload, then for at least
PREWARM_MS of GPU time, until the clock has settled under load) and then
replayed once between two synchronisations, so host launch cost is not
counted; the
time per step comes from HIP events recorded on the launch stream around
that replay, and ``value``, ``ms_per_step`` and ``roofline`` all use it
(the wall clock between the synchronisations is reported beside it).
HBM-bound workloads are priced against HBM with cold inputs (rotated over
copies larger than the MALL).  Prints one JSON line; progress goes to
stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd effective TFLOP/s (valid keys) + µs/call; % of MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
DEFAULT_WORKLOAD = "causal_gqa_prefill"  # the largest workload (most FLOPs and bytes)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["attention_forward_amd/csrc/fa_kernels.hip", "attention_forward_amd/csrc/fa_device.h",
                  "attention_forward_amd/csrc/fa_api.cpp",
                  "attention_forward_amd/csrc/fa_launch.h"]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(w):
    """Algorithmic FLOPs and HBM bytes of one call: 4*D per attended
    (query, key) pair; bytes = Q + valid K + valid V + out (bf16) + lse (fp32)."""
    n = w.valid_keys
    if w.causal:  # query i attends keys 0 .. i + n - Sq (the last query lines up with the last key)
        pairs = w.B * w.Hq * sum(max(0, min(i + 1 + n - w.Sq, n)) for i in range(w.Sq))
    else:
        pairs = w.B * w.Hq * w.Sq * n
    flops = 4 * w.D * pairs
    qo = w.B * w.Sq * w.Hq * w.D * 2
    kv = w.B * n * w.Hkv * w.D * 2
    lse = w.B * w.Hq * w.Sq * 4
    return flops, 2 * qo + 2 * kv + lse


def binding_roofline(flops, nbytes):
    """'mfma' when the arithmetic intensity is above the ridge point, else 'hbm'."""
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    return "mfma" if flops / nbytes > ridge else "hbm"


def roofline_entry(bound, flops, nbytes, sec_per_launch, traffic=None):
    if bound == "mfma":
        achieved = flops / sec_per_launch / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 5), "traffic": traffic}
    achieved = nbytes / sec_per_launch / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 5), "traffic": traffic}


def load_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_sha") != kernel_sha():
        return None
    return e.get("bytes_per_launch")


class Runner:
    """Device-resident inputs and preallocated outputs for one workload."""

    def __init__(self, w, device):
        import torch
        from attention_forward_amd import fa
        from attention_forward_amd.workloads import make_inputs

        self.w = w
        self.fa = fa
        q, k, v, s = make_inputs(w.name)
        self.q, self.k, self.v = (t.to(device) for t in (q, k, v))
        self.s = None if s is None else s.to(device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device=device)
        fa.reserve_workspace(self.q.device, fa.fa_fwd_workspace_bytes(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal))
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
                     self.lse.data_ptr(), w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, int(w.causal),
                     0 if self.s is None else self.s.data_ptr(), w.scale)

    def step(self, stream_handle):
        rc = self.fa.fa_fwd(*self.args, stream_handle)
        if rc != self.fa.FA_OK:
            raise self.fa.FAError(rc, "fa_fwd")


def capture(fn_launch, steps, warmup, device):
    """Run `warmup` eager launches, then capture `steps` launches in one graph
    (uploaded by one untimed replay)."""
    import torch

    indexed = getattr(fn_launch, "takes_index", False)  # fn(stream, i): launch i of the sequence

    def call(h, i):
        if indexed:
            fn_launch(h, i)
        else:
            fn_launch(h)

    stream = torch.cuda.Stream(device=device)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(stream.cuda_stream, i)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            call(torch.cuda.current_stream().cuda_stream, i)
    torch.cuda.synchronize()
    graph.replay()  # first replay uploads the graph; not timed
    torch.cuda.synchronize()
    return graph


def replay_timed(graph, device):
    """One replay between two synchronisations.  Returns (wall seconds,
    seconds between HIP events recorded around it on the replay stream)."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(device)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(cur)
    graph.replay()  # replays on the current stream
    e1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) * 1e-3


PREWARM_MS = 40.0  # untimed replays before a timed one: the GPU reaches its steady clock under load


def prewarm(graph, device, min_ms=PREWARM_MS):
    """Replay `graph` (untimed) until at least `min_ms` of GPU time has run.
    On MI355X the per-call time of a D256 call stays ~15 % above its steady
    value for the first several milliseconds of sustained load (measured:
    causal prefill 32.7 us/call timed over 20 calls right after start-up,
    31.7 over 200, 27.7 over 1000 and in every later timing), so a timed
    replay of a few calls is preceded by this much of the same work.
    Returns (replays, milliseconds)."""
    import torch

    done_ms, n = 0.0, 0
    while done_ms < min_ms:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream(device)
        e0.record(cur)
        graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        done_ms += e0.elapsed_time(e1)
        n += 1
    return n, done_ms


def time_graph(fn_launch, steps, warmup, device, stats=None):
    """Capture `steps` launches in one graph, replay it untimed for at least
    PREWARM_MS, then time one replay.  Returns (wall seconds between the two
    synchronisations, event seconds); `stats`, if a dict, receives the
    untimed replay count and time."""
    g = capture(fn_launch, steps, warmup, device)
    n, ms = prewarm(g, device)
    if stats is not None:
        stats.update({"untimed_replays": n, "untimed_ms": round(ms, 3)})
    return replay_timed(g, device)


def replay_stats(fn_launch, launches, replays, device):
    """p50 / p95 of the per-launch time over `replays` replays of a graph of
    `launches` back-to-back launches (microseconds)."""
    import statistics

    g = capture(fn_launch, launches, 3, device)
    per = sorted(replay_timed(g, device)[1] / launches * 1e6 for _ in range(replays))
    return {"p50": round(statistics.median(per), 3), "p95": round(per[min(len(per) - 1, int(0.95 * len(per)))], 3),
            "launches_per_replay": launches, "replays": replays}


COLD_BYTES = 600 << 20  # more than twice the 256 MiB last-level (MALL) cache


def cold_timing(w, device, replays=5):
    """Per-launch time with the inputs and outputs rotated over enough copies
    that every launch reads Q/K/V from HBM (the copies together exceed twice
    the MALL).  The copies hold the same seeded values; only their addresses
    differ.  Returns µs per launch (median over replays) and the set count."""
    import statistics
    import torch

    r = Runner(w, device)
    flops, nbytes = algorithmic(w)
    per_set = sum(t.numel() * t.element_size() for t in (r.q, r.k, r.v, r.out, r.lse))
    nsets = max(2, min(1024, -(-COLD_BYTES // per_set)))
    sets = []
    for _ in range(nsets):
        q, k, v = r.q.clone(), r.k.clone(), r.v.clone()
        out, lse = torch.empty_like(r.out), torch.empty_like(r.lse)
        sets.append((q, k, v, out, lse, (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
                     + r.args[5:]))
    fa = r.fa

    def launch(h, i):
        rc = fa.fa_fwd(*sets[i % nsets][5], h)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_fwd")
    launch.takes_index = True
    g = capture(launch, nsets, 0, device)
    per = [replay_timed(g, device)[1] / nsets for _ in range(replays)]
    us = statistics.median(per) * 1e6
    del sets, g
    torch.cuda.empty_cache()
    return {"us_per_call": round(us, 3), "sets": nsets, "set_bytes": per_set,
            "hbm_gbs": round(nbytes / us / 1e3, 2), "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 5),
            "tflops": round(flops / us / 1e6, 3)}


def clocks():
    """Current GPU clocks as reported by rocm-smi (text), or None."""
    import subprocess

    for cmd in (["rocm-smi", "--showclocks"], ["amd-smi", "metric", "--clock"]):
        try:
            res = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError):
            continue
        if res.returncode == 0 and res.stdout.strip():
            keep = [ln.strip() for ln in res.stdout.splitlines() if "clk" in ln.lower() or "mhz" in ln.lower()]
            return {"tool": cmd[0], "lines": keep[:16]}
    return None


def dispatch_floor_us(device, steps=200):
    """Per-launch time of a one-element fill kernel in the same graph setup."""
    import torch

    x = torch.zeros(1, device=device)
    _, ev = time_graph(lambda h: x.fill_(1.0), steps, 10, device)
    return ev / steps * 1e6


def _oracle_runs(w, threads, runs):
    """Wall seconds of `runs` calls of the fp64 oracle on workload w with the
    BLAS pool limited to `threads` (one untimed call first)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from attention_forward_amd.workloads import make_inputs
    from oracle import attention_ref

    q, k, v, s = make_inputs(w.name)
    q64, k64, v64 = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    sn = None if s is None else s.numpy()
    out = []
    with threadpool_limits(limits=threads, user_api="blas"):
        for i in range(runs + 1):
            t0 = time.perf_counter()
            attention_ref(q64, k64, v64, causal=w.causal, seqused_k=sn, scale=w.scale)
            if i:
                out.append(time.perf_counter() - t0)
    return out


def cpu_baseline(headline, workloads):
    """The fp64 oracle as it stands, timed on the host on each workload in
    full: with the BLAS pool at the affinity count and with one thread, one
    warm-up call and then the median of three.  The headline workload's
    all-cores figure is the reported baseline."""
    import statistics

    ncpu = os.cpu_count()
    aff = len(os.sched_getaffinity(0))
    table = {}
    for w in workloads:
        flops, _ = algorithmic(w)
        row = {}
        for label, th in (("all_cores", aff), ("one_thread", 1)):
            runs = _oracle_runs(w, th, 3)
            med = statistics.median(runs)
            row[label] = {"threads": th, "ms_median": round(med * 1e3, 3),
                          "ms_runs": [round(x * 1e3, 3) for x in runs], "gflops": round(flops / med / 1e9, 4)}
        table[w.name] = row
    h = table[headline.name]["all_cores"]
    one = table[headline.name]["one_thread"]
    return {"value": round(h["gflops"] / 1e3, 7), "unit": "TFLOP/s", "cores": aff, "kind": "oracle",
            "sample": f"the full {headline.name} workload, fp64 oracle, median of 3 after one warm-up call, "
                      f"BLAS threads = affinity count ({aff})",
            "ms_per_call": h["ms_median"], "one_thread_value": round(one["gflops"] / 1e3, 7),
            "one_thread_ms_per_call": one["ms_median"], "os_cpu_count": ncpu, "affinity_count": aff,
            "per_workload": table}


CALIB_BYTES = 256 << 20  # device-to-device copy used to calibrate the byte counters


STRIDED_ROWS = 1 << 17  # rows of the second calibration: one 144-byte head of a 16-head D72 row each


def traffic_probe(w, reps, device):
    """Eager calls of the workload plus two calibration kernels, for a
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE pass: a device-to-device copy of
    CALIB_BYTES (contiguous), and a negation that reads one 144-byte head row
    out of every 2304-byte row of a [rows, 16, 72] bf16 tensor (the D72
    head layout) into a contiguous tensor."""
    import torch

    r = Runner(w, device)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    heads = torch.ones(STRIDED_ROWS, 16, 72, dtype=torch.bfloat16, device=device)
    one_head = torch.empty(STRIDED_ROWS, 72, dtype=torch.bfloat16, device=device)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
        torch.neg(heads[:, 3, :], out=one_head)
        r.step(torch.cuda.current_stream(device).cuda_stream)
    torch.cuda.synchronize()


def ingest_traffic(workload, fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """HBM bytes per launch of the attention kernels from the counter CSVs
    of two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch).  Each counter is scaled by what it reads for the calibration
    copy of CALIB_BYTES (which moves exactly CALIB_BYTES each way)."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    out = {}
    strided = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        calib = max((statistics.median(v) for k, v in vals.items()
                     if ("copyBuffer" in k or "copy" in k.lower()) and "neg" not in k.lower()), default=None)
        if not calib:
            raise RuntimeError(f"no calibration copy found in {path}")
        factor = CALIB_BYTES / (calib * 1024.0)
        kb = sum(statistics.median(v) for k, v in vals.items() if "fa::" in k)
        out[counter] = {"kib_per_launch": kb, "calibration_kib": calib, "factor": factor,
                        "bytes_per_launch": kb * 1024.0 * factor}
        neg = [statistics.median(v) for k, v in vals.items() if "neg" in k.lower()]
        if neg:
            alg = STRIDED_ROWS * 144  # bytes read (FETCH) or written (WRITE) by the 144-byte-row negation
            strided[counter] = {"kib": neg[0], "bytes_scaled": neg[0] * 1024.0 * factor,
                                "algorithmic_bytes": alg, "ratio": neg[0] * 1024.0 * factor / alg}
    entry = {"kernel_sha": kernel_sha(), "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
             "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
             "strided_144B_calibration": strided or None}
    try:
        with open(out_path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = entry
    with open(out_path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    return entry


def extension_rows(device, steps=200):
    """µs per call of the extended entry points on shapes taken from the
    workloads: fp16, a fused QKV buffer read in place, a packed
    variable-length batch, a causal chunk of new positions attending a cache,
    causal decode over the padded prefix cache, and the NVFP4 output."""
    import torch
    from attention_forward_amd import fa
    from attention_forward_amd.workloads import make_custom

    rows = {}

    def record(name, launch, flops, nbytes):
        _, ev = time_graph(launch, steps, 5, device)
        s = ev / steps
        rows[name] = {"us_per_call": round(s * 1e6, 3), "tflops": round(flops / s / 1e12, 3),
                      "gbs": round(nbytes / s / 1e9, 2)}

    def pairs_causal(sq, n, h):
        return h * sum(max(0, min(i + 1 + n - sq, n)) for i in range(sq))

    B, S, H, D = 3, 256, 16, 72
    vit_flops, vit_bytes = 4 * D * B * H * S * S, 4 * B * S * H * D * 2 + B * H * S * 4
    # fp16 ViT (contiguous, through fa_fwd_strided)
    q, k, v, _ = make_custom(B, S, S, H, H, D, seed=2, dtype=torch.float16)
    q, k, v = (t.to(device) for t in (q, k, v))
    out, lse = torch.empty_like(q), torch.empty(B, H, S, dtype=torch.float32, device=device)
    st = (S * H * D, H * D, D)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, S, S, H, H, D, st, st, st,
            st, fa.FA_FP16, 0, 0, 1.0 / math.sqrt(D))
    record("vit_multiview_fp16", lambda h, a=args: fa.fa_fwd_strided(*a, h), vit_flops, vit_bytes)
    # ViT read from a fused [B, S, 3H, D] QKV buffer (bf16 views)
    qkv = torch.randn(B, S, 3 * H, D, device=device).to(torch.bfloat16)
    out = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=device)
    fs = (S * 3 * H * D, 3 * H * D, D)
    base = qkv.data_ptr()
    args = (base, base + H * D * 2, base + 2 * H * D * 2, out.data_ptr(), lse.data_ptr(), B, S, S, H, H, D, fs, fs,
            fs, st, fa.FA_BF16, 0, 0, 1.0 / math.sqrt(D))
    record("vit_multiview_fused_qkv", lambda h, a=args: fa.fa_fwd_strided(*a, h), vit_flops, vit_bytes)
    # ViT as a packed variable-length batch of three 256-token views
    qp, kp, vp = (torch.randn(B * S, H, D, device=device).to(torch.bfloat16) for _ in range(3))
    outp, lsep = torch.empty_like(qp), torch.empty(H, B * S, dtype=torch.float32, device=device)
    cu = torch.tensor([0, S, 2 * S, 3 * S], dtype=torch.int32, device=device)
    args = (qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), outp.data_ptr(), lsep.data_ptr(), cu.data_ptr(),
            cu.data_ptr(), B, S, S, B * S, B * S, H, H, D, fa.FA_BF16, 0, 1.0 / math.sqrt(D))
    record("vit_multiview_varlen", lambda h, a=args: fa.fa_fwd_varlen(*a, h), vit_flops, vit_bytes)
    # causal chunk: 64 new positions (8 query heads, 1 K/V head, D256) attending a 1024-key cache
    Sq, Sk, Hq, Dd = 64, 1024, 8, 256
    q, k, v, _ = make_custom(1, Sq, Sk, Hq, 1, Dd, seed=3)
    q, k, v = (t.to(device) for t in (q, k, v))
    out, lse = torch.empty_like(q), torch.empty(1, Hq, Sq, dtype=torch.float32, device=device)
    fa.reserve_workspace(q.device, fa.fa_fwd_workspace_bytes(1, Sq, Sk, Hq, 1, Dd, 1))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), 1, Sq, Sk, Hq, 1, Dd, 1, 0,
            0.0625)
    record("causal_chunk_64x1024_gqa", lambda h, a=args: fa.fa_fwd(*a, h), 4 * Dd * pairs_causal(Sq, Sk, Hq),
           (2 * Sq * Hq + 2 * Sk) * Dd * 2 + Hq * Sq * 4)
    # causal decode: one new position over the padded 1056-key prefix cache (1009 valid keys)
    Sq, Sk, n = 1, 1056, 1009
    q, k, v, sq = make_custom(1, Sq, Sk, Hq, 1, Dd, seed=4, n_valid=n)
    q, k, v, sq = (t.to(device) for t in (q, k, v, sq))
    out, lse = torch.empty_like(q), torch.empty(1, Hq, Sq, dtype=torch.float32, device=device)
    fa.reserve_workspace(q.device, fa.fa_fwd_workspace_bytes(1, Sq, Sk, Hq, 1, Dd, 1))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), 1, Sq, Sk, Hq, 1, Dd, 1,
            sq.data_ptr(), 0.0625)
    record("causal_decode_1x1009_gqa", lambda h, a=args: fa.fa_fwd(*a, h), 4 * Dd * Hq * n,
           (2 * Sq * Hq + 2 * n) * Dd * 2 + Hq * Sq * 4)
    # NVFP4 output (fa_fwd_nvfp4) on the two D256 GQA workloads: the output is
    # D/2 code bytes and D/16 scale bytes per row instead of 2D
    from attention_forward_amd.workloads import WORKLOADS, make_inputs
    for name in ("prefix_gqa_padded", "action_expert_small_m"):
        w = WORKLOADS[name]
        q, k, v, sq = (t.to(device) if t is not None else None for t in make_inputs(name))
        codes = torch.empty(w.B, w.Sq, w.Hq, w.D // 2, dtype=torch.uint8, device=device)
        sf = torch.empty(w.B, w.Sq, w.Hq, w.D // 16, dtype=torch.uint8, device=device)
        lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device=device)
        fa.reserve_workspace(q.device, fa.fa_fwd_workspace_bytes(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D, w.causal))
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), codes.data_ptr(), sf.data_ptr(), lse.data_ptr(), w.B, w.Sq,
                w.Sk, w.Hq, w.Hkv, w.D, int(w.causal), 0 if sq is None else sq.data_ptr(), w.scale)
        flops, nbytes = algorithmic(w)
        rows_q = w.B * w.Sq * w.Hq
        record(f"{name}_nvfp4", lambda h, a=args: fa.fa_fwd_nvfp4(*a, h), flops,
               nbytes - rows_q * w.D * 2 + rows_q * (w.D // 2 + w.D // 16))
    return rows


def intake_probe():
    """Run the intake probe built next to the library (attention_forward_amd/intake_probe) as a child
    process and print its JSON line."""
    import subprocess

    exe = os.path.join(ROOT, "attention_forward_amd", "intake_probe")
    if not os.path.exists(exe):
        print(f"{exe} is missing: run the build step first", file=sys.stderr)
        return 1
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    sys.stdout.write(res.stdout)
    sys.stderr.write(res.stderr)
    return res.returncode


def _progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def measure(w, steps, warmup, device, stats=None):
    r = Runner(w, device)
    wall, ev = time_graph(r.step, steps, warmup, device, stats)
    flops, nbytes = algorithmic(w)
    return r, wall, ev, flops, nbytes


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all", action="store_true", help="skip the per-workload table")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the replay statistics and the cold-cache timing (for profiler runs)")
    ap.add_argument("--traffic-probe", type=int, default=0, metavar="REPS",
                    help="only run REPS eager calls plus a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--intake-probe", action="store_true",
                    help="only run the compute-unit intake probe (bytes per clock from L2) and print its JSON")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs into profiles/traffic.json and exit")
    a = ap.parse_args(argv)
    if a.ingest_traffic:
        print(json.dumps(ingest_traffic(a.workload, *a.ingest_traffic)))
        return 0
    if a.intake_probe:
        return intake_probe()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported (this library has no "
              "multi-GPU path; run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    from attention_forward_amd.workloads import WORKLOADS, WORKLOAD_ORDER

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    device = torch.device("cuda:0")
    w = WORKLOADS[a.workload]
    if a.traffic_probe:
        traffic_probe(w, a.traffic_probe, device)
        print(f"traffic probe done: {w.name} x{a.traffic_probe}", flush=True)
        return 0
    pre = {}
    r, wall, ev, flops, nbytes = measure(w, a.steps, a.warmup, device, pre)
    _progress(f"timed {a.steps} steps of {w.name}")
    # value, ms_per_step and the roofline all come from one timing: HIP
    # events on the launch stream around the replay of the K captured steps
    sec_launch = ev / a.steps
    bound = binding_roofline(flops, nbytes)
    traffic = load_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(flops / sec_launch / 1e12, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(sec_launch * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Sq": w.Sq, "Sk": w.Sk, "seqused_k": w.n_valid,
                   "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "causal": w.causal, "parallelism": "none (1 GPU)"},
        "us_per_call": round(sec_launch * 1e6, 3),
        "wall_ms_per_step": round(wall / a.steps * 1e3, 6),
        # before the timed replay: the W eager warm-up calls, the graph's
        # upload replay, and untimed replays of the same graph for at least
        # PREWARM_MS (the GPU's clock settles under sustained load)
        "untimed_before": {"eager_calls": a.warmup, "graph_upload_replays": 1, **pre},
        "algorithmic": {"flops_per_call": flops, "bytes_per_call": nbytes},
        "kernel_sha": kernel_sha(),
        "device": torch.cuda.get_device_name(device),
    }
    if bound == "hbm" and not a.no_extra:
        # an HBM-bound call is priced with its inputs coming from HBM
        cold = cold_timing(w, device)
        line["cold"] = cold
        line["roofline"] = roofline_entry(bound, flops, nbytes, cold["us_per_call"] * 1e-6, traffic)
        line["roofline"]["timing"] = "cold (inputs rotated past the MALL)"
    else:
        line["roofline"] = roofline_entry(bound, flops, nbytes, sec_launch, traffic)
        line["roofline"]["timing"] = "warm (back-to-back calls of one input set)"
    line["dispatch_floor_us"] = round(dispatch_floor_us(device), 3)
    if not a.no_extra:
        line["replay_stats_us"] = replay_stats(r.step, 100, 20, device)
    _progress("headline done")
    if not a.no_all:
        table = {}
        for name in WORKLOAD_ORDER:
            wx = WORKLOADS[name]
            steps = max(50, min(a.steps, 400))
            rx, wl, evx, fx, bx = measure(wx, steps, 5, device)
            s = evx / steps
            bnd = binding_roofline(fx, bx)
            st = replay_stats(rx.step, 100, 20, device)
            row = {"us_per_call": round(s * 1e6, 3), "p50": st["p50"], "p95": st["p95"],
                   "tflops": round(fx / s / 1e12, 3), "bound": bnd,
                   "plan": list(rx.fa.fa_fwd_plan(wx.B, wx.Sq, wx.Sk, wx.Hq, wx.Hkv, wx.D, int(wx.causal)))}
            if bnd == "hbm" and name != "single_head":
                row["cold"] = cold_timing(wx, device)
                re = roofline_entry(bnd, fx, bx, row["cold"]["us_per_call"] * 1e-6)
                row["timing"] = "cold"
            else:
                re = roofline_entry(bnd, fx, bx, s)
                row["timing"] = "warm"
            row.update({"frac": re["frac"], "achieved": re["achieved"], "unit": re["unit"]})
            table[name] = row
            _progress(f"all_workloads: {name} {row['us_per_call']} us")
        line["all_workloads"] = table
        line["extensions"] = extension_rows(device)
        _progress("extensions done")
    line["clocks"] = clocks()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, [WORKLOADS[n] for n in WORKLOAD_ORDER] if not a.no_all else [w])
        _progress("cpu baseline done")
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
