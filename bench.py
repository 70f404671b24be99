"""Benchmark of the MXFP4 GEMM path on one MI355X.

One call = mx_gemm: activation quantisation + block-scaled MFMA contraction
(+ split-K reduction when planned) + bf16 epilogue; the weight is packed once
beforehand.  A step is a batch of CALLS_PER_STEP calls over distinct buffer
copies.  The headline workload is M=256, N=3072, K=1536, the largest of the
five (the MFMA-heaviest); the other four are reported per workload.  Inputs
are seeded N(0,1) bf16 (synthetic stand-ins for the leaderboard's data),
resident in HBM; calls rotate over enough copies of A, the packed weight, C
and the workspace that the working set (>= 512 MiB) cannot sit in the
256 MB Infinity Cache ("cold"), or reuse one set ("hot").

Printed: one JSON line.  `value` is the end-to-end host wall clock per call
of back-to-back eager calls (host launch cost included).  The roofline and
MFMA figures use the GPU time per call with the host out of the loop: the
calls captured into a HIP graph and replayed, HIP events on the replay
stream, which covers every launch of a call (two at 256x3072x1536: the
activation quantiser and the GEMM).  Beside them: the oracle timed on the
host cores (cpu_baseline), what a near-empty kernel and a kernel that only
streams the same weight bytes with the GEMM's own grid cost (reference
floors), the same figures for the other workloads (per_workload), and the
GPU time and fp4 MFMA rate of four large-M shapes, where the contraction
bounds the call (large_m).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA, published
HEADLINE = 4                   # index of M=256, N=3072, K=1536 in inputs.WORKLOADS
CALLS_PER_STEP = 100           # one bench step = this many mx_gemm calls
COLD_BYTES = 512 << 20         # working set of the rotating copies
MAX_COPIES = 1000


def algorithmic_bytes(M, N, K):
    """A bf16 in + packed B (codes + e8m0) + C bf16 out."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


def kernel_source_hash():
    """Hash of the sources the GPU code is built from (the .hip files and the
    headers they include), not of the host-only sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "microscaled_mxfp4_block_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_profile_record(workload):
    """The committed rocprofv3 record of one workload (profiles/gemm_traffic.json):
    traced per-call duration and HBM bytes per call, only if they were taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(workload)


def hw_lib():
    """libmx4hw.so: the streaming-read reference kernel (measurement only)."""
    L = ctypes.CDLL(os.path.join(ROOT, "microscaled_mxfp4_block_amd", "libmx4hw.so"))
    P, I, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
    L.mxhw_stream_read.argtypes = [P, U, I, I, I, U, U, U, P, P]
    return L


class Setup:
    """Rotating device copies of one workload's inputs, outputs and workspace."""

    def __init__(self, torch, B, inputs, M, N, K, seed_idx=None, cold=True):
        self.M, self.N, self.K = M, N, K
        if seed_idx is not None:
            A, Bm = inputs.workload_inputs(seed_idx, 1000)
        else:
            A, Bm = inputs.shape_inputs(M, N, K, seed=1000)
        dev = "cuda:0"
        A0 = A.to(dev)
        P0 = B.mx_pack_weight(Bm.to(dev))
        self.plan = B.mx_gemm_plan(M, N, K)
        ws_bytes = B.mx_gemm_workspace_bytes(M, N, K)
        per_set = A0.numel() * 2 + P0.numel() + M * N * 2 + ws_bytes
        self.copies = min(MAX_COPIES, max(4, -(-COLD_BYTES // per_set))) if cold else 1
        self.As = [A0] + [A0.clone() for _ in range(self.copies - 1)]
        self.Ps = [P0] + [P0.clone() for _ in range(self.copies - 1)]
        self.Cs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(self.copies)]
        self.ws = [torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev) for _ in range(self.copies)]
        self.args = [(a.data_ptr(), M, K, K, p.data_ptr(), N, c.data_ptr(), N, s.data_ptr(), s.numel())
                     for a, p, c, s in zip(self.As, self.Ps, self.Cs, self.ws)]
        self.fn = B.ext().gemm   # CPython fast-call wrapper of mx_gemm
        self.plan16 = B.mx_gemm_a16w4_plan(M, N, K)
        ws16 = B.mx_gemm_a16w4_workspace_bytes(M, N, K)
        self.ws16 = [torch.zeros(max(ws16, 256), dtype=torch.uint8, device=dev) for _ in range(self.copies)]
        self.args16 = [a[:8] + (w.data_ptr(), w.numel()) for a, w in zip(self.args, self.ws16)]
        self.fn16 = B.ext().gemm_a16w4
        torch.cuda.synchronize()

    def launches(self):
        p = self.plan
        return 1 + (p["amode"] in (1, 6)) + (1 if p["splits"] > 1 and not p["finish"] else 0)


def eager_loop(torch, st, steps, warmup, a16w4=False):
    """`steps` x CALLS_PER_STEP back-to-back calls between two
    synchronisations, after `warmup` untimed steps.  Returns (wall-clock us
    per call, event-timed us per call on the launch stream).  The argument
    tuples (rotating copies) are listed before the timed region; each call
    goes through the fast-call wrapper and its return code is checked."""
    fn, args = (st.fn16, st.args16) if a16w4 else (st.fn, st.args)
    stream = torch.cuda.current_stream().cuda_stream
    n = max(steps, warmup) * CALLS_PER_STEP
    seq = [args[i % st.copies] + (stream,) for i in range(n)]
    for a in seq[:warmup * CALLS_PER_STEP]:
        if fn(*a):
            raise RuntimeError("mx_gemm failed")
    torch.cuda.synchronize()
    seq = seq[:steps * CALLS_PER_STEP]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for a in seq:
        if fn(*a):
            raise RuntimeError("mx_gemm failed")
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / len(seq) * 1e6
    return wall, e0.elapsed_time(e1) * 1e3 / len(seq)


def graph_time(torch, call, ncap, min_seconds=0.2):
    """GPU time per captured call with the host out of the loop: `ncap`
    calls (call(i, stream)) captured once into a HIP graph on a side stream,
    replayed between two HIP events on that stream for at least
    `min_seconds`.  Returns us per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        handle = torch.cuda.current_stream().cuda_stream
        for i in range(ncap):
            call(i, handle)
    with torch.cuda.stream(s):
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        reps = max(3, int(min_seconds / max(time.perf_counter() - t0, 1e-6)))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * ncap)


def gemm_graph_time(torch, st, a16w4=False):
    fn, args = (st.fn16, st.args16) if a16w4 else (st.fn, st.args)

    def call(i, stream):
        if fn(*args[i % st.copies], stream):
            raise RuntimeError("mx_gemm failed under capture")
    return graph_time(torch, call, max(st.copies, CALLS_PER_STEP))


def stream_floor(torch, hw, st, B):
    """A kernel that only streams the call's packed weight bytes, with the
    GEMM's own grid (workgroups and waves) and 128-bit non-temporal loads,
    over the same rotating copies, graph-replayed: what moving those bytes
    alone costs at this launch shape."""
    p = st.plan
    nbytes = st.Ps[0].numel()
    ntiles = -(-((st.N + 31) // 32) // (p["nb"] * p["wn"]))
    mtiles = -(-((st.M + 31) // 32) // p["mb"])
    splits = p["splits"]
    wgs = ntiles * splits   # each weight byte once: the M tiles of an N tile share it
    waves = p["wn"] + p["wk"] if p["amode"] == 5 else p["wn"] * p["wk"]   # the shared mode: MFMA + quantiser waves
    chunk = -(-nbytes // wgs)
    chunk = -(-chunk // 16) * 16
    out = torch.empty(wgs * waves, dtype=torch.int32, device="cuda:0")

    def call(i, stream):
        rc = hw.mxhw_stream_read(st.Ps[i % st.copies].data_ptr(), nbytes, wgs, waves, 4, chunk, chunk, 0,
                                 out.data_ptr(), stream)
        if rc:
            raise RuntimeError("mxhw_stream_read returned %d" % rc)
    us = graph_time(torch, call, max(st.copies, CALLS_PER_STEP))
    return {"us": round(us, 3), "bytes": nbytes, "workgroups": wgs, "waves": waves, "gemm_m_tiles": mtiles}


# Streaming-read reference on one packed weight at several grids: the HBM
# rate a grid of that many workgroups can pull, whatever the kernel does.
STREAM_GRIDS = ((112, 4, 4), (112, 4, 16), (224, 4, 16), (256, 4, 16), (512, 4, 8), (1024, 4, 4), (2048, 4, 4),
                (1024, 8, 8))


def stream_rate_by_grid(torch, B, inputs, hw, N=7168, K=7168):
    """profiles/stream_rate_by_grid.md: graph-replay time of the streaming-read
    reference over the packed N x K weight (copies rotating over >= 512 MiB),
    workgroup g reading the g-th of `wgs` equal pieces with `waves` waves and
    `lpl` 16-byte loads in flight per lane (the best of three runs)."""
    gen = torch.Generator("cpu").manual_seed(3)
    P0 = B.mx_pack_weight(inputs.bf16_randn(N, K, gen).to("cuda:0"))
    nbytes = P0.numel()
    copies = max(4, -(-(512 << 20) // nbytes))
    Ps = [P0] + [P0.clone() for _ in range(copies - 1)]
    lines = ["# HBM streaming rate by grid", "",
             "`python3 bench.py --stream-rate`: the streaming-read reference kernel (`mxhw_stream_read`, 128-bit "
             "non-temporal buffer loads, no arithmetic) over the packed %d x %d weight (%d bytes), copies rotating "
             "over >= 512 MiB, HIP-graph replay, best of three runs. Workgroup g reads the g-th of `wgs` equal "
             "pieces." % (N, K, nbytes), "",
             "| workgroups | waves | loads in flight per lane | us | TB/s |", "|---|---|---|---|---|"]
    for wgs, waves, lpl in STREAM_GRIDS:
        chunk = -(-(-(-nbytes // wgs)) // 16) * 16
        out = torch.empty(wgs * waves, dtype=torch.int32, device="cuda:0")

        def call(i, stream):
            if hw.mxhw_stream_read(Ps[i % copies].data_ptr(), nbytes, wgs, waves, lpl, chunk, chunk, 0,
                                   out.data_ptr(), stream):
                raise RuntimeError("mxhw_stream_read failed")
        us = min(graph_time(torch, call, copies, min_seconds=0.05) for _ in range(3))
        lines.append("| %d | %d | %d | %.2f | %.2f |" % (wgs, waves, lpl, us, nbytes / us / 1e6))
        print(lines[-1], file=sys.stderr, flush=True)
    with open(os.path.join(ROOT, "profiles", "stream_rate_by_grid.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def launch_floor(torch, hw):
    """A near-empty kernel (one wave reading 16 bytes), graph-replayed."""
    buf = torch.zeros(256, dtype=torch.uint8, device="cuda:0")
    out = torch.empty(64, dtype=torch.int32, device="cuda:0")

    def call(i, stream):
        if hw.mxhw_stream_read(buf.data_ptr(), 16, 1, 1, 1, 16, 0, 0, out.data_ptr(), stream):
            raise RuntimeError("mxhw_stream_read failed")
    return round(graph_time(torch, call, 200), 3)


def cpu_baseline(idx, inputs, seconds=10.0):
    """The oracle (C, fp64 accumulation, OpenMP over N) on the host cores:
    quantise A + dequantise + GEMM per call; B is quantised and dequantised
    once beforehand, as mx_pack_weight is."""
    import oracle
    w = inputs.WORKLOADS[idx]
    A, Bm = inputs.workload_inputs(idx, 1000)
    Ab = inputs.bits(A)
    cb, sb = oracle.quant(inputs.bits(Bm))
    Bd = oracle.dequant(cb, sb)
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        ca, sa = oracle.quant(Ab)
        oracle.gemm_dequantised(oracle.dequant(ca, sa), Bd)
        times.append(time.perf_counter() - t0)
    return {"value": round(statistics.median(times) * 1e6, 1), "unit": "us/call", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d full calls of %s (quantise A, dequantise, fp64 GEMM, bf16 round), median; "
                      "B quantised once outside the timing" % (len(times), w.name)}


def measure_workload(torch, B, inputs, hw, idx, steps, warmup, name=None, shape=None):
    if shape is None:
        w = inputs.WORKLOADS[idx]
        shape, name = (w.M, w.N, w.K), w.name
    M, N, K = shape
    st = Setup(torch, B, inputs, M, N, K, seed_idx=idx)
    print("workload %s plan %s copies %d" % (name, st.plan, st.copies), file=sys.stderr, flush=True)
    e2e_cold, ev_cold = eager_loop(torch, st, steps, warmup)
    g_cold = gemm_graph_time(torch, st)
    g16 = gemm_graph_time(torch, st, a16w4=True)
    floor = stream_floor(torch, hw, st, B)
    del st
    torch.cuda.empty_cache()
    sh = Setup(torch, B, inputs, M, N, K, seed_idx=idx, cold=False)
    e2e_hot, _ = eager_loop(torch, sh, steps, warmup)
    g_hot = gemm_graph_time(torch, sh)
    plan, launches = sh.plan, sh.launches()
    del sh
    torch.cuda.empty_cache()
    nbytes = algorithmic_bytes(M, N, K)
    flops = 2.0 * M * N * K
    rec = {
        "M": M, "N": N, "K": K, "plan": plan, "launches_per_call": launches,
        "us_per_call_e2e_cold": round(e2e_cold, 3),
        "us_per_call_e2e_hot": round(e2e_hot, 3),
        "gpu_us_per_call_cold": round(g_cold, 3),
        "gpu_us_per_call_hot": round(g_hot, 3),
        "gpu_us_note": "HIP graph replay of the calls (host out of the loop), events on the replay stream; all "
                       "launches of a call",
        "eager_event_us_per_call_cold": round(ev_cold, 3),
        "algorithmic_bytes": nbytes,
        "gbps_cold": round(nbytes / g_cold / 1e3, 1),
        "hbm_frac_cold": round(nbytes / g_cold / 1e3 / HBM_PEAK_GBS, 4),
        "tflops_cold": round(flops / g_cold / 1e6, 2),
        "fp4_mfma_frac_cold": round(flops / g_cold / 1e6 / FP4_PEAK_TFLOPS, 5),
        "stream_floor": floor,
        "gpu_over_stream_floor": round(g_cold / floor["us"], 3),
        "a16w4": {"note": "the a16wfp4 product (A not quantised; a different function), same buffers",
                  "gpu_us_per_call_cold": round(g16, 3)},
    }
    print(json.dumps({name: rec}), file=sys.stderr, flush=True)
    return name, rec


# ---------------------------------------------------------------------------
# rocprofv3 support: runs with no timing, and the summary of their output


def profile_run(torch, B, inputs, hw, calls):
    """No timing.  A 256 MiB device copy (counter calibration), then per
    workload: CALLS mx_gemm calls over the cold rotating copies captured into
    a HIP graph and replayed once (the dispatches follow each other as in the
    bench), then CALLS dispatches of the streaming-read reference over the
    same weights, likewise.  For running under rocprofv3."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("calibration copy: %d bytes read + %d bytes written per dispatch" % (n, n), flush=True)
    del src, dst
    for idx, w in enumerate(inputs.WORKLOADS):
        st = Setup(torch, B, inputs, w.M, w.N, w.K, seed_idx=idx)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            handle = torch.cuda.current_stream().cuda_stream
            for i in range(calls):
                if st.fn(*st.args[i % st.copies], handle):
                    raise RuntimeError("mx_gemm failed under capture")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del g
        floor = stream_floor_profile(torch, hw, st, calls)
        print("profiled %s plan %s: %d calls, then %d streaming-read dispatches (%s)"
              % (w.name, st.plan, calls, calls, floor), flush=True)
        del st
        torch.cuda.empty_cache()


def stream_floor_profile(torch, hw, st, calls):
    p = st.plan
    nbytes = st.Ps[0].numel()
    ntiles = -(-((st.N + 31) // 32) // (p["nb"] * p["wn"]))
    wgs = ntiles * p["splits"]
    waves = p["wn"] + p["wk"] if p["amode"] == 5 else p["wn"] * p["wk"]   # the shared mode: MFMA + quantiser waves
    chunk = -(-(-(-nbytes // wgs)) // 16) * 16
    out = torch.empty(wgs * waves, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        handle = torch.cuda.current_stream().cuda_stream
        for i in range(calls):
            if hw.mxhw_stream_read(st.Ps[i % st.copies].data_ptr(), nbytes, wgs, waves, 4, chunk, chunk, 0,
                                   out.data_ptr(), handle):
                raise RuntimeError("mxhw_stream_read failed")
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return "%d workgroups x %d waves, %d bytes" % (wgs, waves, nbytes)


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_VALU_MFMA_BUSY_CYCLES")


def _csv(d, suffix):
    import csv
    for f in sorted(os.listdir(d)):
        if f.endswith(suffix):
            with open(os.path.join(d, f)) as fh:
                return list(csv.DictReader(fh))
    raise SystemExit("no *%s under %s" % (suffix, d))


def _short(name):
    import re
    return re.sub(r"\(.*", "", name).replace("void ", "")


def _dispatches(rows, counter_names=()):
    """rocprofv3 CSV rows -> one dict per dispatch in dispatch order: kernel
    name, grid (threads), duration in us, and the named counters (summed
    over the rows of a dispatch)."""
    per, order = {}, []
    for r in rows:
        key = int(r["Dispatch_Id"])
        if key not in per:
            grid = int(r["Grid_Size"]) if "Grid_Size" in r else \
                int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            per[key] = {"name": _short(r["Kernel_Name"]), "grid": grid,
                        "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
            order.append(key)
        if r.get("Counter_Name") in counter_names:
            d = per[key]
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in order]


def _calibration(disp, counter):
    """The counter's reading on the calibration copy: the largest among the
    dispatches that run before the first library kernel."""
    pre = []
    for d in disp:
        if d["name"].startswith("mx4::"):
            break
        pre.append(d.get(counter, 0.0))
    if not pre or max(pre) <= 0:
        raise SystemExit("no calibration dispatch before the first mx4 kernel")
    return max(pre)


def _segments(disp):
    """The mx4 dispatches of a --profile run split per workload: each
    segment is the weight pack, the calls' launches, then the
    streaming-read reference dispatches (the segment's end)."""
    segs, cur, in_stream = [], [], False
    for d in disp:
        if not d["name"].startswith("mx4::"):
            continue
        if d["name"].startswith("mx4::hw_stream_kernel"):
            cur.append(d)
            in_stream = True
            continue
        if in_stream:
            segs.append(cur)
            cur, in_stream = [], False
        cur.append(d)
    if cur:
        segs.append(cur)
    return segs


def summarize_profiles(trace_dir, fetch_dir, write_dir, mfma_dir, calls):
    """profiles/gemm_kernels_trace.md and profiles/gemm_traffic.json from the
    rocprofv3 output of four `bench.py --profile CALLS` runs: a kernel trace
    (durations: end minus start timestamp of each dispatch), FETCH_SIZE and
    WRITE_SIZE (each scaled by its reading on the 256 MiB calibration copy)
    and the fp4 MFMA counters.  Per workload the first dispatch (the weight
    pack) is left out; a call's traced duration is the sum of the averages
    of its launches."""
    from microscaled_mxfp4_block_amd import inputs
    trace = _dispatches(_csv(trace_dir, "kernel_trace.csv"))
    fetch = _dispatches(_csv(fetch_dir, "counter_collection.csv"), ("FETCH_SIZE",))
    write = _dispatches(_csv(write_dir, "counter_collection.csv"), ("WRITE_SIZE",))
    mfma = _dispatches(_csv(mfma_dir, "counter_collection.csv"), MFMA_COUNTERS)
    nw = len(inputs.WORKLOADS)
    segs = {k: _segments(v) for k, v in (("trace", trace), ("fetch", fetch), ("write", write), ("mfma", mfma))}
    for k, v in segs.items():
        if len(v) != nw:
            raise SystemExit("%s: %d workload segments, expected %d" % (k, len(v), nw))
    copy_bytes = 256 << 20
    cal_f = _calibration(fetch, "FETCH_SIZE")
    cal_w = _calibration(write, "WRITE_SIZE")
    f_scale, w_scale = copy_bytes / (cal_f * 1024), copy_bytes / (cal_w * 1024)
    cmd = "rocprofv3 %s -f csv -d %s -o %s -- python3 bench.py --profile %d"
    lines = ["# GEMM kernels on MI355X: rocprofv3 kernel trace and counters", "",
             "Kernel durations (end minus start timestamp of each dispatch): `%s`" % (
                 cmd % ("--kernel-trace --stats", trace_dir, "trace", calls)), "",
             "Counters, one run each: `%s`, `%s`, `%s`" % (
                 cmd % ("--pmc FETCH_SIZE", fetch_dir, "fetch", calls),
                 cmd % ("--pmc WRITE_SIZE", write_dir, "write", calls),
                 cmd % ("--pmc " + " ".join(MFMA_COUNTERS), mfma_dir, "mfma", calls)), "",
             "`--profile %d` runs a 256 MiB device copy (the counters' calibration: FETCH_SIZE reads %.0f KiB and "
             "WRITE_SIZE %.0f KiB on it, so they are scaled by %.3f and %.3f to bytes), then per workload: the weight "
             "pack (left out below), %d calls of mx_gemm over cold rotating copies (>= 512 MiB) captured in a HIP "
             "graph and replayed once, and %d dispatches of the streaming-read reference (the packed weight bytes "
             "only, with the GEMM's grid), also graph-replayed." % (calls, cal_f, cal_w, f_scale, w_scale, calls,
                                                                     calls), "",
             "| workload | kernel | grid (threads) | dispatches | avg us | median us | min us | FETCH bytes | "
             "WRITE bytes |", "|---|---|---|---|---|---|---|---|---|"]
    record = {"kernel_source_hash": kernel_source_hash(),
              "source": "profiles/gemm_kernels_trace.md (python3 bench.py --profile %d under rocprofv3)" % calls,
              "workloads": {}}
    mfma_rows = []
    for wi, w in enumerate(inputs.WORKLOADS):
        def groups(seg):
            g, order = {}, []
            for d in seg[1:]:   # the weight pack left out
                key = (d["name"], d["grid"])
                if key not in g:
                    g[key] = []
                    order.append(key)
                g[key].append(d)
            return g, order
        tg, order = groups(segs["trace"][wi])
        fg, _ = groups(segs["fetch"][wi])
        wg, _ = groups(segs["write"][wi])
        mg, _ = groups(segs["mfma"][wi])

        def med(gr, key, cname):
            vals = [d.get(cname) for d in gr.get(key, []) if d.get(cname) is not None]
            return statistics.median(vals) if vals else None
        call_us = call_fetch = call_write = 0.0
        floor_us = None
        for key in order:
            ds = [d["us"] for d in tg[key]]
            fb, wb = med(fg, key, "FETCH_SIZE"), med(wg, key, "WRITE_SIZE")
            fb = None if fb is None else fb * 1024 * f_scale
            wb = None if wb is None else wb * 1024 * w_scale
            lines.append("| %s | `%s` | %d | %d | %.3f | %.3f | %.3f | %s | %s |" % (
                w.name, key[0], key[1], len(ds), statistics.mean(ds), statistics.median(ds), min(ds),
                "%.0f" % fb if fb is not None else "-", "%.0f" % wb if wb is not None else "-"))
            if key[0].startswith("mx4::hw_stream_kernel"):
                floor_us = statistics.mean(ds)
                continue
            call_us += statistics.mean(ds)
            call_fetch += fb or 0.0
            call_write += wb or 0.0
            if key[0].startswith("mx4::gemm"):
                mfma_rows.append((w, key[0], statistics.mean(ds), med(mg, key, "SQ_INSTS_VALU_MFMA_F6F4"),
                                  med(mg, key, "SQ_INSTS_VALU_MFMA_MOPS_F6F4"),
                                  med(mg, key, "SQ_VALU_MFMA_BUSY_CYCLES")))
        flops = 2.0 * w.M * w.N * w.K
        record["workloads"][w.name] = {
            "traced_us_per_call": round(call_us, 3),
            "hbm_bytes_per_call": round(call_fetch + call_write),
            "fetch_bytes_per_call": round(call_fetch), "write_bytes_per_call": round(call_write),
            "algorithmic_bytes": algorithmic_bytes(w.M, w.N, w.K),
            "fp4_mfma_util_traced": round(flops / (call_us * 1e-6) / (FP4_PEAK_TFLOPS * 1e12), 5),
            "traced_stream_floor_us": None if floor_us is None else round(floor_us, 3)}
    lines += ["", "## Per call", "",
              "| workload | traced us per call (sum of averages) | algorithmic bytes | HBM fraction (8 TB/s) | "
              "counted HBM bytes | counted / algorithmic | streaming-read reference us | call / reference |",
              "|---|---|---|---|---|---|---|---|"]
    for w in inputs.WORKLOADS:
        r = record["workloads"][w.name]
        fl = r["traced_stream_floor_us"]
        lines.append("| %s | %.3f | %d | %.4f | %d | %.2f | %s | %s |" % (
            w.name, r["traced_us_per_call"], r["algorithmic_bytes"],
            r["algorithmic_bytes"] / r["traced_us_per_call"] / 1e3 / HBM_PEAK_GBS, r["hbm_bytes_per_call"],
            r["hbm_bytes_per_call"] / r["algorithmic_bytes"], "%.3f" % fl if fl else "-",
            "%.2f" % (r["traced_us_per_call"] / fl) if fl else "-"))
    lines += ["", "## fp4 MFMA counters", "",
              "Medians over each GEMM kernel's dispatches, summed over all XCDs. MOPS x 512 is the counter's flop "
              "count; it equals 2MNK when no MFMA work goes to padding rows or padding K steps. MFMA busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES / (traced duration x 2.4 GHz x 1024 SIMDs); fp4 utilisation = 2MNK / traced "
              "duration of the whole call / %.1f PFLOP/s (dense MXFP4 peak)." % (FP4_PEAK_TFLOPS / 1e3), "",
              "| workload | kernel | traced us | fp4 MFMA insts | MOPS x 512 | 2MNK | ratio | MFMA busy | fp4 "
              "utilisation (call) |", "|---|---|---|---|---|---|---|---|---|"]
    for w, kname, us, insts, mops, busy in mfma_rows:
        flops = 2.0 * w.M * w.N * w.K
        lines.append("| %s | `%s` | %.3f | %s | %s | %.4g | %s | %s | %.2f %% |" % (
            w.name, kname, us, "%.0f" % insts if insts is not None else "-",
            "%.4g" % (mops * 512) if mops is not None else "-", flops,
            "%.3f" % (mops * 512 / flops) if mops is not None else "-",
            "%.2f %%" % (100 * busy / (us * 2400.0 * 1024)) if busy is not None else "-",
            100 * record["workloads"][w.name]["fp4_mfma_util_traced"]))
    out = os.path.join(ROOT, "profiles")
    with open(os.path.join(out, "gemm_kernels_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out, "gemm_traffic.json"), "w") as f:
        json.dump(record, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# The other entry points on the path: the one-time weight pack, the standalone
# activation quantiser and the weight import, each an HBM-bound kernel.

SIDE_SHAPES = [(8192, 8192)]   # rows x K past the workloads, where the launch no longer dominates


def measure_side_ops(torch, B, inputs):
    """GPU time per call of mx_quant_act on each workload's A, and of
    mx_pack_weight and mx_import_weight on each workload's B, with GB/s of
    the bytes each call must move against 8 TB/s; the same on an
    8192 x 8192 operand.  Cold: the calls rotate over copies of their
    inputs and outputs (>= 512 MiB together), graph-replayed back to back."""
    L = B.lib()
    dev = "cuda:0"
    out = {}

    def rec(nbytes, us):
        return {"gpu_us": round(us, 3), "bytes": nbytes, "gbps": round(nbytes / us / 1e3, 1),
                "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}

    def ncopies(per_set):
        return min(MAX_COPIES, max(2, -(-COLD_BYTES // per_set)))
    shapes = [(w.name, w.M, w.N, w.K, i) for i, w in enumerate(inputs.WORKLOADS)]
    shapes += [("%dx%d" % (r, k), r, r, k, None) for r, k in SIDE_SHAPES]
    for name, M, N, K, idx in shapes:
        if idx is not None:
            A0, B0 = inputs.workload_inputs(idx, 1000)
        else:
            A0, B0 = inputs.shape_inputs(M, N, K, seed=1000)
        A0, B0 = A0.to(dev), B0.to(dev)
        P0 = B.mx_pack_weight(B0)
        bc0, bs0 = B.mx_unpack_weight(P0, N, K)
        qa_bytes = 2 * M * K + M * K // 2 + M * K // 32
        pk_bytes = 2 * N * K + P0.numel()
        im_bytes = bc0.numel() + bs0.numel() + P0.numel()
        res = {}
        # activation quantiser: A copies in, natural codes and scales out
        n = ncopies(qa_bytes)
        As = [A0] + [A0.clone() for _ in range(n - 1)]
        cs = [torch.empty((M, K // 2), dtype=torch.uint8, device=dev) for _ in range(n)]
        ss = [torch.empty((M, K // 32), dtype=torch.uint8, device=dev) for _ in range(n)]

        def quant(i, st):
            k = i % n
            if L.mx_quant_act(As[k].data_ptr(), M, K, K, cs[k].data_ptr(), ss[k].data_ptr(), st):
                raise RuntimeError("mx_quant_act failed")
        res["mx_quant_act"] = rec(qa_bytes, graph_time(torch, quant, max(n, 20)))
        del As, cs, ss
        # weight pack: B copies in, packed copies out
        n = ncopies(pk_bytes)
        Bs = [B0] + [B0.clone() for _ in range(n - 1)]
        Ps = [torch.empty_like(P0) for _ in range(n)]

        def pack(i, st):
            k = i % n
            if L.mx_pack_weight(Bs[k].data_ptr(), N, K, K, Ps[k].data_ptr(), Ps[k].numel(), st):
                raise RuntimeError("mx_pack_weight failed")
        res["mx_pack_weight"] = rec(pk_bytes, graph_time(torch, pack, max(n, 20)))
        del Bs
        # weight import: natural codes and scales in, packed out
        n = min(n, ncopies(im_bytes))
        bcs = [bc0] + [bc0.clone() for _ in range(n - 1)]
        bss = [bs0] + [bs0.clone() for _ in range(n - 1)]

        def imp(i, st):
            k = i % n
            if L.mx_import_weight(bcs[k].data_ptr(), bss[k].data_ptr(), N, K, Ps[k].data_ptr(), Ps[k].numel(), st):
                raise RuntimeError("mx_import_weight failed")
        res["mx_import_weight"] = rec(im_bytes, graph_time(torch, imp, max(n, 20)))
        out[name] = res
        print(json.dumps({"side_ops " + name: res}), file=sys.stderr, flush=True)
        del bcs, bss, Ps, A0, B0, P0, bc0, bs0
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# Large M: shapes where the contraction, not the weight stream, bounds the
# call (the tile mode's regime, from 64 x 64 tiles at 128 to 512 rows, the
# first on a grid small enough for the 16-stage ring, to 256 x 256 tiles).
# One set of buffers per shape, called back to back (at these sizes a call
# does far more MFMA work than it moves bytes).

LARGE_M_SHAPES = [(128, 2112, 7168), (256, 7168, 7168), (512, 2112, 7168), (1024, 4096, 4096), (2048, 7168, 2048),
                  (4096, 4096, 4096), (8192, 8192, 8192)]


def _large_name(M, N, K):
    return "%dx%dx%d" % (M, N, K)


def large_setup(torch, B, inputs, M, N, K):
    """Device inputs (seeded N(0,1) bf16), packed weight, output and
    workspace of one large-M shape, and the mx_gemm argument tuple."""
    A, Bm = inputs.shape_inputs(M, N, K, seed=1000)
    dev = "cuda:0"
    Ad = A.to(dev)
    del A
    P = B.mx_pack_weight(Bm.to(dev))
    del Bm
    plan = B.mx_gemm_plan(M, N, K)
    wsb = B.mx_gemm_workspace_bytes(M, N, K)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    args = (Ad.data_ptr(), M, K, K, P.data_ptr(), N, C.data_ptr(), N, ws.data_ptr(), ws.numel())
    torch.cuda.synchronize()
    return {"keep": (Ad, P, ws, C), "args": args, "plan": plan,
            "launches": 1 + (plan["amode"] in (1, 6)) + (1 if plan["splits"] > 1 and not plan["finish"] else 0)}


def load_large_profile():
    """profiles/large_m_traffic.json, only if taken on the current kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "large_m_traffic.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_source_hash") == kernel_source_hash() else None


def measure_large_m(torch, B, inputs):
    """GPU time per mx_gemm call (graph replay of 20 back-to-back calls) and
    the fp4 MFMA rate for each large-M shape; the traced per-kernel figures
    of the committed profile beside it when current."""
    fn = B.ext().gemm
    prof = load_large_profile()
    out = {}
    for (M, N, K) in LARGE_M_SHAPES:
        st = large_setup(torch, B, inputs, M, N, K)
        args = st["args"]

        def call(i, stream):
            if fn(*args, stream):
                raise RuntimeError("mx_gemm failed under capture")
        us = graph_time(torch, call, 20)
        flops = 2.0 * M * N * K
        name = _large_name(M, N, K)
        rec = {"plan": st["plan"], "launches_per_call": st["launches"], "gpu_us_per_call": round(us, 3),
               "tflops": round(flops / us / 1e6, 1), "fp4_mfma_frac": round(flops / us / 1e6 / FP4_PEAK_TFLOPS, 4)}
        if prof is not None and name in prof.get("shapes", {}):
            t = prof["shapes"][name]
            rec["traced"] = t
            gk = t.get("gemm_kernel")
            if gk:
                # the tile GEMM kernel against the dense fp4 MFMA peak (traced
                # duration), with its counted HBM bytes
                rec["roofline"] = {"bound": "mfma", "kernel": gk, "achieved": t["gemm_tflops_traced"],
                                   "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": t["gemm_fp4_frac_traced"],
                                   "traffic": t["kernels"][gk]["hbm_bytes"],
                                   "kernel_us_traced": t["kernels"][gk]["avg_us"]}
        out[name] = rec
        print(json.dumps({"large_m " + name: rec}), file=sys.stderr, flush=True)
        del st
        torch.cuda.empty_cache()
    return out


def profile_large_m(torch, B, inputs, hw, calls):
    """No timing.  The 256 MiB calibration copy, then per large-M shape: the
    weight pack, CALLS mx_gemm calls captured in a HIP graph and replayed
    once, and one near-empty reference dispatch that ends the shape's
    segment.  For running under rocprofv3."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    buf = torch.zeros(256, dtype=torch.uint8, device="cuda:0")
    mark = torch.empty(64, dtype=torch.int32, device="cuda:0")
    fn = B.ext().gemm
    for (M, N, K) in LARGE_M_SHAPES:
        st = large_setup(torch, B, inputs, M, N, K)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            handle = torch.cuda.current_stream().cuda_stream
            for _ in range(calls):
                if fn(*st["args"], handle):
                    raise RuntimeError("mx_gemm failed under capture")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del g
        if hw.mxhw_stream_read(buf.data_ptr(), 16, 1, 1, 1, 16, 0, 0, mark.data_ptr(),
                               torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("mxhw_stream_read failed")
        torch.cuda.synchronize()
        print("profiled %s plan %s: %d calls" % (_large_name(M, N, K), st["plan"], calls), flush=True)
        del st
        torch.cuda.empty_cache()


def summarize_large_m(trace_dir, fetch_dir, write_dir, mfma_dir, calls, out_dir=None):
    """profiles/large_m_trace.md and profiles/large_m_traffic.json from the
    rocprofv3 output of four `bench.py --profile-large-m CALLS` runs (trace,
    FETCH_SIZE, WRITE_SIZE, fp4 MFMA counters), per kernel of a call: traced
    duration, the fp4 MFMA rate of the GEMM kernel against the dense peak,
    and its counted HBM bytes against the bytes it must move."""
    trace = _dispatches(_csv(trace_dir, "kernel_trace.csv"))
    fetch = _dispatches(_csv(fetch_dir, "counter_collection.csv"), ("FETCH_SIZE",))
    write = _dispatches(_csv(write_dir, "counter_collection.csv"), ("WRITE_SIZE",))
    mfma = _dispatches(_csv(mfma_dir, "counter_collection.csv"), MFMA_COUNTERS)
    segs = {k: _segments(v) for k, v in (("trace", trace), ("fetch", fetch), ("write", write), ("mfma", mfma))}
    for k, v in segs.items():
        if len(v) != len(LARGE_M_SHAPES):
            raise SystemExit("%s: %d shape segments, expected %d" % (k, len(v), len(LARGE_M_SHAPES)))
    copy_bytes = 256 << 20
    cal_f = _calibration(fetch, "FETCH_SIZE")
    cal_w = _calibration(write, "WRITE_SIZE")
    f_scale, w_scale = copy_bytes / (cal_f * 1024), copy_bytes / (cal_w * 1024)
    cmd = "rocprofv3 %s -f csv -d %s -o %s -- python3 bench.py --profile-large-m %d"
    lines = ["# Large-M GEMM kernels on MI355X: rocprofv3 kernel trace and counters", "",
             "Kernel durations (end minus start timestamp of each dispatch): `%s`" % (
                 cmd % ("--kernel-trace --stats", trace_dir, "trace", calls)), "",
             "Counters, one run each: `%s`, `%s`, `%s`" % (
                 cmd % ("--pmc FETCH_SIZE", fetch_dir, "fetch", calls),
                 cmd % ("--pmc WRITE_SIZE", write_dir, "write", calls),
                 cmd % ("--pmc " + " ".join(MFMA_COUNTERS), mfma_dir, "mfma", calls)), "",
             "`--profile-large-m %d` runs the 256 MiB calibration copy (FETCH_SIZE reads %.0f KiB and WRITE_SIZE "
             "%.0f KiB on it, so they are scaled by %.3f and %.3f to bytes), then per shape: the weight pack (left "
             "out below) and %d back-to-back mx_gemm calls on one set of seeded N(0,1) bf16 buffers, captured in a "
             "HIP graph and replayed once. Bytes to move: the kernel's inputs and outputs once (pre-quantiser: A "
             "bf16 in, packed A out; GEMM: packed A and packed B in, C bf16 out)." % (
                 calls, cal_f, cal_w, f_scale, w_scale, calls), "",
             "| shape M x N x K | kernel | grid (threads) | dispatches | avg us | min us | fp4 TFLOP/s (avg) | "
             "of 10.1 PFLOP/s | FETCH bytes | WRITE bytes | bytes to move | counted / to move |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    record = {"kernel_source_hash": kernel_source_hash(),
              "source": "profiles/large_m_trace.md (python3 bench.py --profile-large-m %d under rocprofv3)" % calls,
              "shapes": {}}
    mrows = []
    for si, (M, N, K) in enumerate(LARGE_M_SHAPES):
        def groups(seg):
            g, order = {}, []
            for d in seg[1:]:   # the weight pack left out
                if d["name"].startswith("mx4::hw_stream_kernel"):
                    continue
                key = (d["name"], d["grid"])
                if key not in g:
                    g[key] = []
                    order.append(key)
                g[key].append(d)
            return g, order
        tg, order = groups(segs["trace"][si])
        fg, _ = groups(segs["fetch"][si])
        wg, _ = groups(segs["write"][si])
        mg, _ = groups(segs["mfma"][si])

        def med(gr, key, cname):
            vals = [d.get(cname) for d in gr.get(key, []) if d.get(cname) is not None]
            return statistics.median(vals) if vals else None
        flops = 2.0 * M * N * K
        packed = lambda rows: rows * K // 2 + rows * K // 32
        srec = {"kernels": {}}
        call_us = 0.0
        for key in order:
            ds = [d["us"] for d in tg[key]]
            avg = statistics.mean(ds)
            call_us += avg
            fb, wb = med(fg, key, "FETCH_SIZE"), med(wg, key, "WRITE_SIZE")
            fb = None if fb is None else fb * 1024 * f_scale
            wb = None if wb is None else wb * 1024 * w_scale
            gemm = key[0].startswith("mx4::gemm")
            move = packed(M) + packed(N) + 2 * M * N if gemm else 2 * M * K + packed(M)
            tf = flops / avg / 1e6 if gemm else None
            lines.append("| %s | `%s` | %d | %d | %.2f | %.2f | %s | %s | %s | %s | %d | %s |" % (
                _large_name(M, N, K), key[0], key[1], len(ds), avg, min(ds),
                "%.0f" % tf if tf else "-", "%.3f" % (tf / FP4_PEAK_TFLOPS) if tf else "-",
                "%.0f" % fb if fb is not None else "-", "%.0f" % wb if wb is not None else "-", move,
                "%.2f" % ((fb + wb) / move) if fb is not None and wb is not None else "-"))
            srec["kernels"][key[0]] = {"avg_us": round(avg, 3), "bytes_to_move": move,
                                       "hbm_bytes": None if fb is None or wb is None else round(fb + wb)}
            if gemm:
                srec["gemm_kernel"] = key[0]
                srec["gemm_tflops_traced"] = round(tf, 1)
                srec["gemm_fp4_frac_traced"] = round(tf / FP4_PEAK_TFLOPS, 4)
                mrows.append((M, N, K, key[0], avg, med(mg, key, "SQ_INSTS_VALU_MFMA_MOPS_F6F4"),
                              med(mg, key, "SQ_VALU_MFMA_BUSY_CYCLES")))
        srec["traced_us_per_call"] = round(call_us, 3)
        record["shapes"][_large_name(M, N, K)] = srec
    lines += ["", "## fp4 MFMA counters of the GEMM kernel", "",
              "Medians over the dispatches, summed over all XCDs. MOPS x 512 is the counter's flop count; MFMA busy "
              "= SQ_VALU_MFMA_BUSY_CYCLES / (traced duration x 2.4 GHz x 1024 SIMDs).", "",
              "| shape | kernel | traced us | MOPS x 512 | 2MNK | ratio | MFMA busy |", "|---|---|---|---|---|---|---|"]
    for M, N, K, kname, us, mops, busy in mrows:
        flops = 2.0 * M * N * K
        lines.append("| %s | `%s` | %.2f | %s | %.4g | %s | %s |" % (
            _large_name(M, N, K), kname, us, "%.4g" % (mops * 512) if mops is not None else "-", flops,
            "%.3f" % (mops * 512 / flops) if mops is not None else "-",
            "%.1f %%" % (100 * busy / (us * 2400.0 * 1024)) if busy is not None else "-"))
    out = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out, "large_m_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out, "large_m_traffic.json"), "w") as f:
        json.dump(record, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


# The shape grid of the pages (submission 754569, synthesized config CSV):
# 19 (N, K) weight shapes x batch sizes 1 .. 256.
GRID_DIM_PAIRS = [
    (2880, 512), (2112, 7168), (4096, 512), (7168, 2048), (3072, 1536),
    (2880, 1536), (4096, 1536), (2112, 512), (2112, 2048),
    (7168, 512), (7168, 1536), (7168, 7168), (3072, 512),
    (3072, 7168), (3072, 2048), (4096, 2048), (4096, 7168),
    (2880, 2048), (2880, 7168),
]
GRID_BATCH = [1, 2, 4, 8, 16, 32, 64, 128, 256]
# Past the grid: large M over six of its weight shapes (the planner's tile-mode rule).
LARGE_REGRET_PAIRS = [(4096, 512), (3072, 1536), (7168, 2048), (2880, 2048), (2112, 7168), (7168, 7168)]
LARGE_REGRET_M = [256, 384, 512, 768, 1024, 2048]


# The tile mode's workgroup tiles: (mb, nb, wk, wn) = M blocks, N blocks,
# waves along M, waves along N.
TILE_SHAPES = ((8, 8, 2, 4), (4, 8, 2, 2), (8, 4, 2, 2), (4, 4, 2, 2), (4, 4, 2, 4), (2, 2, 2, 2))


def regret_candidates(B, M, N, K):
    """Plans timed against the library's own for one grid shape: the
    register-quantising mode over wave and split counts and two N widths,
    the pre-quantising mode over its tile shapes, the LDS mode, the shared
    mode over its MFMA and quantiser waves and splits, the tile mode over
    its tiles (with 2 to 4 K splits where its grid is small); only those the
    planner accepts."""
    cands = []
    for nb in (1, 2):
        for wk in (2, 4, 8):
            for sp in (1, 2, 4, 7, 8, 14):
                cands.append(dict(mb=1, nb=nb, wn=1, wk=wk, splits=sp, amode=2, finish=0))
    for mb, nb, wn, wk in ((1, 1, 1, 8), (2, 1, 1, 8), (2, 2, 1, 8), (1, 1, 1, 4), (2, 1, 2, 8), (2, 2, 1, 4)):
        for sp in (1, 2, 4):
            cands.append(dict(mb=mb, nb=nb, wn=wn, wk=wk, splits=sp, amode=1, finish=0))
    for sp in (1, 2, 4):
        cands.append(dict(mb=1, nb=1, wn=1, wk=8, splits=sp, amode=0, finish=0))
    for wn in (3, 4):
        for wk in (4, 8):
            for sp in (1, 2, 4, 7, 8, 14):
                cands.append(dict(mb=1, nb=1, wn=wn, wk=wk, splits=sp, amode=5, finish=0))
    if M >= 32:   # the tile mode over its tiles (64 .. 256 rows); K splits where its grid is under 256 workgroups
        for mb, nb, wk, wn in TILE_SHAPES:
            if 32 * mb <= 2 * max(M, 32):
                cands.append(dict(mb=mb, nb=nb, wn=wn, wk=wk, splits=1, amode=6, finish=0))
                wgs = -(-M // (32 * mb)) * -(-N // (32 * nb))
                if K >= 2048 and wgs < 256:
                    for sp in (2, 3, 4):
                        cands.append(dict(mb=mb, nb=nb, wn=wn, wk=wk, splits=sp, amode=6, finish=0))
    out = []
    for p in cands:
        try:
            B.mx_gemm_workspace_bytes(M, N, K, p)
        except B.MxError:
            continue
        out.append(p)
    return out


def random_regret_groups(count=40, seed=2024):
    """Seeded off-grid shapes for the planner's regret: M in 1 .. 1024 (log
    uniform), N in 256 .. 8192 (a multiple of 32, log uniform), K in 256 ..
    8192 (a multiple of 256, log uniform), grouped by (N, K)."""
    rng = np.random.default_rng(seed)
    groups = {}
    for _ in range(count):
        M = int(round(2 ** rng.uniform(0, 10)))
        N = 32 * int(round(2 ** rng.uniform(3, 8)))
        K = 256 * int(round(2 ** rng.uniform(0, 5)))
        groups.setdefault((N, K), []).append(M)
    return [(nk, sorted(set(ms))) for nk, ms in sorted(groups.items())]


def plan_regret(torch, B, inputs, only=None, out=None, large=False, random_groups=None, seed=2024):
    """Graph-replay GPU time per call of the library's plan and of the
    candidate plans for every grid shape (weights rotating over copies
    >= 256 MiB).  With `out`, every candidate's time goes to that JSON file
    (a part, for --regret-merge); else the summary goes to
    profiles/plan_regret.md.  With `large`, the shapes are LARGE_REGRET_PAIRS x
    LARGE_REGRET_M and the summary goes to profiles/plan_regret_large.md."""
    dev = "cuda:0"
    results = []
    pairs = GRID_DIM_PAIRS if only is None else [GRID_DIM_PAIRS[i] for i in only]
    groups = [(nk, GRID_BATCH) for nk in pairs]
    if large:
        groups = [(nk, LARGE_REGRET_M) for nk in LARGE_REGRET_PAIRS]
    if random_groups is not None:
        groups = random_groups
    for (N, K), batches in groups:
        gen = torch.Generator("cpu").manual_seed(5000 + N + K)
        P0 = B.mx_pack_weight(inputs.bf16_randn(N, K, gen).to(dev))
        copies = min(200, max(4, -(-(256 << 20) // P0.numel())))
        Ps = [P0] + [P0.clone() for _ in range(copies - 1)]
        for M in batches:
            A0 = inputs.bf16_randn(M, K, gen).to(dev)
            C0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            lib_plan = B.mx_gemm_plan(M, N, K)
            fn = B.ext().gemm_with_plan
            rows = []
            for p in [lib_plan] + [c for c in regret_candidates(B, M, N, K) if c != lib_plan]:
                wsb = B.mx_gemm_workspace_bytes(M, N, K, p)
                ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)
                pa = (p["mb"], p["nb"], p["wn"], p["wk"], p["splits"], p["amode"], p["finish"])

                def call(i, stream):
                    if fn(A0.data_ptr(), M, K, K, Ps[i % copies].data_ptr(), N, C0.data_ptr(), N, ws.data_ptr(),
                          ws.numel(), *pa, stream):
                        raise RuntimeError("mx_gemm_with_plan failed")
                rows.append((graph_time(torch, call, copies, min_seconds=0.02), p))
                del ws
            lib_us = rows[0][0]
            best_us, best = min(rows, key=lambda r: r[0])
            results.append({"M": M, "N": N, "K": K, "plan": lib_plan, "us": round(lib_us, 3), "best_plan": best,
                            "best_us": round(best_us, 3), "regret": round(lib_us / best_us, 3),
                            "candidates": len(rows), "all": [[round(u, 3), p] for u, p in rows]})
            print("regret %4d x %4d x %4d  plan %.3f us  best %.3f us  x%.3f  %s" % (
                M, N, K, lib_us, best_us, lib_us / best_us, best), file=sys.stderr, flush=True)
            del A0, C0
        del Ps, P0
        torch.cuda.empty_cache()
    if out:
        with open(out, "w") as f:
            json.dump({"shapes": results}, f)
    if random_groups is not None:
        cmd = "`python3 bench.py --plan-regret-random%s`" % ("" if seed == 2024 else " --regret-seed %d" % seed)
        regret_summary(results, cmd, random=True, seed=seed)
    elif large:
        regret_summary(results, "`python3 bench.py --plan-regret-large`", large=True)
    elif not out:
        regret_summary(results, "`python3 bench.py --plan-regret`")


def regret_summary(results, command, large=False, random=False, seed=2024):
    """profiles/plan_regret.md from the timed shapes (without the
    per-candidate times); with `large`, profiles/plan_regret_large.md."""
    regrets = [r["regret"] for r in results]
    geo = float(np.exp(np.mean(np.log(regrets)))) if regrets else float("nan")
    if random:
        lines = ["# Planner regret on seeded off-grid shapes", "",
                 "%s: for each of %d seeded random shapes (`random_regret_groups`, seed %d: M in 1 .. 1024, N in "
                 "256 .. 8192, K in 256 .. 8192, log uniform; off the pages' grid), the HIP-graph-replay GPU time "
                 "per call of the plan mx_gemm picks against the fastest of up to %d candidate plans (those of the "
                 "grid sweep), weights rotating over copies of >= 256 MiB. Regret = plan time / best time; "
                 "geometric mean %.3f, worst %.3f." % (command, len(results), seed,
                                                       max((r["candidates"] for r in results), default=0), geo,
                                                       max(regrets, default=0)),
                 "", "| M | N | K | plan (mb nb wn wk splits amode) | us | best plan | best us | regret |",
                 "|---|---|---|---|---|---|---|---|"]
        return _regret_tables(results, lines, "plan_regret_random" + ("" if seed == 2024 else "_seed%d" % seed))
    if large:
        lines = ["# Planner regret at large M", "",
                 "%s: for each of the %d shapes (M = %s x six (N, K) weight shapes of the pages' grid; the grid "
                 "itself stops at M = 256), the HIP-graph-replay GPU time per call of the plan mx_gemm picks "
                 "against the fastest of up to %d candidate plans (those of the grid sweep, the tile mode's "
                 "tiles among them), weights rotating over copies of >= 256 MiB. Regret = plan time / best time; "
                 "geometric mean %.3f, worst %.3f." % (
                     command, len(results), ", ".join(str(m) for m in LARGE_REGRET_M),
                     max((r["candidates"] for r in results), default=0), geo, max(regrets, default=0)),
                 "", "| M | N | K | plan (mb nb wn wk splits amode) | us | best plan | best us | regret |",
                 "|---|---|---|---|---|---|---|---|"]
        return _regret_tables(results, lines, "plan_regret_large")
    lines = ["# Planner regret on the pages' shape grid", "",
             "%s: for each of the %d shapes (19 (N, K) weight shapes of the "
             "kernelindex.com amd-mxfp4-mm pages' synthesized config CSV, submission 754569, times M = 1 .. 256), "
             "the HIP-graph-replay GPU time per call of the plan mx_gemm picks (the measured table for the "
             "workloads, the model elsewhere) against the fastest of up to %d candidate plans (register-quantising "
             "mode over waves, splits and N widths; pre-quantising mode over its tiles; LDS mode; quantiser-wave "
             "shared mode over its waves and splits; from M = 32 the tile mode over its tiles), weights rotating "
             "over copies of >= 256 MiB. "
             "Regret = plan time / best time; geometric mean %.3f, worst %.3f." % (
                 command, len(results), max((r["candidates"] for r in results), default=0), geo,
                 max(regrets, default=0)),
             "", "| M | N | K | plan (mb nb wn wk splits amode) | us | best plan | best us | regret |",
             "|---|---|---|---|---|---|---|---|"]

    return _regret_tables(results, lines, "plan_regret")


def _regret_tables(results, lines, stem):
    def ps(p):
        return "%d %d %d %d %d %d" % (p["mb"], p["nb"], p["wn"], p["wk"], p["splits"], p["amode"])
    for r in results:
        lines.append("| %d | %d | %d | %s | %.3f | %s | %.3f | %.3f |" % (
            r["M"], r["N"], r["K"], ps(r["plan"]), r["us"], ps(r["best_plan"]), r["best_us"], r["regret"]))
    with open(os.path.join(ROOT, "profiles", stem + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_markdown(stats_csv, command):
    """profiles/bench_kernel_stats.md: the rocprofv3 --stats summary of the
    mx4 kernels of one bench.py run under the tracer."""
    import csv
    with open(stats_csv) as f:
        rows = [r for r in csv.DictReader(f) if "mx4::" in r["Name"]]
    lines = ["# Kernel statistics of bench.py under rocprofv3", "",
             "`%s` (the bench command of the bench line, fewer steps), `*_kernel_stats.csv` rows of the mx4 "
             "kernels. Under the tracer consecutive dispatches start about 9 us apart, so each traced duration is "
             "that of a kernel starting on an idle GPU; the bench line's GPU time per call is the untraced HIP-graph "
             "replay." % command, "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("| `%s` | %s | %.3f | %.3f | %.3f |" % (_short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                                                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    with open(os.path.join(ROOT, "profiles", "bench_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of %d calls each" % CALLS_PER_STEP)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads")
    ap.add_argument("--profile", type=int, default=0, metavar="CALLS",
                    help="no timing: a 256 MiB device copy (counter calibration), then per workload CALLS cold "
                         "mx_gemm calls and CALLS streaming-read reference dispatches, for running under rocprofv3")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                    help="no GPU: summarise the rocprofv3 output of --profile runs into profiles/")
    ap.add_argument("--summarize-calls", type=int, default=100, help="the --profile CALLS being summarised")
    ap.add_argument("--no-large-m", action="store_true", help="skip the large-M (MFMA-bound) shapes")
    ap.add_argument("--profile-large-m", type=int, default=0, metavar="CALLS",
                    help="no timing: the calibration copy, then per large-M shape CALLS mx_gemm calls, for "
                         "running under rocprofv3")
    ap.add_argument("--summarize-large-m", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                    help="no GPU: summarise the rocprofv3 output of --profile-large-m runs into profiles/")
    ap.add_argument("--plan-regret", nargs="?", const="all", default=None, metavar="PAIRS",
                    help="time the library's plan against candidate plans on the pages' shape grid (PAIRS: "
                         "comma-separated indices of the (N, K) pairs, default all) and write profiles/plan_regret.md")
    ap.add_argument("--plan-regret-large", action="store_true",
                    help="the same at M = 256 .. 2048 over six of the grid's weight shapes, tile plans among the "
                         "candidates; writes profiles/plan_regret_large.md")
    ap.add_argument("--plan-regret-random", action="store_true",
                    help="the same over 40 seeded off-grid shapes (random_regret_groups); writes "
                         "profiles/plan_regret_random.md")
    ap.add_argument("--regret-seed", type=int, default=2024,
                    help="with --plan-regret-random: the seed of the shapes (other than 2024: "
                         "profiles/plan_regret_random_seedSEED.md)")
    ap.add_argument("--regret-out", default=None, metavar="JSON",
                    help="with --plan-regret: write every candidate's time to JSON (a part for --regret-merge) "
                         "instead of profiles/plan_regret.md")
    ap.add_argument("--regret-merge", nargs="+", metavar="JSON",
                    help="no GPU: profiles/plan_regret.md from --regret-out parts (in grid order)")
    ap.add_argument("--stream-rate", action="store_true",
                    help="the streaming-read reference over a 7168 x 7168 packed weight at several grids; writes "
                         "profiles/stream_rate_by_grid.md")
    ap.add_argument("--stats-md", nargs=2, metavar=("STATS_CSV", "COMMAND"),
                    help="no GPU: profiles/bench_kernel_stats.md from a rocprofv3 --stats kernel_stats.csv")
    args = ap.parse_args()
    if args.stats_md:
        stats_markdown(*args.stats_md)
        return
    if args.regret_merge:
        results = []
        for path in args.regret_merge:
            with open(path) as f:
                results += json.load(f)["shapes"]
        order = {nk: i for i, nk in enumerate(GRID_DIM_PAIRS)}
        results.sort(key=lambda r: (order[(r["N"], r["K"])], r["M"]))
        regret_summary(results, "`python3 bench.py --plan-regret PAIRS --regret-out PART` over parts of the grid, "
                                "then `python3 bench.py --regret-merge PART...`")
        return
    if args.summarize:
        summarize_profiles(*args.summarize, args.summarize_calls)
        return
    if args.summarize_large_m:
        summarize_large_m(*args.summarize_large_m, args.summarize_calls)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from microscaled_mxfp4_block_amd import binding as B
    from microscaled_mxfp4_block_amd import inputs
    hw = hw_lib()

    if args.profile:
        profile_run(torch, B, inputs, hw, args.profile)
        return
    if args.stream_rate:
        stream_rate_by_grid(torch, B, inputs, hw)
        return
    if args.profile_large_m:
        profile_large_m(torch, B, inputs, hw, args.profile_large_m)
        return
    if args.plan_regret:
        only = None if args.plan_regret == "all" else [int(i) for i in args.plan_regret.split(",")]
        plan_regret(torch, B, inputs, only, args.regret_out)
        return
    if args.plan_regret_random:
        plan_regret(torch, B, inputs, out=args.regret_out, random_groups=random_regret_groups(seed=args.regret_seed),
                    seed=args.regret_seed)
        return
    if args.plan_regret_large:
        plan_regret(torch, B, inputs, out=args.regret_out, large=True)
        return

    per_workload = {}
    order = [HEADLINE] + ([] if args.only_headline else [i for i in range(len(inputs.WORKLOADS)) if i != HEADLINE])
    for idx in order:
        name, rec = measure_workload(torch, B, inputs, hw, idx, args.steps, args.warmup)
        per_workload[name] = rec
    if not args.only_headline:
        for w in inputs.EXTRA_WORKLOADS:
            name, rec = measure_workload(torch, B, inputs, hw, None, max(5, args.steps // 4), args.warmup,
                                         name=w.name, shape=(w.M, w.N, w.K))
            per_workload[name] = rec
    w = inputs.WORKLOADS[HEADLINE]
    rec = per_workload[w.name]
    nbytes = algorithmic_bytes(w.M, w.N, w.K)
    flops = 2.0 * w.M * w.N * w.K
    prof = load_profile_record(w.name)
    line = {
        "metric": "us/call per (M,N,K) MXFP4 GEMM incl. A-quant (end-to-end, cold weights)",
        "value": rec["us_per_call_e2e_cold"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["us_per_call_e2e_cold"] * CALLS_PER_STEP / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "baseline_note": "no published figure for this metric and workload; the pages' 16.2 us end-to-end for "
                         "this shape (CK route, MI355X) is context only",
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "plan": rec["plan"],
                   "calls_per_step": CALLS_PER_STEP, "seed": 1000, "distribution": "N(0,1) bf16",
                   "weights": "cold: rotating copies, >= 512 MiB working set"},
        "roofline": {
            "bound": "hbm",
            "achieved": rec["gbps_cold"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": rec["hbm_frac_cold"],
            "traffic": None if prof is None else prof.get("hbm_bytes_per_call"),
            "kernel": "one mx_gemm call: %s" % ("gemm_shared_kernel (one launch)" if rec["launches_per_call"] == 1
                                                else "%d launches" % rec["launches_per_call"]),
            "kernel_us": rec["gpu_us_per_call_cold"],
            "kernel_us_method": "HIP graph replay of cold calls, HIP events on the replay stream (all launches "
                                "of a call, host out of the loop)",
            "kernel_us_traced": None if prof is None else prof.get("traced_us_per_call"),
            "bytes_per_launch": nbytes,
        },
        "mfma": {
            "dtype": "fp4 (e2m1 x e2m1, e8m0 block scales)",
            "achieved_tflops": rec["tflops_cold"],
            "peak_tflops": FP4_PEAK_TFLOPS,
            "frac": rec["fp4_mfma_frac_cold"],
            "flops_per_call": flops,
        },
        "reference_floors": {
            "near_empty_kernel_us": launch_floor(torch, hw),
            "stream_same_weight_us": rec["stream_floor"]["us"],
            "method": "HIP graph replay; the streaming-read kernel reads the call's packed weight bytes with the "
                      "GEMM's grid and stores one dword per wave",
        },
        "per_workload": per_workload,
    }
    if not args.only_headline:
        line["side_ops"] = {
            "note": "the other entry points on the path, GPU us per call in HIP graph replay of back-to-back calls "
                    "over rotating copies (>= 512 MiB, cold): mx_quant_act on A (bytes 2MK in + MK/2 + MK/32 out), "
                    "mx_pack_weight on B (2NK in + the packed bytes out), mx_import_weight (natural codes and "
                    "scales in + the packed bytes out); GB/s of those bytes against 8 TB/s",
            "shapes": measure_side_ops(torch, B, inputs)}
    if not args.no_large_m and not args.only_headline:
        line["large_m"] = {
            "note": "MFMA-bound shapes (tile mode): GPU us per mx_gemm call in HIP graph replay of 20 back-to-back "
                    "calls on one set of buffers, all launches of a call; fp4 rate against the 10.1 PFLOP/s dense "
                    "peak; 'traced' = the committed rocprofv3 figures per kernel when taken on the current sources",
            "shapes": measure_large_m(torch, B, inputs)}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(HEADLINE, inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
