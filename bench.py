"""Benchmark of the MXFP4 GEMM path on one MI355X.

One step = one mx_gemm call (activation quantisation + block-scaled MFMA
contraction + split-K reduction when planned + bf16 epilogue) on the
M=32, N=4096, K=512 decode workload; the weight is packed once beforehand.
Inputs are seeded N(0,1) bf16 (synthetic stand-ins for the leaderboard's
data) resident in HBM; the timed loop rotates over enough copies of A, the
packed weight and C that the working set (>= 1 GiB) cannot sit in the 256 MB
Infinity Cache, so every call streams its weight from HBM ("cold").

Printed: one JSON line with the end-to-end µs per call (value, wall clock
over the timed region), the GEMM kernel's average launch time (HIP events on
the launch stream over the same region; one launch per call) against the HBM
roofline, the oracle timed on the host cores (cpu_baseline) and the same
figures for the other four workloads (per_workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA, published
HEADLINE = 1                   # index of M=32, N=4096, K=512 in inputs.WORKLOADS
PAGES_E2E_US = {"m32_n4096_k512": 10.6}   # pages' end-to-end figure for this workload (MI355X)
WORKING_SET = 1 << 30


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


def load_traffic(workload):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


class Setup:
    """Rotating device copies of one workload's inputs, outputs and workspace."""

    def __init__(self, idx, torch, B, inputs):
        w = inputs.WORKLOADS[idx]
        self.w = w
        A, Bm = inputs.workload_inputs(idx, 1000)
        dev = "cuda:0"
        self.A_cpu, self.B_cpu = A, Bm
        A0 = A.to(dev)
        P0 = B.mx_pack_weight(Bm.to(dev))
        self.plan = B.mx_gemm_plan(w.M, w.N, w.K)
        ws_bytes = B.mx_gemm_workspace_bytes(w.M, w.N, w.K)
        per_set = A0.numel() * 2 + P0.numel() + w.M * w.N * 2 + ws_bytes
        self.copies = max(4, WORKING_SET // per_set)
        self.As = [A0] + [A0.clone() for _ in range(self.copies - 1)]
        self.Ps = [P0] + [P0.clone() for _ in range(self.copies - 1)]
        self.Cs = [torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev) for _ in range(self.copies)]
        self.ws = [torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev) for _ in range(self.copies)]
        stream = torch.cuda.current_stream().cuda_stream
        self.args = [(a.data_ptr(), w.M, w.K, w.K, p.data_ptr(), w.N, c.data_ptr(), w.N, s.data_ptr(), s.numel(),
                      stream) for a, p, c, s in zip(self.As, self.Ps, self.Cs, self.ws)]
        self.fn = B.ext().gemm   # CPython fast-call wrapper of mx_gemm
        # the a16wfp4 product on the same buffers (context figures)
        self.plan16 = B.mx_gemm_a16w4_plan(w.M, w.N, w.K)
        ws16 = B.mx_gemm_a16w4_workspace_bytes(w.M, w.N, w.K)
        self.ws16 = [torch.zeros(max(ws16, 256), dtype=torch.uint8, device=dev) for _ in range(min(self.copies, 8))]
        self.args16 = [a[:8] + (self.ws16[i % len(self.ws16)].data_ptr(), self.ws16[0].numel(), stream)
                       for i, a in enumerate(self.args)]
        self.fn16 = B.ext().gemm_a16w4
        torch.cuda.synchronize()

    def call(self, i):
        rc = self.fn(*self.args[i % self.copies])
        if rc:
            raise RuntimeError("mx_gemm returned %d" % rc)

    def call16(self, i):
        rc = self.fn16(*self.args16[i % self.copies])
        if rc:
            raise RuntimeError("mx_gemm_a16w4 returned %d" % rc)


def time_loop(torch, st, steps, warmup, rotate=True, a16w4=False):
    """`steps` back-to-back mx_gemm calls between two synchronisations.
    Returns (wall-clock µs per call, event-timed µs per launch): HIP events
    recorded on the launch stream bracket the whole timed region.  The
    argument tuples of the calls (rotating buffer copies) are listed before
    the region; each call goes through the fast-call wrapper and its return
    code is checked."""
    fn, args = (st.fn16, st.args16) if a16w4 else (st.fn, st.args)
    seq = [args[i % st.copies if rotate else 0] for i in range(max(steps, warmup))]
    for a in seq[:warmup]:
        if fn(*a):
            raise RuntimeError("mx_gemm failed")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    seq = seq[:steps]
    t0 = time.perf_counter()
    e0.record()
    for a in seq:
        if fn(*a):
            raise RuntimeError("mx_gemm failed")
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e6
    return wall, e0.elapsed_time(e1) * 1e3 / steps


def graph_loop(torch, st, ncap=100, reps=20):
    """GPU time per call with the host out of the loop: `ncap` calls over
    distinct buffer copies are captured once into a HIP graph on a side
    stream and replayed `reps` times between two events on that stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        handle = torch.cuda.current_stream().cuda_stream
        for i in range(ncap):
            rc = st.fn(*st.args[i % st.copies][:-1], handle)
            if rc:
                raise RuntimeError("mx_gemm returned %d under capture" % rc)
    with torch.cuda.stream(s):
        g.replay()
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * ncap)


def launch_floor(torch, same_bytes, ncap=100, reps=20):
    """What any kernel costs on this GPU, replayed from a HIP graph so that the
    host is out of the loop: a near-empty kernel (torch's one-cycle sleep),
    a plain 1 MiB device copy, and a device copy that moves `same_bytes` HBM
    bytes (same_bytes / 2 read + the same written), over rotating buffers."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    n = 1 << 20
    src = [torch.ones(n, dtype=torch.uint8, device="cuda:0") for _ in range(ncap)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(ncap)]
    h = same_bytes // 2
    src2 = [torch.ones(h, dtype=torch.uint8, device="cuda:0") for _ in range(ncap)]
    dst2 = [torch.empty(h, dtype=torch.uint8, device="cuda:0") for _ in range(ncap)]
    torch.cuda.synchronize()
    out = {}
    for name, body in (("empty_kernel_us", lambda i: torch.cuda._sleep(1)),
                       ("copy_1MiB_us", lambda i: dst[i].copy_(src[i])),
                       ("copy_same_bytes_us", lambda i: dst2[i].copy_(src2[i]))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(ncap):
                body(i)
        with torch.cuda.stream(s):
            g.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * ncap), 3)
    out["same_bytes"] = 2 * h
    out["method"] = ("HIP graph of %d launches replayed %d times, HIP events on the replay stream; the same-bytes "
                     "copy moves as many HBM bytes as one call of the headline workload" % (ncap, reps))
    return out


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
    return {"value": statistics.median(times) * 1e6, "unit": "us/call", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d full calls of %s (quantise A, dequantise, fp64 GEMM, bf16 round), median; "
                      "B quantised once outside the timing" % (len(times), w.name)}


def profile_run(torch, B, inputs, calls, graph=False):
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("calibration copy: %d bytes read + %d bytes written per dispatch" % (n, n), flush=True)
    del src, dst
    for idx in range(len(inputs.WORKLOADS)):
        st = Setup(idx, torch, B, inputs)
        if graph:
            # the calls captured once into a HIP graph and replayed: the
            # dispatches then follow each other as in an untraced eager loop
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                handle = torch.cuda.current_stream().cuda_stream
                for i in range(calls):
                    if st.fn(*st.args[i % st.copies][:-1], handle):
                        raise RuntimeError("mx_gemm failed under capture")
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            del g
        else:
            for i in range(calls):
                st.call(i)
        torch.cuda.synchronize()
        print("profiled %s plan %s: %d calls%s" % (st.w.name, st.plan, calls, " (graph replay)" if graph else ""),
              flush=True)
        del st
        torch.cuda.empty_cache()


def profile_floor_run(torch, inputs, calls):
    """Reference kernels for a rocprofv3 kernel trace, no timing: `calls`
    near-empty kernels (torch's one-cycle sleep), then per workload, in the
    workload order, `calls` plain device copies that move the same HBM bytes
    as one GEMM call (algorithmic bytes / 2 read + the same written), over
    rotating buffers with a >= 1 GiB working set like the GEMM calls."""
    for _ in range(calls):
        torch.cuda._sleep(1)
    torch.cuda.synchronize()
    print("profiled %d near-empty kernels" % calls, flush=True)
    for w in inputs.WORKLOADS:
        n = algorithmic_bytes(w.M, w.N, w.K) // 2
        copies = max(4, WORKING_SET // (2 * n))
        # torch.empty launches nothing, so the trace holds only the copies
        src = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
        dst = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
        for i in range(calls):
            dst[i % copies].copy_(src[i % copies])
        torch.cuda.synchronize()
        print("profiled %s: %d copies of %d bytes" % (w.name, calls, n), flush=True)
        del src, dst
        torch.cuda.empty_cache()


def floor_lines(floor_dir, calls):
    """Rows of the reference-kernel table from a trace of --profile-floor,
    whose dispatches are exactly `calls` near-empty kernels, then `calls`
    copies per workload in the workload order."""
    import csv
    from microscaled_mxfp4_block_amd import inputs
    rows = None
    for f in sorted(os.listdir(floor_dir)):
        if f.endswith("kernel_trace.csv"):
            with open(os.path.join(floor_dir, f)) as fh:
                rows = list(csv.DictReader(fh))
    if rows is None:
        raise SystemExit("no *kernel_trace.csv under %s" % floor_dir)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    labels = ["near-empty kernel (torch.cuda._sleep(1))"] + [
        "device copy moving %d HBM bytes, as one %s call" % (2 * (algorithmic_bytes(w.M, w.N, w.K) // 2), w.name)
        for w in inputs.WORKLOADS]
    rows = rows[-calls * len(labels):]
    if len(rows) != calls * len(labels):
        raise SystemExit("expected %d dispatches in the floor trace" % (calls * len(labels)))
    out = []
    for li, label in enumerate(labels):
        part = rows[li * calls:(li + 1) * calls]
        ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in part]
        short = part[0]["Kernel_Name"].split("(")[0].replace("void ", "")[:60]
        out.append("| %s | `%s` | %d | %.3f | %.3f | %.3f |" % (
            label, short, len(part), statistics.mean(ds), statistics.median(ds), min(ds)))
    return out


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")


def mfma_lines(mfma_dir, calls, trace_us):
    """Rows of the MFMA table from one --pmc pass over the MFMA counters of
    a --profile run: per GEMM kernel, the fp4 MFMA instructions and their
    flops (MOPS x 512) against 2MNK, the MFMA-busy share of the 1024 SIMDs'
    cycles over the kernel's traced duration `trace_us[(kernel, grid)]` at
    the 2.4 GHz peak clock, and the useful fp4 rate 2MNK / duration against
    the dense MXFP4 peak."""
    import collections
    import csv
    import re
    from microscaled_mxfp4_block_amd import inputs
    rows = None
    for f in sorted(os.listdir(mfma_dir)):
        if f.endswith("counter_collection.csv"):
            with open(os.path.join(mfma_dir, f)) as fh:
                rows = list(csv.DictReader(fh))
    if rows is None:
        raise SystemExit("no *counter_collection.csv under %s" % mfma_dir)
    per = collections.OrderedDict()   # (kernel, grid) -> dispatch id -> counter -> value
    for r in rows:
        grid = int(r["Grid_Size"]) if "Grid_Size" in r else int(r["Grid_Size_X"])
        key = (re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", ""), grid)
        d = per.setdefault(key, collections.OrderedDict()).setdefault(r.get("Dispatch_Id", r.get("Correlation_Id")), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    gemms = [(k, v) for k, v in per.items() if k[0].startswith("mx4::gemm_kernel") and len(v) == calls]
    out = []
    for w, ((name, grid), disp) in zip(inputs.WORKLOADS, gemms):
        med = {c: statistics.median(d.get(c, 0.0) for d in disp.values()) for c in MFMA_COUNTERS}
        flops = med["SQ_INSTS_VALU_MFMA_MOPS_F6F4"] * 512
        us = trace_us.get((name, grid))
        busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (us * 2400.0 * 1024) if us else float("nan")
        useful = 2.0 * w.M * w.N * w.K / (us * 1e-6) / (FP4_PEAK_TFLOPS * 1e12) if us else float("nan")
        out.append("| %s | `%s` | %d | %.0f | %.4g | %.4g | %.3f | %.0f | %.3f | %.2f %% | %.2f %% |" % (
            w.name, name, grid, med["SQ_INSTS_VALU_MFMA_F6F4"], flops, 2.0 * w.M * w.N * w.K,
            flops / (2.0 * w.M * w.N * w.K), med["SQ_VALU_MFMA_BUSY_CYCLES"], us or float("nan"),
            100 * busy, 100 * useful))
    return out


def summarize_profiles(trace_dir, fetch_dir, write_dir, calls_trace, calls_pmc, floor_dir=None, mfma_dir=None):
    """Write profiles/gemm_kernels_trace.md (per-kernel durations from a
    rocprofv3 kernel trace of `bench.py --profile`, HBM bytes from the
    FETCH_SIZE and WRITE_SIZE passes) and profiles/gemm_traffic.json (the
    bytes per GEMM launch that the bench line reports as roofline traffic).
    The counters are scaled by their reading on the 256 MiB copy that
    `--profile` runs first."""
    import collections
    import csv
    import re

    def table(d, suffix):
        for f in sorted(os.listdir(d)):
            if f.endswith(suffix):
                with open(os.path.join(d, f)) as fh:
                    return list(csv.DictReader(fh))
        raise SystemExit("no *%s under %s" % (suffix, d))

    def grid_of(r):
        if "Grid_Size_X" in r:   # kernel trace: per dimension; counters: the product
            return int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1)) * int(r.get("Grid_Size_Z", 1))
        return int(r["Grid_Size"])

    durations = collections.OrderedDict()
    for r in table(trace_dir, "kernel_trace.csv"):
        key = (r["Kernel_Name"], str(grid_of(r)))
        durations.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counter(d):
        agg = collections.OrderedDict()
        for r in table(d, "counter_collection.csv"):
            agg.setdefault((r["Kernel_Name"], str(grid_of(r))), []).append(float(r["Counter_Value"]))
        return agg

    fetch, write = counter(fetch_dir), counter(write_dir)
    copy_bytes = 256 << 20
    cal_f = max(max(v) for v in fetch.values())
    cal_w = max(max(v) for v in write.values())
    f_scale, w_scale = copy_bytes / (cal_f * 1024), copy_bytes / (cal_w * 1024)
    cmd_t = ("rocprofv3 --kernel-trace --stats -f csv -d %s -o trace -- python3 bench.py --profile %d"
             % (trace_dir, calls_trace))
    cmd_f = ("rocprofv3 --pmc FETCH_SIZE -f csv -d %s -o fetch -- python3 bench.py --profile %d"
             % (fetch_dir, calls_pmc))
    cmd_w = ("rocprofv3 --pmc WRITE_SIZE -f csv -d %s -o write -- python3 bench.py --profile %d"
             % (write_dir, calls_pmc))
    lines = ["# GEMM kernels on MI355X: rocprofv3 kernel trace and HBM counters", "",
             "Kernel durations (end minus start timestamp of each dispatch): `%s`" % cmd_t, "",
             "Counters, one per run: `%s` and `%s`" % (cmd_f, cmd_w), "",
             "Calibration: the 256 MiB device copy that `--profile` runs first reads FETCH_SIZE = %.0f KiB and "
             "WRITE_SIZE = %.0f KiB per dispatch, so FETCH_SIZE is scaled by %.3f and WRITE_SIZE by %.3f to "
             "bytes." % (cal_f, cal_w, f_scale, w_scale), "",
             "`--profile` runs, per workload in order: the weight pack (one dispatch, large grid), then the "
             "calls of mx_gemm over rotating buffer copies (>= 1 GiB working set).", "",
             "| kernel | grid (threads) | dispatches | avg us | median us | min us | FETCH bytes | WRITE bytes |",
             "|---|---|---|---|---|---|---|---|"]
    per_launch = collections.OrderedDict()
    for (name, grid), ds in durations.items():
        if "mx4::" not in name:
            continue
        fb = statistics.median(fetch[(name, grid)]) * 1024 * f_scale if (name, grid) in fetch else None
        wb = statistics.median(write[(name, grid)]) * 1024 * w_scale if (name, grid) in write else None
        short = re.sub(r"\(.*", "", name).replace("void ", "")
        lines.append("| `%s` | %s | %d | %.3f | %.3f | %.3f | %s | %s |" % (
            short, grid, len(ds), statistics.mean(ds), statistics.median(ds), min(ds),
            "%.0f" % fb if fb is not None else "-", "%.0f" % wb if wb is not None else "-"))
        if short.startswith("mx4::gemm_kernel") and len(ds) > 1:
            per_launch[(short, grid)] = (statistics.mean(ds), fb, wb)
    from microscaled_mxfp4_block_amd import inputs
    gemms = list(per_launch.items())
    traffic = {"kernel_source_hash": kernel_source_hash(),
               "source": "profiles/gemm_kernels_trace.md: FETCH_SIZE and WRITE_SIZE passes over python3 bench.py "
                         "--profile %d, scaled by their reading on a 256 MiB device copy (x%.3f, x%.3f)"
                         % (calls_pmc, f_scale, w_scale),
               "workloads": {}}
    if len(gemms) == len(inputs.WORKLOADS):
        for w, ((short, grid), (avg, fb, wb)) in zip(inputs.WORKLOADS, gemms):
            traffic["workloads"][w.name] = {
                "kernel": short, "grid": int(grid), "avg_us": round(avg, 3),
                "fetch_bytes": None if fb is None else round(fb),
                "write_bytes": None if wb is None else round(wb),
                "hbm_bytes_per_launch": None if fb is None or wb is None else round(fb + wb)}
    if floor_dir:
        lines += ["", "## Reference kernels", "",
                  "What any launch costs here, from `rocprofv3 --kernel-trace --stats -f csv -d %s -o floor -- "
                  "python3 bench.py --profile-floor %d`: the near-empty kernel is the floor of every dispatch, and "
                  "each copy reads and writes as many HBM bytes as one GEMM call of its workload moves (cold, "
                  "rotating buffers), so it is the time a kernel that only moved those bytes would take."
                  % (floor_dir, calls_trace), "",
                  "| reference | kernel | dispatches | avg us | median us | min us |", "|---|---|---|---|---|---|"]
        lines += floor_lines(floor_dir, calls_trace)
    if mfma_dir:
        lines += ["", "## MFMA counters", "",
                  "`rocprofv3 --pmc %s -f csv -d %s -o mfma -- python3 bench.py --profile %d`, medians over the "
                  "GEMM dispatches of each workload (counters summed over all XCDs and shader engines). MOPS x 512 "
                  "is the counter's flop count; it equals 2MNK when no MFMA work goes to padding rows or padding "
                  "K steps. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (traced duration x 2.4 GHz x 1024 SIMDs); "
                  "fp4 utilisation = 2MNK / traced duration / %.1f PFLOP/s (dense MXFP4 peak). The duration is the "
                  "kernel's average in the trace above." % (" ".join(MFMA_COUNTERS), mfma_dir, calls_pmc,
                                                           FP4_PEAK_TFLOPS / 1e3), "",
                  "| workload | kernel | grid | fp4 MFMA insts | MOPS x 512 | 2MNK | ratio | MFMA busy cycles | "
                  "traced us | MFMA busy | fp4 utilisation |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        trace_us = {}
        for (name, grid), ds in durations.items():
            trace_us[(re.sub(r"\(.*", "", name).replace("void ", ""), int(grid))] = statistics.mean(ds)
        lines += mfma_lines(mfma_dir, calls_pmc, trace_us)
    out = os.path.join(ROOT, "profiles")
    with open(os.path.join(out, "gemm_kernels_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out, "gemm_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--only-headline", action="store_true", help="skip the other four workloads")
    ap.add_argument("--profile", type=int, default=0, metavar="CALLS",
                    help="no timing: a 256 MiB device copy (counter calibration), then CALLS cold mx_gemm "
                         "calls per workload, for running under rocprofv3")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarise rocprofv3 output of --profile runs into profiles/")
    ap.add_argument("--graph", action="store_true",
                    help="with --profile: capture each workload's calls into a HIP graph and replay it once")
    ap.add_argument("--profile-floor", type=int, default=0, metavar="CALLS",
                    help="no timing: CALLS near-empty kernels, then CALLS device copies per workload that move "
                         "the bytes of one of its GEMM calls, for running under rocprofv3")
    ap.add_argument("--floor-dir", help="with --summarize: rocprofv3 trace directory of a --profile-floor run")
    ap.add_argument("--mfma-dir", help="with --summarize: rocprofv3 --pmc directory of the MFMA counter pass")
    ap.add_argument("--summarize-calls", nargs=2, type=int, default=[200, 20], metavar=("TRACE", "PMC"),
                    help="the --profile CALLS of the trace and of the counter runs being summarised")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(*args.summarize, *args.summarize_calls, floor_dir=args.floor_dir, mfma_dir=args.mfma_dir)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from microscaled_mxfp4_block_amd import binding as B
    from microscaled_mxfp4_block_amd import inputs

    if args.profile:
        profile_run(torch, B, inputs, args.profile, graph=args.graph)
        return
    if args.profile_floor:
        profile_floor_run(torch, inputs, args.profile_floor)
        return

    per_workload = {}
    headline = None
    order = [HEADLINE] + ([i for i in range(len(inputs.WORKLOADS)) if i != HEADLINE]
                          if not args.only_headline else [])
    for idx in order:
        st = Setup(idx, torch, B, inputs)
        w = st.w
        print("workload %s plan %s copies %d" % (w.name, st.plan, st.copies), file=sys.stderr, flush=True)
        steps = args.steps if idx == HEADLINE else max(200, args.steps // 4)
        e2e_cold, gpu_cold = time_loop(torch, st, steps, args.warmup)
        e2e_hot, gpu_hot = time_loop(torch, st, steps, args.warmup, rotate=False)
        gpu_graph = graph_loop(torch, st)
        e2e16, gpu16 = time_loop(torch, st, max(200, steps // 4), args.warmup, a16w4=True)
        nbytes = algorithmic_bytes(w.M, w.N, w.K)
        flops = 2.0 * w.M * w.N * w.K
        rec = {
            "M": w.M, "N": w.N, "K": w.K, "plan": st.plan,
            "launches_per_call": 1 + (st.plan["amode"] == 1) + (1 if st.plan["splits"] > 1 and not st.plan["finish"] else 0),
            "us_per_call_e2e_cold": round(e2e_cold, 3), "us_per_call_e2e_hot": round(e2e_hot, 3),
            "gpu_us_cold": round(gpu_cold, 3), "gpu_us_hot": round(gpu_hot, 3),
            "gpu_us_graph_replay": round(gpu_graph, 3),
            "algorithmic_bytes": nbytes, "gbps_cold": round(nbytes / gpu_cold / 1e3, 1),
            "hbm_frac_cold": round(nbytes / gpu_cold / 1e3 / HBM_PEAK_GBS, 4),
            "tflops_cold": round(flops / gpu_cold / 1e6, 2),
            "mfma_frac_cold": round(flops / gpu_cold / 1e6 / FP4_PEAK_TFLOPS, 5),
            "a16w4": {"note": "the a16wfp4 product (A not quantised; a different function), same buffers",
                      "plan": st.plan16, "us_per_call_e2e_cold": round(e2e16, 3), "gpu_us_cold": round(gpu16, 3)},
        }
        per_workload[w.name] = rec
        print(json.dumps({w.name: rec}), file=sys.stderr, flush=True)
        if idx == HEADLINE:
            headline = (st, rec, steps)
        del st
        torch.cuda.empty_cache()

    st, rec, steps = headline
    w = st.w
    nbytes = algorithmic_bytes(w.M, w.N, w.K)
    line = {
        "metric": "us/call per (M,N,K) MXFP4 GEMM incl. A-quant (end-to-end, cold weights)",
        "value": rec["us_per_call_e2e_cold"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["us_per_call_e2e_cold"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(rec["us_per_call_e2e_cold"] / PAGES_E2E_US[w.name], 4),
        "baseline_note": "pages' end-to-end 10.6 us/call on MI355X for this shape (kernelindex.com submission "
                         "733989 docstring); context only",
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "plan": st.plan,
                   "seed": 1000, "distribution": "N(0,1) bf16"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(nbytes / rec["gpu_us_cold"] / 1e3, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes / rec["gpu_us_cold"] / 1e3 / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(w.name),
            "kernel": "mx4::gemm_kernel (the only launch of a call for this plan)",
            "kernel_us": rec["gpu_us_cold"],
            "bytes_per_launch": nbytes,
        },
        "per_workload": per_workload,
        "launch_floor": launch_floor(torch, nbytes),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(HEADLINE, inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
