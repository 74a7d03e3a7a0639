"""MLA decode benchmark on one MI355X.

A step is one decode of the batch (mla_decode_run: the stage-1 split kernel,
then the stage-2 LSE merge) over seeded synthetic inputs already resident in
HBM.
The default workload is bs=64, kv_len=8192, bf16 q, fp8 E4M3FN KV (the
bs>=32 / kv=8192 / fp8 shape the bandwidth target is stated for).  Every
workload's KV buffer is rotated over enough copies (>= 768 MB in total, so
163 copies of the 4.7 MB bs=4 batch) that each call reads KV that is not
resident in the 256 MB last-level cache: the bandwidth is HBM bandwidth, not
cache bandwidth.

Prints one JSON line: value = KV bytes read per second over the timed steps
(GB/s; K calls back to back between two synchronisations, after W warm-up
calls that follow about 0.1 s of untimed calls which settle the device's
clocks to this kernel), plus per-call
microseconds, the stage-1 kernel's roofline (its average launch duration from
K stage-1 launches back to back between two HIP events on the launch stream),
stage 1's matrix-unit rate (the method's QK^T and PV flops over the same launch
time, against the dense bf16 peak) and the CPU oracle timed on a bounded sample
of the same workload.  The table
of workloads gives the same figures for each of the five workloads (and the
headline shape with two and four query rows), each with the oracle timed on a
bounded sample of that workload.  A plain read kernel over one 1 GiB buffer
(at most 200 launches) gives the read rate of this device as context.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
DEFAULT_WORKLOAD = "bs64_kv8192_fp8"
KERNEL_SRC = os.path.join(ROOT, "mla_decode_split_amd", "csrc", "mla_decode.hip")

# HBM bytes of one stage-1 launch on the default workload, from two rocprofv3
# counter passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by
# what the same counter reads for a plain device copy of 512 MiB.  Valid only
# for the kernel code they were taken on: the sha256 of the kernel source with
# its comments removed and its whitespace collapsed (code_sha256 below), so
# that editing a comment keeps them and changing code drops them (traffic is
# then reported as null).  The counters were taken on the source whose full
# sha256 is 94e7d37e...c16d6a8d.
TRAFFIC_MEASURED = {
    "workload": DEFAULT_WORKLOAD,
    "code_sha256": "0090a0d63fc373d41d71d6fc4d7fa5f8630579376d244f2711498ce12743093a",
    "fetch_kib": 149906.6,
    "write_kib": 8224.0,
    "fetch_scale": 2.0,
    "write_scale": 1.0,
}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--logit-cap", type=float, default=0.0, help="> 0: soft-cap the scaled scores")
    ap.add_argument("--paged", action="store_true",
                    help="paged KV: rows (or pages, see --page-size) scattered over a buffer 1/8 larger by a "
                         "random permutation")
    ap.add_argument("--page-size", type=int, default=1, help="with --paged: rows per page (a power of two)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query rows per sequence (multi-token prediction / speculative decoding)")
    ap.add_argument("--rows-per-split", type=int, default=0)
    ap.add_argument("--wgs-per-cu", type=int, default=0)
    ap.add_argument("--age-skew", type=int, default=0,
                    help="per mille of the range moved to each CU's first workgroup (0 planner, -1 none)")
    ap.add_argument("--hot", action="store_true", help="no KV rotation (cache-resident numbers, secondary)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU thread-seconds of each oracle sample")
    ap.add_argument("--only-headline", action="store_true", help="skip the per-workload table")
    ap.add_argument("--read-ceiling-s", type=float, default=0.2,
                    help="seconds of the plain read kernel over one 1 GiB buffer (at most 200 launches; 0: skip)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MB (reference for HBM counters)")
    return ap.parse_args()


def _host_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16
    (a one-GPU share of the GPU hosts here)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_description() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(w, kv_bytes_per_row: float, target_s: float) -> dict:
    """The oracle, unchanged, on a bounded sample of the workload's sequences:
    about `target_s` thread-seconds on _host_threads() threads."""
    import oracle

    threads = _host_threads()
    lengths = np.diff(w.kv_indptr).astype(np.int64)
    qo = np.diff(np.asarray(w.qo_indptr, dtype=np.int64))
    order = np.arange(len(lengths))
    # calibrate on one sequence, then take as many as fit the time budget
    first = int(np.flatnonzero(lengths > 0)[0])
    t0 = time.perf_counter()
    oracle.decode_workload(w, seq_ids=[first], threads=1)
    per_row = (time.perf_counter() - t0) / max(int(lengths[first]) * max(int(qo[first]), 1), 1)
    budget_rows = target_s / max(per_row, 1e-9)  # per_row is one thread's time
    take, rows = [], 0
    for b in order:
        if rows + lengths[b] * max(int(qo[b]), 1) > budget_rows and take:
            break
        take.append(int(b))
        rows += int(lengths[b]) * max(int(qo[b]), 1)
    kv_rows = int(lengths[take].sum())
    # when the whole workload is smaller than the budget, time repeated passes over it
    passes, dt = 0, 0.0
    while passes == 0 or dt * threads < target_s:
        t0 = time.perf_counter()
        oracle.decode_workload(w, seq_ids=take, threads=threads)
        dt += time.perf_counter() - t0
        passes += 1
    res = {"value": round(passes * kv_rows * kv_bytes_per_row / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{len(take)} of {len(lengths)} sequences ({kv_rows} KV rows) x {passes} pass(es), fp64 C, "
                     f"{dt:.2f} s wall on {threads} threads"}
    res.update(_cpu_description())
    return res


def mfma_flop(w) -> int:
    """The method's matrix work per call: for every (KV row, query row) pair of a
    sequence, QK^T over 576 dims and PV over 512 columns for 16 heads, 2 flop
    per multiply-add."""
    kv = np.diff(np.asarray(w.kv_indptr, dtype=np.int64))
    q = np.diff(np.asarray(w.qo_indptr, dtype=np.int64))
    return int(2 * 16 * (576 + 512) * int((kv * q).sum()))


def mfma_block(flop: int, us: float) -> dict:
    """Stage 1's matrix-unit rate from the method's flops and its launch time,
    against the dense bf16 peak (the PV products are bf16; the rocprofv3
    MfmaUtil counter per workload is in profiles/)."""
    achieved = flop / (us * 1e-6) / 1e12
    return {"flop_per_launch": flop, "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "peak_dtype": "bf16"}


def code_sha256(path: str = KERNEL_SRC) -> str:
    """sha256 of a C++ source with its comments removed (string and character
    literals kept as they are) and every run of whitespace collapsed to one
    space."""
    import hashlib

    text = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # a literal: copied up to its closing quote
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
            out.append(" ")
        else:
            out.append(c)
            i += 1
    code = " ".join("".join(out).split())
    return hashlib.sha256(code.encode()).hexdigest()


def _measured_traffic(name: str):
    t = TRAFFIC_MEASURED
    if name != t["workload"] or not t["code_sha256"] or t["code_sha256"] != code_sha256():
        return None
    return int(round(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])))


def read_ceiling(seconds: float) -> float:
    """GB/s of the plain read kernel (mla_debug_stream_read) over one 1 GiB
    buffer: a few warm-up launches, then up to 200 timed launches (about
    `seconds`) between two HIP events, with a synchronisation every 50."""
    import torch
    import mla_decode_split_amd as mla

    nbytes = 1 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        mla.mla_debug_stream_read(buf, nbytes, sink, stream)
    torch.cuda.synchronize()
    reps = max(10, min(200, int(seconds * 6e12 / nbytes)))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(reps):
        mla.mla_debug_stream_read(buf, nbytes, sink, stream)
        if i % 50 == 49:
            b.record(stream)
            b.synchronize()
    b.record(stream)
    torch.cuda.synchronize()
    rate = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return rate


class Timed:
    """One workload resident on the GPU, its plan and rotated KV copies."""

    def __init__(self, name, args, threads, q_len=1):
        import torch
        import synth
        from mla_decode_split_amd import device as dev

        self.name = name if q_len == 1 else f"{name}_q{q_len}"
        self.q_len = q_len
        self.spec = synth.WORKLOADS[name]
        t = time.perf_counter()
        self.w = synth.make_workload(name, threads=threads, q_len=q_len)
        self.w.logit_cap = float(getattr(args, "logit_cap", 0.0))
        if getattr(args, "paged", False):
            ps = int(getattr(args, "page_size", 1))
            self.w = synth.page_workload(self.w, seed=99, spare_rows=self.w.total_kv // 8, threads=threads,
                                         page_size=ps)
            self.name += "_paged" if ps == 1 else f"_pages{ps}"
        self.t_gen = time.perf_counter() - t
        self.kv_bytes = self.w.kv_bytes()
        self.rows = int(self.w.kv_indptr[-1] - self.w.kv_indptr[0])
        self.batch = dev.upload(self.w)
        t = time.perf_counter()
        self.plan = dev.plan_for(self.batch, rows_per_split=args.rows_per_split, wgs_per_cu=args.wgs_per_cu,
                                 age_skew=getattr(args, "age_skew", 0))
        self.t_plan = time.perf_counter() - t
        self.ncopy = 1 if args.hot else max(1, math.ceil(768e6 / max(self.kv_bytes, 1)))
        self.kvs = [self.batch.kv] + [self.batch.kv.clone() for _ in range(self.ncopy - 1)]
        self.out = torch.empty((self.batch.total_q, 16, 512), dtype=torch.bfloat16, device="cuda")
        self.ws = dev.workspace_for(self.plan)
        self.stream = torch.cuda.current_stream()

    def step(self, i):
        """One decode: mla_decode_run (stage 1, then stage 2 when the plan needs it)."""
        from mla_decode_split_amd import device as dev

        self.batch.kv = self.kvs[i % self.ncopy]
        dev.run(self.plan, self.batch, self.out, self.ws, self.stream)

    def settle(self, seconds):
        """Untimed calls for about `seconds` (device clocks settle to this kernel)."""
        import torch

        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.step(i)
                i += 1
            torch.cuda.synchronize()

    def time(self, steps, warmup):
        """Seconds for `steps` whole calls back to back, after `warmup` untimed ones."""
        import torch

        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def split_launch_us(self, steps):
        """Average stage-1 launch duration: `steps` stage-1 launches back to back
        on the launch stream between one pair of HIP events on that stream."""
        import torch
        from mla_decode_split_amd import device as dev

        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.step(0)
        a.record(self.stream)
        for i in range(steps):
            self.batch.kv = self.kvs[i % self.ncopy]
            dev.run_split(self.plan, self.batch, self.out, self.ws, self.stream)
        b.record(self.stream)
        torch.cuda.synchronize()
        dev.run_merge(self.plan, self.batch, self.out, self.ws, self.stream)
        return 1e3 * a.elapsed_time(b) / steps

    def ring_read_us(self, steps):
        """Average duration of mla_debug_stream_ring over this call's KV bytes
        (the KV copies rotated as for the calls, as many workgroups as stage 1
        launches): stage 1's memory side with no arithmetic.  fp8 KV only (the
        ring has the fp8 kernel's geometry); None otherwise."""
        import torch
        import mla_decode_split_amd as mla

        if self.w.kv_dtype != "fp8" or self.w.kv_indices is not None or self.kv_bytes % 18432:
            return None
        wgs = mla.mla_decode_plan_describe(self.plan)["num_splits"]
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        for i in range(3):
            mla.mla_debug_stream_ring(self.kvs[i % self.ncopy], self.kv_bytes, wgs, sink, self.stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for i in range(steps):
            mla.mla_debug_stream_ring(self.kvs[i % self.ncopy], self.kv_bytes, wgs, sink, self.stream)
        b.record(self.stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / steps

    def describe(self):
        import mla_decode_split_amd as mla

        d = mla.mla_decode_plan_describe(self.plan)
        return {"workload": self.name, "batch_size": self.spec["bs"], "kv_len": self.spec["kv_len"],
                "q_len": self.q_len, "logit_cap": self.w.logit_cap, "paged": self.w.kv_indices is not None,
                "page_size": int(getattr(self.w, "page_size", 1)),
                "q_dtype": self.w.q_dtype, "kv_dtype": self.w.kv_dtype, "kv_rows": self.rows,
                "kv_bytes": self.kv_bytes, "kv_copies_rotated": self.ncopy, "num_splits": d["num_splits"],
                "rows_per_split": d["rows_per_split"], "stage2": bool(d["stage2"]),
                "paired_splits": d["paired_splits"], "second_rows_per_split": d["second_rows_per_split"]}


def main() -> int:
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(sequences would shard across GPUs with no exchange; each GPU runs this same path on its share)",
              file=sys.stderr)
        return 2

    import torch

    import mla_decode_split_amd as mla

    if not os.path.exists(mla.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)
    threads = _host_threads()
    name = args.workload

    h = Timed(name, args, threads, args.q_len)
    ceiling = read_ceiling(args.read_ceiling_s) if args.read_ceiling_s > 0 else None
    # about 0.1 s of decode calls before the W warm-up steps: the device settles
    # its clocks to the kernel it runs (after the read kernel or the host-side
    # input generation, the first few ms of calls run up to 5 % slower)
    h.settle(0.1)
    # throughput: K whole calls back to back, nothing recorded between them
    elapsed = h.time(args.steps, args.warmup)
    # roofline: K stage-1 launches back to back between two events on their stream
    split_us = h.split_launch_us(args.steps)
    ring_us = h.ring_read_us(args.steps)
    ms_per_step = 1e3 * elapsed / args.steps
    value = h.kv_bytes * args.steps / elapsed / 1e9
    achieved = h.kv_bytes / (split_us * 1e-6) / 1e9
    cfg = h.describe()

    res = {
        "metric": "MLA decode achieved HBM bandwidth on KV bytes (stage 1 + stage 2 per call)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(1e3 * ms_per_step, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "read_ceiling_GBs": round(ceiling, 1) if ceiling else None,
        "frac_of_read_ceiling": round(value / ceiling, 4) if ceiling else None,
        # stage 1's memory side alone (mla_debug_stream_ring over the same bytes)
        "ring_read_us": round(ring_us, 3) if ring_us else None,
        "ring_read_GBs": round(h.kv_bytes / (ring_us * 1e-6) / 1e9, 1) if ring_us else None,
        "stage1_frac_of_ring_read": round(ring_us / split_us, 4) if ring_us else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if (h.w.q_dtype == "fp8" and h.w.kv_dtype == "fp8") else "bf16",
        "data": "synthetic (seeded N(0,1), quantised per the workload's KV format)",
        "config": cfg,
        "roofline": {"bound": "hbm", "kernel": "mla_split_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _measured_traffic(h.name), "avg_launch_us": round(split_us, 3),
                     "bytes_per_launch": h.kv_bytes},
        # the matrix unit is not the bound: stage 1's flop rate against its peak
        "mfma": mfma_block(mfma_flop(h.w), split_us),
        "plan_us": round(1e6 * h.t_plan, 1),
        "input_generation_s": round(h.t_gen, 2),
    }
    if args.copy_calibration_mb > 0:
        src = torch.empty(args.copy_calibration_mb << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = int(src.numel())
    w_head, bpr = h.w, h.kv_bytes / h.rows
    del h
    if not args.only_headline:
        import synth

        table = []
        # the five workloads, and the headline shape with several query rows per sequence
        for other, q_len in [(n, 1) for n in synth.WORKLOADS] + [(DEFAULT_WORKLOAD, 2), (DEFAULT_WORKLOAD, 4)]:
            t = Timed(other, args, threads, q_len)
            # about 50 ms of calls per workload, after 0.1 s untimed, so that
            # short calls are timed at the part's working clocks
            t.settle(0.1)
            probe = t.time(20, args.warmup) / 20
            steps = int(min(20000, max(args.steps, 0.05 / max(probe, 1e-7))))
            el = t.time(steps, 0)
            us = 1e6 * el / steps
            s1 = t.split_launch_us(min(steps, 2000))
            d = t.describe()
            row = {"workload": t.name, "q_len": q_len, "us_per_call": round(us, 2), "calls": steps,
                   "GBs": round(t.kv_bytes / (us * 1e-6) / 1e9, 1),
                   "frac_of_peak": round(t.kv_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "stage1_us": round(s1, 2), "stage1_frac_of_peak": round(t.kv_bytes / (s1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "stage1_mfma_frac": mfma_block(mfma_flop(t.w), s1)["frac"],
                   "kv_bytes": t.kv_bytes, "kv_copies_rotated": t.ncopy, "num_splits": d["num_splits"],
                   "rows_per_split": d["rows_per_split"], "stage2": d["stage2"]}
            if q_len == 1:
                ring = t.ring_read_us(min(steps, 200))
                if ring:
                    row["ring_read_us"] = round(ring, 2)
                    row["stage1_frac_of_ring_read"] = round(ring / s1, 4)
            if not args.no_cpu_baseline and q_len == 1:
                row["cpu_baseline"] = cpu_baseline(t.w, t.kv_bytes / t.rows, args.cpu_seconds)
            table.append(row)
            del t
            torch.cuda.empty_cache()
        res["workloads"] = table
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w_head, bpr, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
