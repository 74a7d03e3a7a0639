"""Where the time of a stage-1 launch goes, per workgroup (a measurement aid).

Runs the measurement build of the library (built beforehand on the host with
``python3 -c "from mla_decode_split_amd import build; build.build_trace()"``)
on a synthetic workload, resident in HBM and rotated over >= 768 MB of KV
copies as in bench.py, and reads back each stage-1 workgroup's start, first
tile and end (mla_debug_wg_trace).  Six traced calls, each after ten untimed
ones; it prints the percentiles of the call whose last workgroup ends at the
median, the end times per XCD in every call, and the end times by a
workgroup's age on its CU (the order in which the CU's workgroups started).

    python3 -m mla_decode_split_amd.wg_trace [--out DIR] WORKLOAD [WORKLOAD ...]
"""
from __future__ import annotations

import argparse
import math
import os

import numpy as np


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("workloads", nargs="*", default=["bs64_kv8192_fp8"])
    ap.add_argument("--calls", type=int, default=6)
    ap.add_argument("--out", default=None, help="directory for one .npz of timelines per workload")
    args = ap.parse_args(argv)

    from . import build
    import mla_decode_split_amd as mla

    if not os.path.exists(build.LIB_TRACE):
        raise SystemExit(f"{build.LIB_TRACE} is not built: run build.build_trace() on the host first")
    mla.LIB_PATH = build.LIB_TRACE
    import torch
    import synth
    from . import device as dev

    torch.cuda.set_device(0)
    for name in args.workloads:
        w = synth.make_workload(name)
        b = dev.upload(w)
        plan = dev.plan_for(b)
        d = mla.mla_decode_plan_describe(plan)
        G = d["num_splits"]
        if G > 8192:
            raise SystemExit(f"{name}: {G} workgroups, the timeline holds 8192")
        ws = dev.workspace_for(plan)
        out = torch.empty((b.total_q, 16, 512), dtype=torch.bfloat16, device="cuda")
        ncopy = max(1, math.ceil(768e6 / max(w.kv_bytes(), 1)))
        kvs = [b.kv] + [b.kv.clone() for _ in range(ncopy - 1)]
        runs = []
        for call in range(args.calls):
            for i in range(10):  # untimed calls: clocks settle, the traced copy is not in cache
                b.kv = kvs[i % ncopy]
                dev.run_split(plan, b, out, ws)
            torch.cuda.synchronize()
            mla.mla_debug_wg_trace(None, clear=True)
            b.kv = kvs[(call + 3) % ncopy]
            dev.run_split(plan, b, out, ws)
            torch.cuda.synchronize()
            buf = np.zeros(4 * G, dtype=np.uint64)
            mla.mla_debug_wg_trace(buf)
            t = buf.reshape(G, 4).astype(np.int64)
            live = t[:, 0] > 0  # workgroups that own rows
            t0 = t[live, 0].min()
            us = lambda col: (t[:, col] - t0) / 100.0  # 100 MHz counter
            hw = t[:, 3] >> 8
            runs.append(dict(live=live, start=us(0), first=us(1), end=us(2), xcc=t[:, 3] & 0xF,
                             cu=(hw >> 8) & 0xF, se=(hw >> 13) & 0x7))
        print(f"== {name}: {G} workgroups, rows per range {d['rows_per_split']}"
              f"{'/' + str(d['second_rows_per_split']) if d['paired_splits'] else ''}")
        for i, r in enumerate(runs):
            lv = r["live"]
            print(f"   call {i}: last end {r['end'][lv].max():6.1f} us; mean end per XCD "
                  + " ".join(f"{r['end'][lv & (r['xcc'] == x)].mean():5.1f}" for x in range(8)
                             if (lv & (r['xcc'] == x)).any()))
        order = np.argsort([r["end"][r["live"]].max() for r in runs])
        r = runs[order[len(order) // 2]]
        lv = r["live"]
        pct = lambda a: " ".join(f"{v:6.1f}" for v in np.percentile(a[lv], [0, 10, 50, 90, 100]))
        print("  median call, us after the first start (p0 / p10 / p50 / p90 / p100):")
        print(f"    start      {pct(r['start'])}")
        print(f"    first tile {pct(r['first'])}")
        print(f"    end        {pct(r['end'])}")
        for x in range(8):
            m = lv & (r["xcc"] == x)
            if m.any():
                print(f"    XCD {x}: {m.sum():3d} workgroups, end min / median / max "
                      f"{r['end'][m].min():6.1f} {np.median(r['end'][m]):6.1f} {r['end'][m].max():6.1f}")
        key = r["xcc"] * 1000 + r["se"] * 100 + r["cu"]
        cus = {}
        for g in np.nonzero(lv)[0]:
            cus.setdefault(int(key[g]), []).append(int(g))
        by_age = {}
        for gs in cus.values():
            gs.sort(key=lambda g: r["start"][g])
            for a, g in enumerate(gs):
                by_age.setdefault((len(gs), a), []).append(g)
        for (k, a), gs in sorted(by_age.items()):
            e = r["end"][gs]
            print(f"    CUs with {k} workgroups, age {a}: {len(gs):3d}, end p10 / p50 / p90 "
                  + " ".join(f"{v:.1f}" for v in np.percentile(e, [10, 50, 90])))
        if args.out:
            os.makedirs(args.out, exist_ok=True)
            np.savez(os.path.join(args.out, f"wg_trace_{name}.npz"),
                     **{f"{k}_{i}": v for i, run in enumerate(runs) for k, v in run.items()})


if __name__ == "__main__":
    main()
