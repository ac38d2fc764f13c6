"""Profiling helpers: a workload driver for rocprofv3 runs and summaries of rocprofv3's CSV output.

  python -m bit_gemv_decode_amd.profiling drive
      Runs, in one process: the stream-read kernel over a 2 GiB buffer (known bytes read), a 1 GiB
      fill (known bytes written), then one warm-up and one timed grouped BITCOS step over the
      Llama3-8B-shaped layer set (the same workload bench.py times).
  python -m bit_gemv_decode_amd.profiling stats STATS_CSV OUT.md "COMMAND" [TRACE_CSV SKIP COUNT]
      Writes a short markdown summary of a --kernel-trace --stats run (with TRACE_CSV, SKIP and COUNT,
      also the average of BITCOS dispatches SKIP .. SKIP + COUNT - 1: the timed region of a bench.py
      run is its dispatches WARMUP .. WARMUP + STEPS - 1).
  python -m bit_gemv_decode_amd.profiling traffic FETCH_CSV WRITE_CSV OUT.json "COMMANDS"
      From a --pmc FETCH_SIZE run and a --pmc WRITE_SIZE run of `drive`: calibrates both counters
      against the known-size kernels and converts the BITCOS dispatch's counts into HBM bytes.
  python -m bit_gemv_decode_amd.profiling counters OUT.md "COMMANDS" CSV [CSV ...]
      From --pmc runs of `drive` (one counter set each): the timed BITCOS dispatch's counters, per
      128-weight wave-group (one lane's group; 64 of them make a wave-step of 8192 weights) and as
      shares of the waves' resident cycles.
  python -m bit_gemv_decode_amd.profiling transient OUT.md [LAUNCHES]
      Launch by launch from an idle GPU: the grouped BITCOS and five-trit steps over the Llama3-8B
      layer set and a stream read of the same number of bytes, each after two idle seconds, with a
      clock probe (tg_clock_probe) between consecutive launches: per time window, the launches'
      average duration, their rate and the shader clock. Twice each, in rotated order.

The counters report KiB summed over the dispatch; the calibration factor is what the counter reads
for the known-size kernel divided by the bytes that kernel moves.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# the BITCOS kernel's source, the device headers it compiles from and the planner that divides its work
KERNEL_SRCS = [os.path.join(PKG, "csrc", f)
               for f in ("bitcos_gemv.hip", "bitcos_tables.h", "gemv_pipeline.h", "device_common.h",
                         "tg_internal.h", "api.cpp")]
READ_BYTES = 2 * 1024 ** 3
WRITE_BYTES = 1024 ** 3


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def drive():
    import torch

    sys.path.insert(0, ROOT)
    import bench
    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import binding as bd
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.empty(READ_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(cus * 4 * 4, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    bd.stream_read(buf, sink, cus * 4, 1)           # calibration: READ_BYTES read
    torch.cuda.synchronize()
    del buf
    w = torch.empty(WRITE_BYTES // 4, dtype=torch.int32, device=dev)
    w.fill_(3)                                       # calibration: WRITE_BYTES written
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()
    ls = bench.LayerSet(B, synth, torch, dev, B.FMT_BITCOS)
    plan = ls.plan(B)
    plan.run()
    torch.cuda.synchronize()
    plan.run()
    torch.cuda.synchronize()
    print(json.dumps({"step_bytes": ls.step_bytes}), flush=True)


def drive32b(warmup=3, launches=10):
    """The 32B-shaped stack (64 layers, hidden 5120, 6.0 GB of BITCOS) as one grouped launch: `warmup`
    launches, then `launches` more, for rocprofv3 kernel traces and counters of the row-walk build
    (wide lanes for its 5120-weight rows, the dead-row skip)."""
    import torch

    sys.path.insert(0, ROOT)
    import bench
    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    st, _ = bench.stack32b(B, synth, torch, dev)
    plan = st.plan(B)
    for _ in range(warmup + launches):
        plan.run()
    torch.cuda.synchronize()
    print(json.dumps({"step_bytes": st.step_bytes, "live_rows": plan.plan.live_rows}), flush=True)


def _curve(torch, bd, fn, launches, spin=100):
    """Durations (µs) of `launches` back-to-back calls of fn() from an idle GPU, and the shader clock
    (MHz) sampled before each of them and after the last."""
    import time

    dev = torch.device("cuda:0")
    buf = torch.zeros(4 * (launches + 1), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    time.sleep(2.0)
    for i in range(launches):
        bd.clock_probe(buf, i, spin)
        fn()
    bd.clock_probe(buf, launches, spin)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().reshape(-1, 4).astype("float64")
    dur = (b[1:, 0] - b[:-1, 2]) / 100.0  # from the end of one probe to the start of the next
    mhz = (b[:, 3] - b[:, 1]) / (b[:, 2] - b[:, 0]) * 100.0
    return dur, mhz


def transient(out_md, launches=300):
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import bench
    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import binding as bd
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lb = bench.LayerSet(B, synth, torch, dev, B.FMT_BITCOS)
    lt = bench.LayerSet(B, synth, torch, dev, B.FMT_5TRIT)
    pb, pt = lb.plan(B), lt.plan(B)
    sbuf = torch.empty(lb.step_bytes // 256 * 256, dtype=torch.uint8, device=dev)
    sbuf.fill_(1)
    sink = torch.empty(cus * 4 * 4, dtype=torch.int32, device=dev)
    work = {"BITCOS step": (pb.run, lb.step_bytes), "five-trit step": (pt.run, lt.step_bytes),
            "stream read": (lambda: bd.stream_read(sbuf, sink, cus * 4, 1), sbuf.numel())}
    windows = ((0, 1), (1, 3), (3, 6), (6, 10), (10, 15), (15, 20), (20, 30), (30, 40), (40, 60), (60, 80), (80, 120))
    res = {k: [] for k in work}
    names = list(work)
    for rep in range(2):
        for name in names[rep % 3:] + names[:rep % 3]:
            fn, nbytes = work[name]
            dur, mhz = _curve(torch, bd, fn, launches)
            t = np.cumsum(dur) / 1e3
            rows = []
            for lo, hi in windows:
                sel = (t > lo) & (t <= hi)
                if sel.any():
                    rows.append((f"{lo}-{hi}", int(sel.sum()), float(dur[sel].mean()), nbytes / float(dur[sel].mean()) / 1e3,
                                 float(mhz[1:][sel].mean())))
            res[name].append(rows)
            print(json.dumps({"transient": name, "rep": rep, "rows": rows}), flush=True)
    lines = [f"# Launch-by-launch rate and shader clock from an idle GPU: `{os.path.basename(out_md)}`", "",
             "Command (from the repository root):", "",
             f"    python3 -m bit_gemv_decode_amd.profiling transient {os.path.relpath(out_md, ROOT)} {launches}", "",
             "Each workload starts after two idle seconds and runs back to back; a one-wave clock probe between "
             "consecutive launches timestamps them and samples the shader clock (s_memtime against the 100 MHz "
             "s_memrealtime). Windows are milliseconds since the first launch.", ""]
    for name in names:
        for rep, rows in enumerate(res[name]):
            lines += [f"## {name}, run {rep + 1}", "", "| Window (ms) | Launches | µs per launch | GB/s | Shader clock (MHz) |",
                      "|---|---|---|---|---|"]
            lines += [f"| {w} | {n} | {d:.1f} | {g:.0f} | {c:.0f} |" for w, n, d, g, c in rows]
            lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def stats(stats_csv, out_md, command, trace_csv=None, skip=0, count=0):
    rows = _rows(stats_csv)
    lines = [f"# Kernel durations: `{os.path.basename(out_md)}`", "", "Command (from the repository root):", "",
             f"    {command}", "", "| Kernel | Calls | Average (µs) | Min (µs) | Max (µs) | Share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    if trace_csv and count:
        # the timed region of bench.py: BITCOS dispatches skip .. skip + count - 1
        tr = [r for r in _rows(trace_csv) if "bitcos_gemv_kernel" in r["Kernel_Name"]]
        tr.sort(key=lambda r: int(r["Start_Timestamp"]))
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr[skip:skip + count]]
        if d:
            lines += ["", f"Timed region (BITCOS dispatches {skip} .. {skip + len(d) - 1}, after {skip} warm-up ones): "
                          f"average {sum(d) / len(d):.2f} µs, min {min(d):.2f}, max {max(d):.2f}; "
                          f"all {len(tr)} BITCOS dispatches of the run (warm-up, timed, then the settled-rate "
                          f"launches): average {sum((int(r['End_Timestamp']) - int(r['Start_Timestamp'])) / 1e3 for r in tr) / len(tr):.2f} µs."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(out_md, command, csvs, workload="layerset"):
    """Summary of the last BITCOS dispatch of `drive` (the timed step; workload "layerset") or of
    `drive32b` (workload "stack32b") over one or more --pmc runs."""
    sys.path.insert(0, ROOT)
    import bench

    vals = {}
    for path in csvs:
        rows = _rows(path)
        ds = sorted({int(r["Dispatch_Id"]) for r in rows if "bitcos_gemv_kernel" in r["Kernel_Name"]})
        if not ds:
            continue
        last = ds[-1]
        for r in rows:
            if int(r["Dispatch_Id"]) == last:
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if workload == "stack32b":
        weights = bench.STACK32B_LAYERS * sum(n * k for _, n, k in bench.STACK32B)
        what = f"`drive32b` (the 32B-shaped stack x{bench.STACK32B_LAYERS}"
    else:
        weights = bench.LAYERS * sum(n * k for _, n, k in bench.LAYER)
        what = f"`drive` (the Llama3-8B-shaped layer set x{bench.LAYERS}"
    wave_steps = weights / 8192.0  # 64 lanes x 128 weights
    lines = [f"# SQ counters of the grouped BITCOS step: `{os.path.basename(out_md)}`", "",
             "Commands (from the repository root):", "", f"    {command}", "",
             f"Timed dispatch of {what}, {weights / 1e9:.2f} G weights, "
             f"{wave_steps:.0f} wave-steps of 8192 weights).", "", "| Counter | Total | Per wave-step |", "|---|---|---|"]
    for name in sorted(vals):
        lines.append(f"| `{name}` | {vals[name]:.4g} | {vals[name] / wave_steps:.2f} |")
    wc = vals.get("SQ_WAVE_CYCLES")
    if wc:
        lines += ["", "Shares of the waves' resident cycles (`SQ_WAVE_CYCLES`):", ""]
        for name in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS",
                     "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY"):
            if name in vals:
                lines.append(f"- `{name}`: {100 * vals[name] / wc:.1f} %")
    if vals.get("SQ_INSTS_LDS") and vals.get("SQ_LDS_BANK_CONFLICT"):
        lines.append(f"- bank-conflict cycles per LDS instruction: "
                     f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_INSTS_LDS']:.2f}")
    if wc and vals.get("SQ_ACTIVE_INST_VALU") and vals.get("SQ_WAVES"):
        # 256 CUs x 4 SIMDs; the waves of the launch are resident together (one block per CU)
        per_simd = vals["SQ_WAVES"] / (256 * 4)
        lines += ["", "Reading: `SQ_WAVE_CYCLES` and `SQ_ACTIVE_INST_*` count quad-cycles summed over waves, and "
                  "each VALU instruction holds its SIMD for one (`SQ_ACTIVE_INST_VALU` = `SQ_INSTS_VALU`: "
                  f"{vals['SQ_ACTIVE_INST_VALU'] / wave_steps:.1f} against "
                  f"{vals.get('SQ_INSTS_VALU', float('nan')) / wave_steps:.1f} per wave-step). With "
                  f"{per_simd:.0f} waves per SIMD, the SIMD's VALU is busy about {per_simd:.0f} x "
                  f"{100 * vals['SQ_ACTIVE_INST_VALU'] / wc:.1f} % = "
                  f"{100 * per_simd * vals['SQ_ACTIVE_INST_VALU'] / wc:.0f} % of the dispatch: the step is bound by "
                  "VALU issue, and one wave's waits are filled by the other waves of its SIMD."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(path, counter):
    agg = defaultdict(float)
    names = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        agg[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(d, names[d], agg[d]) for d in sorted(agg)]


def traffic(fetch_csv, write_csv, out_json, command):
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    pick = lambda rows, key: [r for r in rows if key in r[1]]
    f_cal = pick(fetch, "stream_read")[-1][2] * 1024 / READ_BYTES
    w_cal = pick(write, "FillFunctor<int>")[-1][2] * 1024 / WRITE_BYTES
    f_k = pick(fetch, "bitcos_gemv_kernel")[-1][2] * 1024 / f_cal
    w_k = pick(write, "bitcos_gemv_kernel")[-1][2] * 1024 / w_cal
    out = {"kernel": "bitcos_gemv_kernel (grouped step over the Llama3-8B-shaped layer set x32)",
           "kernel_source_sha256_16": kernel_source_hash(),
           "fetch_calibration": round(f_cal, 5), "write_calibration": round(w_cal, 5),
           "hbm_read_bytes_per_launch": int(f_k), "hbm_write_bytes_per_launch": int(w_k),
           "bytes_per_launch": int(f_k + w_k), "commands": command}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "drive":
        drive()
    elif cmd == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4], *(sys.argv[5:6]), *(int(a) for a in sys.argv[6:8]))
    elif cmd == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif cmd == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif cmd == "counters32b":
        counters(sys.argv[2], sys.argv[3], sys.argv[4:], workload="stack32b")
    elif cmd == "drive32b":
        drive32b()
    elif cmd == "transient":
        transient(sys.argv[2], *(int(a) for a in sys.argv[3:4]))
    else:
        raise SystemExit(f"unknown command {cmd}")
