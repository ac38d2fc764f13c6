"""Benchmark: ternary GEMV effective HBM bandwidth on MI355X (one GPU).

Workload (default): the Llama3-8B-shaped decode layer set at batch 1 -- q, o 4096x4096; k, v
1024x4096; gate, up 14336x4096; down 4096x14336 -- iid ternary weights at zero density 0.40,
group-128 fp16 scales, int8 activations, seed 0. The layer is replicated 32 times (Llama3-8B depth)
so the 1.5 GB BITCOS working set is far larger than the 256 MB Infinity Cache and every byte comes
from HBM. One step = one pass over the 32 layers x 7 GEMVs in BITCOS. `value` is packed bytes read
per second (bitmap + signs + sign index + fp16 scales), whole job. The five-trit and 2-bit formats
are timed on the same layer set for comparison.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
REPLICAS = 32
Z = 0.40


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_layer(B, synth, dev, fmt):
    """Pack the 7 matrices of one layer in `fmt`; returns per-matrix device weights, scales, x, y."""
    import torch

    mats = []
    for role, (name, n, k) in enumerate(LAYER):
        w = synth.ternary(n, k, Z, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        s = synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))
        x = synth.activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_X))
        p = B.pack(fmt, w)
        mats.append(dict(name=name, n=n, k=k, packed=p, w=w, s=s,
                         dw=B.DeviceWeights(p, dev), st=torch.from_numpy(s).to(dev),
                         xt=torch.from_numpy(x).to(dev), y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    return mats


def replicate(B, mats):
    """REPLICAS copies of every matrix's packed buffer and scales (distinct HBM addresses)."""
    reps = []
    for r in range(REPLICAS):
        layer = []
        for m in mats:
            dw = B.DeviceWeights.from_tensor(m["dw"].desc, m["dw"].tensor.clone())
            layer.append(dict(m, dw=dw, st=m["st"].clone()))
        reps.append(layer)
    return reps


def packed_bytes(m):
    """Algorithmic bytes one GEMV reads: packed payload plus the fp16 scales."""
    return m["dw"].payload_bytes + 2 * m["n"] * (m["k"] // 128)


def run_pass(B, reps, stream):
    for layer in reps:
        for m in layer:
            B.ternary_gemv(m["dw"], m["st"], m["xt"], m["y"], stream=stream)


def time_steps(B, reps, steps, warmup, stream):
    import torch

    for _ in range(warmup):
        run_pass(B, reps, stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        run_pass(B, reps, stream)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def per_matrix_us(B, mats, stream, iters=50):
    """Median event-timed duration of each matrix's GEMV (cycling over fresh replicas is not needed for
    the per-call figure, so this one is L2/MALL-warm and is reported separately)."""
    import torch

    out = {}
    for m in mats:
        ts = []
        for _ in range(iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            B.ternary_gemv(m["dw"], m["st"], m["xt"], m["y"], stream=stream)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        out[m["name"]] = float(np.median(ts))
    return out


def cpu_baseline(O, mats, budget_s=12.0):
    """The oracle decoding BITCOS rows from packed bytes on the host cores, over the whole layer set."""
    total_bytes = sum(packed_bytes(m) for m in mats)
    times = []
    t_all = time.time()
    while True:
        t0 = time.perf_counter()
        for m in mats:
            p = m["packed"]
            O.gemv_packed(O.FMT_BITCOS, p.section("codes"), p.sign_bytes(), p.rowoff(), m["s"], m["n"], m["k"],
                          m["xt"].cpu().numpy())
        times.append(time.perf_counter() - t0)
        if time.time() - t_all > budget_s or len(times) >= 5:
            break
    t = float(np.median(times))
    return dict(value=total_bytes / t / 1e9, unit="GB/s", cores=O.threads(), kind="oracle",
                sample=f"one Llama3-8B-shaped layer set (7 GEMVs, {total_bytes / 1e6:.1f} MB BITCOS), median of "
                       f"{len(times)} passes, {t * 1e3:.0f} ms per pass", seconds_per_pass=t)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--formats", default="bitcos,5trit,2bit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the ternary GEMV is sharded by rows or by K across GPUs in a "
              "deployment, but this build runs on a single MI355X; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    fmt_ids = {"bitcos": B.FMT_BITCOS, "5trit": B.FMT_5TRIT, "2bit": B.FMT_2BIT}
    results = {}
    bitcos_mats = None
    for fname in args.formats.split(","):
        fmt = fmt_ids[fname]
        log(f"[bench] packing the layer set as {fname}")
        mats = make_layer(B, synth, dev, fmt)
        reps = replicate(B, mats)
        step_bytes = REPLICAS * sum(packed_bytes(m) for m in mats)
        steps = args.steps if fmt == B.FMT_BITCOS else max(5, args.steps // 5)
        log(f"[bench] {fname}: {step_bytes / 1e9:.3f} GB per step, {steps} steps")
        secs = time_steps(B, reps, steps, args.warmup if fmt == B.FMT_BITCOS else 3, stream)
        per_call = per_matrix_us(B, mats, stream)
        results[fname] = dict(gbs=step_bytes * steps / secs / 1e9, ms_per_step=secs / steps * 1e3,
                              step_bytes=step_bytes, steps=steps, launches_per_step=REPLICAS * len(mats),
                              per_matrix_us_warm=per_call,
                              layer_bytes={m["name"]: packed_bytes(m) for m in mats})
        log(f"[bench] {fname}: {results[fname]['gbs']:.1f} GB/s, {results[fname]['ms_per_step']:.3f} ms/step")
        if fmt == B.FMT_BITCOS:
            bitcos_mats = mats
        del reps
        if fmt != B.FMT_BITCOS:
            del mats
        torch.cuda.empty_cache()

    bc = results["bitcos"]
    launches = bc["launches_per_step"] * bc["steps"]
    avg_launch_s = bc["ms_per_step"] / 1e3 / bc["launches_per_step"]
    avg_launch_bytes = bc["step_bytes"] / bc["launches_per_step"]
    achieved = avg_launch_bytes / avg_launch_s / 1e9
    out = {
        "metric": "ternary GEMV effective HBM GB/s (packed bytes/s) + % of MI355X peak, us/call",
        "value": round(bc["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(bc["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded iid ternary z=0.40, fp16 scales U[0.01,0.1], int8 x U[-127,127])",
        "config": {"workload": "Llama3-8B-shaped decode layer set, batch 1, BITCOS, x32 layer replicas",
                   "matrices": {n: [r, c] for n, r, c in LAYER}, "zero_density": Z, "group": 128,
                   "replicas": REPLICAS, "format": "bitcos"},
        "pct_of_hbm_peak": round(100 * bc["gbs"] / HBM_PEAK_GBS, 2),
        "us_per_layer": round(bc["ms_per_step"] * 1e3 / REPLICAS, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "bitcos_gemv_valu<1,false>", "launches": launches,
                     "avg_launch_us": round(avg_launch_s * 1e6, 3), "avg_launch_bytes": int(avg_launch_bytes)},
        "formats": {f: {"gbs": round(r["gbs"], 2), "ms_per_step": round(r["ms_per_step"], 4),
                        "step_bytes": r["step_bytes"], "per_matrix_us_warm": {k: round(v, 3) for k, v in
                                                                              r["per_matrix_us_warm"].items()}}
                    for f, r in results.items()},
    }
    if "5trit" in results:
        out["bitcos_vs_5trit_time"] = round(results["5trit"]["ms_per_step"] / bc["ms_per_step"], 4)
        out["5trit_vs_bitcos_bytes"] = round(results["5trit"]["step_bytes"] / bc["step_bytes"], 4)
    if "2bit" in results:
        out["bitcos_vs_2bit_time"] = round(results["2bit"]["ms_per_step"] / bc["ms_per_step"], 4)
        out["2bit_vs_bitcos_bytes"] = round(results["2bit"]["step_bytes"] / bc["step_bytes"], 4)
    if not args.no_cpu:
        import oracle as O

        log("[bench] timing the CPU oracle baseline")
        cb = cpu_baseline(O, bitcos_mats)
        out["cpu_baseline"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in cb.items()}
        out["gpu_vs_cpu"] = round(bc["gbs"] / cb["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
