"""Benchmark: ternary GEMV effective HBM bandwidth on MI355X (one GPU).

Workload: the Llama3-8B-shaped decode layer set at batch 1 -- q, o 4096x4096; k, v 1024x4096;
gate, up 14336x4096; down 4096x14336 -- iid ternary weights at zero density 0.40, group-128 fp16
scales, int8 activations, seed 0. Each matrix is stored 32 times (one copy per layer of a 32-layer
model), so the 1.51 GB of BITCOS weights are far larger than the 256 MB Infinity Cache and every
byte comes from HBM. One step = one pass over the 32 x 7 = 224 GEMVs, issued as one grouped launch
(tg_plan_init / ternary_gemv_plan). `value` is packed bytes read per second (bitmap + sign stream +
sign index + fp16 scales), whole job.

Also measured and reported beside it (same process): the same pass as 32 per-layer launches and as
224 single-GEMV launches (captured in a HIP graph), each matrix's single-call time, the pass on
float activations quantised per group (quantiser time per call, grouped GEMV with activation group
scales), the five-trit, 2-bit and t5b formats on the same layer set (each fixed code also with its
table-free decode), the same launch with its weights in the Infinity Cache and a 2560x2560 matrix
referenced 768 times from L2 (the decode's own rate), the stream-read ceiling of this GPU, and the CPU
oracle.

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

from bit_gemv_decode_amd.binding import FMT_T5B  # noqa: E402  (numpy and ctypes only)

HBM_PEAK_GBS = 8000.0
SETTLE_MS = 60.0  # GPU time of back-to-back launches before a sustained-rate measurement
LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LAYERS = 32
Z = 0.40
T5B_SCALE = 0.05  # the per-tensor scale of t5b matrices (the other formats draw per-group scales)
METRIC = "ternary GEMV effective HBM GB/s (packed bytes/s) + % of MI355X peak, µs/call"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bitcos_layerset.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    from bit_gemv_decode_amd.profiling import kernel_source_hash as h
    return h()


class LayerSet:
    """Matrices of one decoder layer packed in `fmt`, stored `layers` times in device memory.

    shapes: (name, n, k) per matrix role; z: zero density; dead: row indices that are all zero in the
    roles named in dead_roles (the same indices in each, as in the 32B-shaped stack)."""

    def __init__(self, B, synth, torch, dev, fmt, layers=LAYERS, shapes=None, z=Z, dead=None,
                 dead_roles=("gate", "up")):
        self.fmt = fmt
        self.shapes = list(shapes) if shapes is not None else list(LAYER)
        self.layers = layers
        self.mats = []      # per layer copy: list of dict(w=DeviceWeights, s, x, y)
        self.host = []      # one host copy per matrix role (for the CPU baseline)
        base = []
        for role, (name, n, k) in enumerate(self.shapes):
            w = synth.ternary(n, k, z, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
            if dead is not None and name in dead_roles:
                w[dead] = 0
            s = synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))
            x = synth.activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_X))
            # t5b carries one scale per tensor instead of per-group scales
            p = B.pack_t5b(w, T5B_SCALE) if fmt == B.FMT_T5B else B.pack(fmt, w)
            self.host.append(dict(name=name, n=n, k=k, packed=p, s=s, x=x))
            base.append((B.DeviceWeights(p, dev), torch.from_numpy(s).to(dev), torch.from_numpy(x).to(dev)))
            del w
        for layer in range(layers):
            row = []
            for (dw, s, x), (name, n, k) in zip(base, self.shapes):
                t = dw.tensor if layer == 0 else dw.tensor.clone()
                row.append(dict(name=name, w=B.DeviceWeights.from_tensor(dw.desc, t), s=s if layer == 0 else s.clone(),
                                x=x, y=torch.empty((1, n), dtype=torch.float32, device=dev)))
            self.mats.append(row)
        self.layer_bytes = [packed_bytes(m["w"]) for m in self.mats[0]]
        self.step_bytes = layers * sum(self.layer_bytes)

    def flat(self):
        return [m for row in self.mats for m in row]

    def plan(self, B, mats=None):
        mats = mats if mats is not None else self.flat()
        return B.Plan([m["w"] for m in mats], [m["x"] for m in mats],
                      scales=None if self.fmt == B.FMT_T5B else [m["s"] for m in mats], ys=[m["y"] for m in mats])


# The 32B-shaped dense decoder: 64 layers, hidden 5120, FFN 25600, GQA k/v 1024 rows, z = 0.47, and
# 4.76 % of FFN neurons (1219 of 25600) all-zero at the same indices in gate and up ("Sub-Two-Bit
# Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract: dead FFN neurons).
STACK32B = [("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
            ("gate", 25600, 5120), ("up", 25600, 5120), ("down", 5120, 25600)]
STACK32B_LAYERS = 64
STACK32B_Z = 0.47
STACK32B_DEAD = 1219


def stack32b(B, synth, torch, dev, layers=STACK32B_LAYERS):
    """The 32B-shaped stack in BITCOS: one layer generated and stored `layers` times (6.08 GB for 64)."""
    dead = synth.dead_rows(25600, STACK32B_DEAD, seed=0)
    return LayerSet(B, synth, torch, dev, B.FMT_BITCOS, layers=layers, shapes=STACK32B, z=STACK32B_Z, dead=dead), dead


def time_launches(torch, fn, steps, warmup):
    """Run fn() warmup times, then time `steps` calls with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(steps):
        fn()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3  # seconds


def settle(torch, fn, ms=SETTLE_MS):
    """Launch fn() until about `ms` of GPU time has passed, so that the timed launches that follow run
    at the sustained rate, past the power transient of the first back-to-back launches."""
    cur = torch.cuda.current_stream()
    spent, batch = 0.0, 1
    while spent < ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(batch):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        batch = min(batch * 2, 64)


def stream_ceiling(torch, bd, dev):
    """Best rate of the stream-read reference kernel over a 2 GiB buffer (a few launch shapes)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 2 * 1024 ** 3
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(cus * 8 * 4, dtype=torch.int32, device=dev)
    best = 0.0
    for bpc, unroll in ((4, 1), (2, 4), (8, 1), (1, 8)):
        secs = time_launches(torch, lambda: bd.stream_read(buf, sink, cus * bpc, unroll), 5, 1)
        best = max(best, nbytes * 5 / secs / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def cpu_model():
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout.splitlines()
        return [l.split(":", 1)[1].strip() for l in out if l.startswith("Model name")][0]
    except Exception:
        return "unknown"


def cpu_baseline(O, ls, budget_s=12.0, one_core_budget_s=8.0):
    """The oracle decoding BITCOS rows from packed bytes on the host cores, over one layer set: on
    every core it may use (`value`, `cores`), and on one core."""
    total_bytes = sum(ls.layer_bytes)

    def passes(budget, most):
        times = []
        t_all = time.time()
        while True:
            t0 = time.perf_counter()
            for h in ls.host:
                p = h["packed"]
                O.gemv_packed(O.FMT_BITCOS, p.section("codes"), p.sign_bytes(), p.rowoff(), h["s"], h["n"], h["k"],
                              h["x"])
            times.append(time.perf_counter() - t0)
            if time.time() - t_all > budget or len(times) >= most:
                return float(np.median(times)), len(times)

    cores = len(os.sched_getaffinity(0))
    t, n = passes(budget_s, 7)
    used = int(O.threads())
    O.set_threads(1)
    t1, n1 = passes(one_core_budget_s, 3)
    O.set_threads(used)
    return dict(value=round(total_bytes / t / 1e9, 4), unit="GB/s", cores=used, kind="oracle",
                sample=f"one layer set (the 7 GEMVs, {total_bytes / 1e6:.1f} MB BITCOS, ~1/32 of a step), "
                       f"median of {n} passes, {t * 1e3:.1f} ms per pass",
                one_core={"value": round(total_bytes / t1 / 1e9, 4), "unit": "GB/s",
                          "ms_per_pass": round(t1 * 1e3, 1), "passes": n1},
                cpu_model=cpu_model(), cores_available=cores)


CACHE_FIT_BYTES = 200e6  # distinct weight bytes kept well inside the 256 MB Infinity Cache


def cache_resident(torch, B, ls, launches=60, decode=None):
    """The step's own launch (all LAYERS x 7 GEMVs, same plan shape) with its weights taken from the
    first few layer copies only (as many as fit CACHE_FIT_BYTES: 4 of BITCOS, 189 MB), each referenced
    in turn, so after SETTLE_MS of the same launches the weights come from the Infinity Cache instead
    of HBM. The rate (algorithmic bytes of the 224 GEMVs per second) is the decode's own rate at the
    step's launch shape. (Repeated GEMVs write the same outputs with the same values.)"""
    distinct = max(1, min(4, int(CACHE_FIT_BYTES // sum(ls.layer_bytes))))
    mats = [m for layer in range(ls.layers) for m in ls.mats[layer % distinct]]
    p = ls.plan(B, mats)
    if decode is not None:
        p.set_decode(decode)
    settle(torch, p.run)
    s = time_launches(torch, p.run, launches, 0) / launches
    res = {"copies": distinct, "distinct_mb": round(distinct * sum(ls.layer_bytes) / 1e6, 1), "us_per_launch": round(s * 1e6, 2),
           "gbs": round(ls.step_bytes / s / 1e9, 1)}
    del p
    return res


L2_SHAPE, L2_Z, L2_REFS = (2560, 2560), 0.42, 768


def l2_resident(torch, B, synth, dev, launches=40):
    """The decode rate with the matrix in L2: one 2560x2560 matrix (z = 0.42: 1.41 MB of BITCOS), referenced
    768 times in one grouped launch with one output. Consecutive wave ranges share an XCD, so each XCD's
    4 MB L2 holds the whole matrix after its first read and serves the other references; the rate is the
    768 references' algorithmic bytes per second after SETTLE_MS of the same launches. BITCOS, five-trit and
    2-bit (the fixed codes with their LDS table and table-free)."""
    n, k = L2_SHAPE
    w = synth.ternary(n, k, L2_Z, seed=0)
    s = torch.from_numpy(synth.scales(n, k // 128, seed=0)).to(dev)
    x = torch.from_numpy(synth.activations(1, k, seed=0)).to(dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    out = {"shape": [n, k], "z": L2_Z, "references": L2_REFS}
    for fname, fmt in (("bitcos", B.FMT_BITCOS), ("5trit", B.FMT_5TRIT), ("2bit", B.FMT_2BIT)):
        dw = B.DeviceWeights(B.pack(fmt, w), dev)
        for decode in ((None,) if fmt == B.FMT_BITCOS else (B.DECODE_BYTE, B.DECODE_ARITH)):
            p = B.Plan([dw] * L2_REFS, [x] * L2_REFS, scales=[s] * L2_REFS, ys=[y] * L2_REFS)
            if decode is not None:
                p.set_decode(decode)
            settle(torch, p.run)
            secs = time_launches(torch, p.run, launches, 0) / launches
            key = f"{fname}_table_free" if decode == B.DECODE_ARITH else fname
            out[key] = {"mb": round(packed_bytes(dw) / 1e6, 3), "us_per_launch": round(secs * 1e6, 2),
                        "gbs": round(L2_REFS * packed_bytes(dw) / secs / 1e9, 1)}
            del p
        del dw
    return out


def activation_quant(torch, B, synth, ls, dev, steps, warmup):
    """The same layer set on float activations quantised per group of 128: the quantiser's time per
    call (graph-replayed, host launch path removed) and the grouped step of the GEMV with activation
    group scales over the quantised rows (one quantised row per matrix role, shared by its 32 copies)."""
    xq, xsc = [], []
    for role, (name, n, k) in enumerate(LAYER):
        xf = synth.float_activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_XF))
        q, sc = B.quantize_x(torch.from_numpy(xf).to(dev))
        xq.append(q)
        xsc.append(sc)
    mats = [(role, m) for row in ls.mats for role, m in enumerate(row)]
    plan = B.Plan([m["w"] for _, m in mats], [xq[r] for r, _ in mats], scales=[m["s"] for _, m in mats],
                  ys=[m["y"] for _, m in mats], x_scales=[xsc[r] for r, _ in mats])
    secs = time_launches(torch, plan.run, steps, warmup)
    step_s = secs / steps
    out = {"gemv_xs_grouped": {"gbs": round(ls.step_bytes / step_s / 1e9, 1), "ms_per_step": round(step_s * 1e3, 4)}}
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    for m, k in ((1, 4096), (1, 14336), (16, 14336)):
        xf = torch.from_numpy(synth.float_activations(m, k, seed=1)).to(dev)
        q = torch.empty((m, k), dtype=torch.int8, device=dev)
        sc = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for _ in range(32):
                B.quantize_x(xf, q, sc, stream=st)
        t = time_launches(torch, g.replay, 5, 1)
        out[f"quantize_m{m}_k{k}_us"] = round(t / (5 * 32) * 1e6, 3)
        del g
    del plan
    return out


def fp16_activations(torch, B, synth, ls, dev, steps, warmup):
    """The BITCOS layer set against fp16 activations: the grouped step (tg_plan_init_f16, one launch for
    the 224 GEMVs, one fp16 row per matrix role) and single calls (ternary_gemv_f16; one launch per
    GEMV, replayed from a graph that cycles through the 32 copies of each matrix)."""
    x16s = []
    for role, (name, n, k) in enumerate(LAYER):
        xf = synth.float_activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_XF))
        x16s.append(torch.from_numpy(xf.astype(np.float16)).to(dev))
    mats = [(role, m) for row in ls.mats for role, m in enumerate(row)]
    plan = B.Plan([m["w"] for _, m in mats], [x16s[r] for r, _ in mats], scales=[m["s"] for _, m in mats],
                  ys=[m["y"] for _, m in mats], f16=True)
    step_s = time_launches(torch, plan.run, steps, warmup) / steps
    out = {"grouped_one_launch": {"gbs": round(ls.step_bytes / step_s / 1e9, 1),
                                  "ms_per_step": round(step_s * 1e3, 4)}}
    del plan
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    total_us = 0.0
    for role, (name, n, k) in enumerate(LAYER):
        x16 = x16s[role]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for row in ls.mats:
                m = row[role]
                B.ternary_gemv_f16(m["w"], m["s"], x16, m["y"], stream=st)
        us = time_launches(torch, g.replay, 5, 1) / (5 * LAYERS) * 1e6
        total_us += us * LAYERS
        out[name] = {"us_per_call": round(us, 3), "gbs": round(ls.layer_bytes[role] / us / 1e3, 1)}
        del g
    out["layer_set_per_gemv_graph"] = {"gbs": round(ls.step_bytes / total_us / 1e3, 1),
                                       "ms_per_step": round(total_us / 1e3, 3)}
    return out


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 --pmc runs, if they match this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t


# ----- measurement suite: every configuration of the workload table, beside the headline step -----

def replicas(B, dw0, count):
    """`count` device copies of one packed matrix (distinct memory, same bytes)."""
    return [dw0] + [B.DeviceWeights.from_tensor(dw0.desc, dw0.tensor.clone()) for _ in range(count - 1)]


def packed_bytes(dw):
    """Algorithmic bytes of one packed matrix: its payload plus its scales (fp16 per 128-group, or
    the 4-byte tensor scale of t5b)."""
    if dw.fmt == FMT_T5B:
        return dw.payload_bytes + 4
    return dw.payload_bytes + 2 * dw.n * (dw.k // 128)


def per_call_us(torch, calls, warmup=10):
    """Eager launches of calls() (a list of thunks); one HIP event between consecutive launches, so
    each duration includes its launch gap. Returns median, p10, p90 in microseconds."""
    for f in calls[:warmup]:
        f()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    ev[0].record()
    for i, f in enumerate(calls):
        f()
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(len(calls))])
    return {"median_us": round(float(np.median(d)), 3), "p10_us": round(float(np.percentile(d, 10)), 3),
            "p90_us": round(float(np.percentile(d, 90)), 3), "calls": len(calls)}


def graph_call_us(torch, calls, reps=5):
    """The same calls captured in one HIP graph and replayed: microseconds per call with the host
    launch path removed (kernel time plus the gap between consecutive graph nodes)."""
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        for f in calls:
            f()
    settle(torch, g.replay, ms=20.0)
    secs = time_launches(torch, g.replay, reps, 0)
    del g
    return round(secs / (reps * len(calls)) * 1e6, 3)


PATHS = {0: "vector", 1: "matrix-core", 2: "fp16 vector", 3: "fp16 matrix-core", 4: "vector, 12 waves"}


def sustained(torch, B, dws, xs, ss, ys, launches=5, f16=False):
    """One grouped launch over all GEMVs: packed bytes per second and ms per launch (f16: fp16
    activations)."""
    plan = B.Plan(dws, xs, scales=ss, ys=ys, f16=f16)
    settle(torch, plan.run)
    secs = time_launches(torch, plan.run, launches, 0)
    total = sum(packed_bytes(d) for d in dws)
    return {"gbs": round(total * launches / secs / 1e9, 1), "ms_per_launch": round(secs / launches * 1e3, 4),
            "bytes_per_launch": total, "path": PATHS[plan.plan.path]}


def suite_single(torch, B, synth, dev, n, k, z, reps, fmts, rounds=5, m=1, label=""):
    """One matrix shape in `fmts`, `reps` device copies each: per-call stats cycling through the copies
    (>= 200 calls), and the grouped sustained rate measured `rounds` times with the format order
    rotated every round; format comparisons are medians of per-round time ratios."""
    w = synth.ternary(n, k, z, seed=0)
    s = torch.from_numpy(synth.scales(n, k // 128, seed=0)).to(dev)
    x = torch.from_numpy(synth.activations(m, k, seed=0)).to(dev)
    sets = {}
    for f in fmts:
        dw0 = B.DeviceWeights(B.pack_t5b(w, T5B_SCALE) if f == B.FMT_T5B else B.pack(f, w), dev)
        sets[f] = replicas(B, dw0, reps)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    out = {"n": n, "k": k, "m": m, "z": z, "replicas": reps, "x_bytes": m * k, "y_bytes": 4 * m * n}
    rates = {f: [] for f in fmts}
    for r in range(rounds):
        order = fmts[r % len(fmts):] + fmts[:r % len(fmts)]
        for f in order:
            dws = sets[f]
            sf = None if f == B.FMT_T5B else [s] * len(dws)
            rates[f].append(sustained(torch, B, dws, [x] * len(dws), sf, [y] * len(dws), launches=3))
    for f in fmts:
        dws = sets[f]
        ncalls = max(200, len(dws))
        s1 = None if f == B.FMT_T5B else s
        calls = [(lambda d=dws[i % len(dws)]: B.ternary_gemv(d, s1, x, y)) for i in range(ncalls)]
        pc = per_call_us(torch, calls)
        pc["gbs_at_median"] = round(packed_bytes(dws[0]) / pc["median_us"] / 1e3, 1)
        pc["graph_us_per_call"] = graph_call_us(torch, calls)
        pc["graph_gbs"] = round(packed_bytes(dws[0]) / pc["graph_us_per_call"] / 1e3, 1)
        ms = [r["ms_per_launch"] for r in rates[f]]
        out[B.FMT_NAMES[f]] = {"packed_bytes": packed_bytes(dws[0]),
                               "sustained_gbs_median": round(float(np.median([r["gbs"] for r in rates[f]])), 1),
                               "sustained_ms_per_launch_median": round(float(np.median(ms)), 4),
                               "per_call": pc}
    if B.FMT_BITCOS in fmts:
        for f in fmts:
            if f == B.FMT_BITCOS:
                continue
            ratio = [a["ms_per_launch"] / b["ms_per_launch"] for a, b in zip(rates[f], rates[B.FMT_BITCOS])]
            out[f"time_{B.FMT_NAMES[f]}_over_bitcos"] = round(float(np.median(ratio)), 4)
            out[f"bytes_{B.FMT_NAMES[f]}_over_bitcos"] = round(packed_bytes(sets[f][0]) /
                                                              packed_bytes(sets[B.FMT_BITCOS][0]), 4)
    del sets
    torch.cuda.empty_cache()
    log(f"[suite] {label} done")
    return out


def suite_thin(torch, B, synth, dev, reps=96, ms=(1, 2, 4, 8, 16)):
    """gate 14336x4096 and down 4096x14336 at z = 0.44, BITCOS, activation rows m in `ms`: int8
    activations (per-call and grouped) and fp16 activations (grouped)."""
    out = {}
    for name, n, k, role in (("gate", 14336, 4096, 4), ("down", 4096, 14336, 6)):
        w = synth.ternary(n, k, 0.44, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        s = torch.from_numpy(synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))).to(dev)
        dws = replicas(B, B.DeviceWeights(B.pack_bitcos(w), dev), reps)
        for m in ms:
            x = torch.from_numpy(synth.activations(m, k, seed=m)).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            st = sustained(torch, B, dws, [x] * reps, [s] * reps, [y] * reps)
            calls = [(lambda d=dws[i % reps]: B.ternary_gemv(d, s, x, y)) for i in range(max(200, reps))]
            pc = per_call_us(torch, calls)
            pc["graph_us_per_call"] = graph_call_us(torch, calls)
            x16 = torch.from_numpy(synth.float_activations(m, k, seed=m).astype(np.float16)).to(dev)
            sh = sustained(torch, B, dws, [x16] * reps, [s] * reps, [y] * reps, f16=True)
            out[f"{name}_m{m}"] = {"n": n, "k": k, "m": m, "path": st["path"],
                                   "sustained_gbs": st["gbs"], "sustained_us_per_gemv": round(st["ms_per_launch"] * 1e3 / reps, 3),
                                   "per_call": pc, "packed_bytes": packed_bytes(dws[0]), "x_bytes": m * k,
                                   "y_bytes": 4 * m * n,
                                   "fp16": {"path": sh["path"], "sustained_gbs": sh["gbs"],
                                            "sustained_us_per_gemv": round(sh["ms_per_launch"] * 1e3 / reps, 3)}}
        del dws
        torch.cuda.empty_cache()
    log("[suite] thin batch done")
    return out


def suite_32b(torch, B, synth, dev, layers=STACK32B_LAYERS):
    """32B-shaped layer stack at batch 1 (q, o 5120x5120; k, v 1024x5120; gate, up 25600x5120;
    down 5120x25600), 1219 dead FFN rows per layer at the same indices in gate and up. One layer is
    generated and stored `layers` times (6.08 GB of BITCOS for 64), so every byte comes from HBM."""
    st_set, dead = stack32b(B, synth, torch, dev, layers)
    mats = st_set.flat()
    dws, xs, ss, ys = [m["w"] for m in mats], [m["x"] for m in mats], [m["s"] for m in mats], [m["y"] for m in mats]
    st = sustained(torch, B, dws, xs, ss, ys, launches=5)
    per_layer = [st_set.plan(B, row) for row in st_set.mats]
    settle(torch, lambda: [p.run() for p in per_layer])
    sl = time_launches(torch, lambda: [p.run() for p in per_layer], 3, 0)
    out = {"layers": layers, "z": STACK32B_Z, "dead_rows_per_layer": int(dead.size), "bytes_per_pass": st["bytes_per_launch"],
           "grouped_one_launch": {"gbs": st["gbs"], "us_per_pass": round(st["ms_per_launch"] * 1e3, 1)},
           "per_layer_launch": {"gbs": round(st["bytes_per_launch"] * 3 / sl / 1e9, 1),
                                "us_per_pass": round(sl / 3 * 1e6, 1)}}
    del st_set, per_layer
    torch.cuda.empty_cache()
    log("[suite] 32B-shaped stack done")
    return out


# One GPU's share of an 8-way tensor-parallel split, laid out as the column-split dataflow of the
# untitled page on a NUMA-aware decode engine for ternary models (Sec. 5): q, k, v, gate and up split
# by output rows, o and down by the reduction dimension (group-aligned), so each GPU runs these shapes
# and the partial outputs of o and down meet in one all-reduce per matrix (not part of one GPU's step).
TP = 8
SHARD_32B = [("q", 5120 // TP, 5120), ("k", 1024 // TP, 5120), ("v", 1024 // TP, 5120), ("o", 5120, 5120 // TP),
             ("gate", 25600 // TP, 5120), ("up", 25600 // TP, 5120), ("down", 5120, 25600 // TP)]
SHARD_8B = [("q", 4096 // TP, 4096), ("k", 1024 // TP, 4096), ("v", 1024 // TP, 4096), ("o", 4096, 4096 // TP),
            ("gate", 14336 // TP, 4096), ("up", 14336 // TP, 4096), ("down", 4096, 14336 // TP)]


def suite_shards(torch, B, synth, dev):
    """The first GPU's shard of an 8-way split of the 32B-shaped stack (64 layers; its gate and up rows
    keep the dead rows that fall in the first 3200) and of the Llama3-8B layer set (32 layers, 189 MB:
    the share fits the 256 MB cache), one grouped launch per pass and per-layer launches, settled."""
    out = {"tp": TP}
    dead = synth.dead_rows(25600, STACK32B_DEAD, seed=0)
    for key, shapes, layers, z, dd in (("stack32b", SHARD_32B, STACK32B_LAYERS, STACK32B_Z, dead[dead < 25600 // TP]),
                                       ("llama3_8b", SHARD_8B, LAYERS, Z, None)):
        ls = LayerSet(B, synth, torch, dev, B.FMT_BITCOS, layers=layers, shapes=shapes, z=z, dead=dd)
        mats = ls.flat()
        st = sustained(torch, B, [m["w"] for m in mats], [m["x"] for m in mats], [m["s"] for m in mats],
                       [m["y"] for m in mats], launches=10)
        per_layer = [ls.plan(B, row) for row in ls.mats]
        settle(torch, lambda: [p.run() for p in per_layer])
        sl = time_launches(torch, lambda: [p.run() for p in per_layer], 3, 0)
        out[key] = {"shapes": [list(x) for x in shapes], "layers": layers, "z": z,
                    "dead_rows_per_layer": 0 if dd is None else int(dd.size), "bytes_per_pass": st["bytes_per_launch"],
                    "grouped_one_launch": {"gbs": st["gbs"], "us_per_pass": round(st["ms_per_launch"] * 1e3, 1)},
                    "per_layer_launch": {"gbs": round(st["bytes_per_launch"] * 3 / sl / 1e9, 1),
                                         "us_per_layer": round(sl / 3 / layers * 1e6, 2)}}
        del ls, per_layer, mats
        torch.cuda.empty_cache()
    log("[suite] tensor-parallel shards done")
    return out


def suite_cpu(O, B, synth):
    """The oracle from packed BITCOS bytes on one core and on all cores (2560x2560 and 4096x4096)."""
    cores = len(os.sched_getaffinity(0))
    out = {"cpu_model": cpu_model(), "cores_available": cores}
    for n, k, z in ((2560, 2560, 0.42), (4096, 4096, 0.40)):
        w = synth.ternary(n, k, z, seed=0)
        p = B.pack_bitcos(w)
        s = synth.scales(n, k // 128, seed=0)
        x = synth.activations(1, k, seed=0)
        nbytes = p.desc.bytes_payload + 2 * n * (k // 128)
        res = {}
        for th in (1, cores):
            O.set_threads(th)
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                O.gemv_packed(O.FMT_BITCOS, p.section("codes"), p.sign_bytes(), p.rowoff(), s, n, k, x)
                ts.append(time.perf_counter() - t0)
            t = float(np.median(ts))
            res[f"threads_{th}"] = {"ms": round(t * 1e3, 3), "gbs": round(nbytes / t / 1e9, 4)}
        out[f"{n}x{k}"] = res
    O.set_threads(cores)
    return out


def run_suite(path):
    import torch

    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import binding as bd
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    F = [B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT, B.FMT_T5B]
    res = {"command": f"python3 bench.py --suite {path}", "device": torch.cuda.get_device_name(0),
           "hbm_peak_gbs": HBM_PEAK_GBS,
           "note": "packed bytes = bitmap + sign stream + row index + fp16 scales (BITCOS) or codes + fp16 "
                   "scales; x and y bytes are listed apart; per-call times are HIP-event intervals between "
                   "consecutive eager launches (launch gaps included), cycling through the copies; "
                   "graph_us_per_call replays the same calls from one HIP graph (host launch path removed)"}
    log("[suite] stream-read ceiling")
    res["stream_read_ceiling_gbs"] = round(stream_ceiling(torch, bd, dev), 1)
    res["single_2560"] = suite_single(torch, B, synth, dev, 2560, 2560, 0.42, 768, F, label="2560x2560")
    res["zero_density_8192"] = {str(z): suite_single(torch, B, synth, dev, 8192, 8192, z, 96, F, label=f"8192 z={z}")
                                for z in (0.30, 0.375, 0.42, 0.47, 0.515)}
    res["thin_batch"] = suite_thin(torch, B, synth, dev)
    res["stack32b"] = suite_32b(torch, B, synth, dev)
    res["tp8_shards"] = suite_shards(torch, B, synth, dev)
    import oracle as O
    log("[suite] CPU oracle")
    res["cpu_oracle"] = suite_cpu(O, B, synth)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps({"suite": path}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Back-to-back launches of a decode-heavy kernel on MI355X run through a clock transient: the
    # shader clock drops a few milliseconds into the load and recovers over some tens of
    # milliseconds (`python -m bit_gemv_decode_amd.profiling transient` measures it). The timed
    # region is what --steps/--warmup say, transient included; the `settled` field times the same
    # launches again after SETTLE_MS of load.
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--quick", action="store_true", help="only the timed BITCOS step (for profiling runs)")
    ap.add_argument("--suite", metavar="PATH", help="run the measurement suite over every workload "
                    "configuration instead (several minutes) and write its JSON report to PATH")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the ternary GEMV would shard across GPUs by rows (or by k with one "
              "all-reduce of the output vector), and the multi-GPU path is not implemented. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.suite:
        run_suite(args.suite)
        return

    import torch

    import bit_gemv_decode_amd as B
    from bit_gemv_decode_amd import binding as bd
    from bit_gemv_decode_amd import synth

    dev = torch.device("cuda:0")
    log("[bench] packing the Llama3-8B-shaped layer set (BITCOS) and storing 32 layer copies")
    ls = LayerSet(B, synth, torch, dev, B.FMT_BITCOS)
    plan = ls.plan(B)
    log(f"[bench] BITCOS: {ls.step_bytes / 1e9:.3f} GB per step, {plan.plan.units} work units, "
        f"{plan.plan.waves} waves; timing {args.steps} steps")
    secs = time_launches(torch, plan.run, args.steps, args.warmup)
    step_s = secs / args.steps
    gbs = ls.step_bytes / step_s / 1e9
    log(f"[bench] BITCOS grouped: {gbs:.1f} GB/s, {step_s * 1e3:.3f} ms/step")

    traffic = load_traffic()
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded iid ternary z=0.40, fp16 scales U[0.01,0.1], int8 x U[-127,127])",
        "config": {"workload": "Llama3-8B-shaped decode layer set at batch 1 (q,o 4096x4096; k,v 1024x4096; "
                               "gate,up 14336x4096; down 4096x14336), BITCOS, 32 layer copies, one grouped "
                               "launch per step",
                   "zero_density": Z, "group": 128, "layers": LAYERS, "gemvs_per_step": LAYERS * len(LAYER),
                   "format": "bitcos", "m": 1},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     # HBM bytes per launch over the same launch time as `achieved` (GB/s)
                     "traffic": (round(traffic["bytes_per_launch"] / step_s / 1e9, 2) if traffic else None),
                     "traffic_ratio": (round(traffic["bytes_per_launch"] / ls.step_bytes, 4) if traffic else None),
                     "hbm_bytes_per_launch": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": "bitcos_gemv_kernel<1, false, false, false, false, false> (grouped, one launch per step)",
                     "algorithmic_bytes_per_launch": ls.step_bytes,
                     "avg_launch_us": round(step_s * 1e6, 2)},
    }
    if traffic:
        out["roofline"]["traffic_note"] = (f"traffic: HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                           f"scaled by the counters' readings for a stream read and a fill of "
                                           f"known size; {os.path.relpath(TRAFFIC_FILE, ROOT)}) over the "
                                           f"launch time of `achieved`; traffic_ratio: the same bytes over "
                                           f"the algorithmic bytes")
    # the same launches again once the GPU has run them back to back for SETTLE_MS (an extra field:
    # `value` above is the timed region of this command as given)
    settle(torch, plan.run)
    s_set = time_launches(torch, plan.run, args.steps, 0) / args.steps
    out["settled"] = {"gbs": round(ls.step_bytes / s_set / 1e9, 1), "ms_per_step": round(s_set * 1e3, 4),
                      "note": f"same step, timed after {SETTLE_MS:.0f} ms of back-to-back launches"}
    if args.quick:
        print(json.dumps(out), flush=True)
        return

    # same pass as 32 per-layer launches (7 GEMVs each) and as 224 single-GEMV launches in a graph
    layer_plans = [ls.plan(B, row) for row in ls.mats]
    s_layer = time_launches(torch, lambda: [p.run() for p in layer_plans], max(3, args.steps // 4), max(1, args.warmup // 4))
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        for m in ls.flat():
            B.ternary_gemv(m["w"], m["s"], m["x"], m["y"], stream=st)
    s_call = time_launches(torch, g.replay, max(3, args.steps // 4), max(1, args.warmup // 4))
    n_pl = max(3, args.steps // 4)
    out["modes"] = {
        "grouped_one_launch": {"gbs": round(gbs, 1), "ms_per_step": round(step_s * 1e3, 3)},
        "per_layer_launch": {"gbs": round(ls.step_bytes * n_pl / s_layer / 1e9, 1),
                             "ms_per_step": round(s_layer / n_pl * 1e3, 3), "launches_per_step": LAYERS,
                             "us_per_launch": round(s_layer / n_pl / LAYERS * 1e6, 2)},
        "per_gemv_launch_graph": {"gbs": round(ls.step_bytes * n_pl / s_call / 1e9, 1),
                                  "ms_per_step": round(s_call / n_pl * 1e3, 3),
                                  "launches_per_step": LAYERS * len(LAYER)},
    }
    # single-call time of each matrix: a graph cycling through the 32 copies (weights from HBM)
    per_mat = {}
    for role, (name, n, k) in enumerate(LAYER):
        gm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gm, stream=st):
            for row in ls.mats:
                m = row[role]
                B.ternary_gemv(m["w"], m["s"], m["x"], m["y"], stream=st)
        sm = time_launches(torch, gm.replay, 5, 1)
        us = sm / (5 * LAYERS) * 1e6
        per_mat[name] = {"us_per_call": round(us, 3), "gbs": round(ls.layer_bytes[role] / us / 1e3, 1)}
        del gm
    out["per_matrix_single_call"] = per_mat
    del layer_plans, g
    torch.cuda.empty_cache()
    log("[bench] cache-resident decode rate (the step over 4 distinct layer copies)")
    out["cache_resident"] = {"bitcos": cache_resident(torch, B, ls)}
    log("[bench] L2-resident decode rate (one 2560x2560 matrix, 768 references)")
    out["l2_resident"] = l2_resident(torch, B, synth, dev)

    log("[bench] float activations: quantiser and GEMV with activation group scales")
    out["activation_quant"] = activation_quant(torch, B, synth, ls, dev, max(3, args.steps // 2), args.warmup)

    log("[bench] BITCOS nibble-keyed decode")
    pn = ls.plan(B).set_decode(B.DECODE_NIBBLE)
    n_n = max(3, args.steps // 2)
    sn = time_launches(torch, pn.run, n_n, args.warmup)
    out["nibble_decode"] = {"gbs": round(ls.step_bytes * n_n / sn / 1e9, 1), "ms_per_step": round(sn / n_n * 1e3, 4)}
    del pn

    log("[bench] fp16 activations")
    out["fp16_activations"] = fp16_activations(torch, B, synth, ls, dev, max(3, args.steps // 2), args.warmup)

    log("[bench] stream-read ceiling")
    ceil = stream_ceiling(torch, bd, dev)
    out["stream_read_ceiling_gbs"] = round(ceil, 1)
    out["pct_of_stream_ceiling"] = round(100 * gbs / ceil, 2)

    bitcos_host = ls
    formats = {"bitcos": {"gbs": round(gbs, 1), "ms_per_step": round(step_s * 1e3, 3), "step_bytes": ls.step_bytes}}
    del plan
    for fname, fmt in (("5trit", B.FMT_5TRIT), ("2bit", B.FMT_2BIT), ("t5b", B.FMT_T5B)):
        log(f"[bench] {fname} layer set")
        lf = LayerSet(B, synth, torch, dev, fmt)
        pf = lf.plan(B)
        default = pf.plan.decode  # the table-free decode for 2-bit, the LDS table for the others
        n_f = max(3, args.steps // 2)
        rates = {}
        # the LDS-table decode and the table-free one (five-trit digits by multiply and shift, 2-bit codes
        # by shift and mask; no LDS table), the plan's default decode reported at the top level
        for decode in (B.DECODE_BYTE, B.DECODE_ARITH):
            pf.set_decode(decode)
            sf = time_launches(torch, pf.run, n_f, args.warmup)
            rates[decode] = {"gbs": round(lf.step_bytes * n_f / sf / 1e9, 1), "ms_per_step": round(sf / n_f * 1e3, 3)}
        formats[fname] = {**rates[default], "step_bytes": lf.step_bytes,
                          "decode": "table_free" if default == B.DECODE_ARITH else "table",
                          "table": rates[B.DECODE_BYTE], "table_free": rates[B.DECODE_ARITH]}
        if fname != "t5b":
            out["cache_resident"][fname] = cache_resident(torch, B, lf, decode=B.DECODE_BYTE)
            out["cache_resident"][f"{fname}_table_free"] = cache_resident(torch, B, lf, decode=B.DECODE_ARITH)
        del pf, lf
        torch.cuda.empty_cache()
    out["formats"] = formats
    out["bitcos_vs_5trit_time"] = round(formats["5trit"]["ms_per_step"] / formats["bitcos"]["ms_per_step"], 4)
    out["5trit_vs_bitcos_bytes"] = round(formats["5trit"]["step_bytes"] / formats["bitcos"]["step_bytes"], 4)
    out["bitcos_vs_2bit_time"] = round(formats["2bit"]["ms_per_step"] / formats["bitcos"]["ms_per_step"], 4)
    out["2bit_vs_bitcos_bytes"] = round(formats["2bit"]["step_bytes"] / formats["bitcos"]["step_bytes"], 4)
    out["bitcos_vs_t5b_time"] = round(formats["t5b"]["ms_per_step"] / formats["bitcos"]["ms_per_step"], 4)
    out["t5b_vs_bitcos_bytes"] = round(formats["t5b"]["step_bytes"] / formats["bitcos"]["step_bytes"], 4)

    if not args.no_cpu:
        import oracle as O

        log("[bench] timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(O, bitcos_host)
        out["gpu_vs_cpu"] = round(gbs / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
