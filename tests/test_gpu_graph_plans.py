"""Grouped launches captured in a HIP graph: plans of every launch configuration a decode step may use
(the row walk with empty rows and wide lanes at m = 1, the 12-wave build at m = 2, the thin-batch
kernel with two- and three-tile units at m = 4 and 16, the quantised-activation path, the five-trit
table-free decode, and a plan whose table lives in the library's static array) replayed several
times, with eager work and synchronisation between the replays. Every replay must reproduce the eager
results exactly, and those match the oracle ("Breaking the 1.58-bit Barrier for Ternary LLMs",
Sec. II-C).
"""
import sys

import numpy as np
import pytest

import bit_gemv_decode_amd as B
import oracle as O
from oracle import bounds
from bit_gemv_decode_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _plan(dev, fmt, m, shapes, seed, xs=False, decode=B.DECODE_BYTE, noalloc=False):
    cases = []
    for i, (n, k, dead) in enumerate(shapes):
        w = synth.ternary(n, k, 0.44, seed=seed + i)
        if dead:
            w[synth.dead_rows(n, dead, seed=seed + i)] = 0
        s = synth.scales(n, k // 128, seed=seed + i)
        c = dict(n=n, s=s, st=torch.from_numpy(s).to(dev), dw=B.DeviceWeights(B.pack(fmt, w), dev))
        if xs:
            xf = synth.float_activations(m, k, seed=seed + i)
            xq_ref, c["xs_ref"] = O.quantize_x(xf)
            c["acc"] = O.gemv_acc(w, xq_ref)
            c["y_ref"] = O.combine_xs(c["acc"], s, c["xs_ref"])
            c["x"], c["xs"] = B.quantize_x(torch.from_numpy(xf).to(dev))
        else:
            x = synth.activations(m, k, seed=seed + i)
            c["acc"] = O.gemv_acc(w, x)
            c["y_ref"] = O.combine(c["acc"], s)
            c["x"] = torch.from_numpy(x).to(dev)
        c["y"] = torch.full((m, n), float("nan"), dtype=torch.float32, device=dev)
        cases.append(c)
        del w
    plan = B.Plan([c["dw"] for c in cases], [c["x"] for c in cases], scales=[c["st"] for c in cases],
                  ys=[c["y"] for c in cases], x_scales=[c["xs"] for c in cases] if xs else None, noalloc=noalloc)
    if decode != B.DECODE_BYTE:
        plan.set_decode(decode)
    return plan, cases


def test_graph_replays_of_plans_match_eager():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    specs = [  # (label, fmt, m, shapes (n, k, empty rows), expected path, options)
        ("row walk m=1", B.FMT_BITCOS, 1, [(300, 5120, 9), (1024, 5120, 0), (777, 4096, 13), (96, 14336, 0)], 0, {}),
        ("xs m=1", B.FMT_BITCOS, 1, [(200, 5120, 0), (333, 4096, 0)], 0, dict(xs=True)),
        ("12 waves m=2", B.FMT_BITCOS, 2, [(500, 4096, 0), (130, 2560, 0), (64, 8192, 0)], 4, {}),
        ("thin batch m=4", B.FMT_BITCOS, 4, [(300, 4096, 0), (100, 14336, 0)], 1, {}),
        ("thin batch m=16", B.FMT_BITCOS, 16, [(300, 4096, 0), (100, 14336, 0)], 1, {}),
        ("five-trit table-free", B.FMT_5TRIT, 1, [(400, 4096, 0), (90, 14336, 0)], 0, dict(decode=B.DECODE_ARITH)),
        ("static table", B.FMT_BITCOS, 1, [(256, 5120, 4), (512, 4096, 0)], 0, dict(noalloc=True)),
    ]
    plans = []
    for j, (label, fmt, m, shapes, path, opts) in enumerate(specs):
        plan, cases = _plan(dev, fmt, m, shapes, 3000 + 50 * j, **opts)
        assert plan.plan.path == path, f"{label}: path {plan.plan.path}"
        plans.append((label, plan, cases))
    # eager results first, checked against the oracle
    eager = []
    for label, plan, cases in plans:
        plan.run()
        torch.cuda.synchronize()
        for c in cases:
            got = c["y"].cpu().numpy()
            if "xs_ref" in c:
                ok, _ = bounds.int8_y_ok(got, c["y_ref"], c["acc"], c["s"], c["xs_ref"])
            else:
                ok, _ = bounds.int8_y_ok(got, c["y_ref"], c["acc"], c["s"])
            assert ok, f"{label}: eager result outside the bound ({c['n']} rows)"
        eager.append([c["y"].clone() for c in cases])
    _say("[gpu] graph of 7 plans: capture")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for _, plan, _ in plans:
            plan.run(stream=st)
    scratch = torch.zeros(1 << 20, dtype=torch.float32, device=dev)
    for rep in range(3):
        for _, _, cases in plans:
            for c in cases:
                c["y"].fill_(float("nan"))
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (label, _, cases), ref in zip(plans, eager):
            for c, r in zip(cases, ref):
                assert torch.equal(c["y"], r), f"{label}: replay {rep} differs from the eager launch ({c['n']} rows)"
