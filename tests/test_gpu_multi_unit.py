"""GPU parity of grouped launches whose per-wave ranges hold several work units, for every format and
output kind: 8 copies of six shapes (single-chunk rows of 32, 20 and 8 groups, a ragged row of 40
groups, chunked rows of 112 and 200 groups), each copy with its own outputs, in one launch. The
small-shape plan tests give most waves at most one unit; here ranges cross unit, chunk-pass and GEMV
boundaries many times. fp32 outputs, int32 group sums and the outputs with activation group scales
are checked against the oracle ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C), every
output of every copy; the int32 sums bit for bit.
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

SHAPES = [(4096, 4096), (2048, 2560), (4096, 1024), (1024, 5120), (512, 14336), (256, 25600)]
COPIES = 8
FMTS = [B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT]
CASES = [(f, m) for f in FMTS for m in (1, 2, 3)] + [(B.FMT_BITCOS, m) for m in (4, 16)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fmt,m", CASES, ids=[f"{B.FMT_NAMES[f]}-m{m}" for f, m in CASES])
def test_multi_unit_plans(fmt, m):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    _say(f"[gpu] multi-unit plans fmt={B.FMT_NAMES[fmt]} m={m}: {COPIES} x {len(SHAPES)} GEMVs")
    cases = []
    for i, (n, k) in enumerate(SHAPES):
        seed = 9100 + 10 * i + m
        w = synth.ternary(n, k, 0.4 + 0.02 * i, seed=seed)
        x = synth.activations(m, k, seed=seed)
        xf = synth.float_activations(m, k, seed=seed)
        s = synth.scales(n, k // 128, seed=seed)
        acc = O.gemv_acc(w, x)
        xq_ref, xs_ref = O.quantize_x(xf)
        acc_q = O.gemv_acc(w, xq_ref)
        xq, xs = B.quantize_x(torch.from_numpy(xf).to(dev))
        cases.append(dict(n=n, k=k, s=s, acc=acc, y=O.combine(acc, s), acc_q=acc_q, xs_ref=xs_ref,
                          y_xs=O.combine_xs(acc_q, s, xs_ref), dw=B.DeviceWeights(B.pack(fmt, w), dev),
                          x=torch.from_numpy(x).to(dev), st=torch.from_numpy(s).to(dev), xq=xq, xs=xs))
        del w
    order = [c for _ in range(COPIES) for c in cases]
    dws = [c["dw"] for c in order]
    ys = [torch.full((m, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
    accs = [torch.full((m, c["n"], c["k"] // 128), -7, dtype=torch.int32, device=dev) for c in order]
    yxs = [torch.full((m, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
    B.Plan(dws, [c["x"] for c in order], scales=[c["st"] for c in order], ys=ys).run()
    B.Plan(dws, [c["x"] for c in order], accs=accs).run()
    B.Plan(dws, [c["xq"] for c in order], scales=[c["st"] for c in order], ys=yxs,
           x_scales=[c["xs"] for c in order]).run()
    torch.cuda.synchronize()
    for j, c in enumerate(order):
        label = f"GEMV {j} ({c['n']}x{c['k']})"
        assert np.array_equal(accs[j].cpu().numpy(), c["acc"]), f"{label}: int32 sums differ"
        ok, ndiff = bounds.int8_y_ok(ys[j].cpu().numpy(), c["y"], c["acc"], c["s"])
        assert ok, f"{label}: y outside the bound ({ndiff} differ)"
        ok, ndiff = bounds.int8_y_ok(yxs[j].cpu().numpy(), c["y_xs"], c["acc_q"], c["s"], c["xs_ref"])
        assert ok, f"{label}: y with activation scales outside the bound ({ndiff} differ)"
