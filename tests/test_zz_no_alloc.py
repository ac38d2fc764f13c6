"""Plans whose table lives in the library's static device array (tg_plan_init_noalloc), for callers that
cannot allocate device memory: two calls in a row, the second with fewer GEMVs, each checked against the
same GEMVs planned with a caller-owned table (tg_plan_init) and against the oracle. The first plan is
refused once the second call has replaced the static table.
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


def _gemvs(dev, fmt, shapes, m, seed):
    out = []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.42, seed=seed + i)
        if i % 3 == 1:
            w[synth.dead_rows(n, max(1, n // 16), seed=seed + i)] = 0
        x = synth.activations(m, k, seed=seed + 100 + i)
        s = synth.scales(n, k // 128, seed=seed + 200 + i)
        acc = O.gemv_acc(w, x)
        out.append(dict(w=w, s=s, acc=acc, y=O.combine(acc, s), dw=B.DeviceWeights(B.pack(fmt, w), dev),
                        x=torch.from_numpy(x).to(dev), st=torch.from_numpy(s).to(dev)))
    return out


def test_noalloc_plan_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    # call 1: BITCOS, m = 1, fp32 outputs; one-row steps with empty rows, several rows per step, chunked rows
    g1 = _gemvs(dev, B.FMT_BITCOS, [(301, 5120), (1024, 5120), (130, 4096), (77, 14336), (512, 2560),
                                    (64, 8192), (33, 25600)], 1, 900)
    _say("[gpu] no-alloc plan, call 1: 7 BITCOS GEMVs, m = 1")
    ys = [torch.full((1, g["w"].shape[0]), float("nan"), dtype=torch.float32, device=dev) for g in g1]
    ref = [torch.empty_like(y) for y in ys]
    p1 = B.Plan([g["dw"] for g in g1], [g["x"] for g in g1], scales=[g["st"] for g in g1], ys=ys, noalloc=True)
    assert p1.plan.table_gen != 0 and p1.table is None
    p1.run()
    B.Plan([g["dw"] for g in g1], [g["x"] for g in g1], scales=[g["st"] for g in g1], ys=ref).run()
    torch.cuda.synchronize()
    for i, (g, y, r) in enumerate(zip(g1, ys, ref)):
        yn = y.cpu().numpy()
        assert np.array_equal(yn, r.cpu().numpy()), f"call 1 GEMV {i}: differs from the caller-table plan"
        ok, ndiff = bounds.int8_y_ok(yn, g["y"], g["acc"], g["s"])
        assert ok and ndiff == 0, f"call 1 GEMV {i}: {ndiff} outputs differ from the oracle"
    # call 2: fewer GEMVs, five-trit, m = 2, int32 accumulator outputs
    g2 = _gemvs(dev, B.FMT_5TRIT, [(200, 4096), (96, 14336), (40, 2560)], 2, 950)
    _say("[gpu] no-alloc plan, call 2: 3 five-trit GEMVs, m = 2, accumulators")
    accs = [torch.full(g["acc"].shape, -7, dtype=torch.int32, device=dev) for g in g2]
    accr = [torch.empty_like(a) for a in accs]
    p2 = B.Plan([g["dw"] for g in g2], [g["x"] for g in g2], accs=accs, noalloc=True)
    assert p2.plan.table_gen != p1.plan.table_gen
    p2.run()
    B.Plan([g["dw"] for g in g2], [g["x"] for g in g2], accs=accr).run()
    torch.cuda.synchronize()
    for i, (g, a, r) in enumerate(zip(g2, accs, accr)):
        an = a.cpu().numpy()
        assert np.array_equal(an, r.cpu().numpy()), f"call 2 GEMV {i}: differs from the caller-table plan"
        assert np.array_equal(an, g["acc"]), f"call 2 GEMV {i}: differs from the oracle"
    # the first plan's table was replaced: it is refused, and nothing runs
    with pytest.raises(B.TgError) as e:
        p1.run()
    assert e.value.code == -1
    # the second still runs and gives the same accumulators
    for a in accs:
        a.fill_(-7)
    p2.run()
    torch.cuda.synchronize()
    for g, a in zip(g2, accs):
        assert np.array_equal(a.cpu().numpy(), g["acc"])
