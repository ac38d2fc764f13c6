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


@pytest.mark.parametrize("m", [1, 2, 4, 16])
def test_multi_unit_f16_plans(m):
    # fp16 activations (BITCOS): the vector kernel at m = 1, the matrix-core kernel above (the long rows
    # hold most of these weights at m = 2), with the bound of the fp16 path
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    _say(f"[gpu] multi-unit fp16 plans m={m}: {COPIES} x {len(SHAPES)} GEMVs")
    cases = []
    for i, (n, k) in enumerate(SHAPES):
        seed = 9300 + 10 * i + m
        w = synth.ternary(n, k, 0.42, seed=seed)
        s = synth.scales(n, k // 128, seed=seed)
        x16 = synth.float_activations(m, k, seed=seed).astype(np.float16)
        y_ref = O.gemv_f16(w, s, x16)
        cases.append(dict(n=n, bound=bounds.f16_bound(w, s, x16, y_ref), y=y_ref,
                          dw=B.DeviceWeights(B.pack_bitcos(w), dev), st=torch.from_numpy(s).to(dev),
                          x=torch.from_numpy(x16).to(dev)))
        del w
    order = [c for _ in range(COPIES) for c in cases]
    ys = [torch.full((m, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
    B.Plan([c["dw"] for c in order], [c["x"] for c in order], scales=[c["st"] for c in order], ys=ys,
           f16=True).run()
    torch.cuda.synchronize()
    for j, c in enumerate(order):
        err = np.abs(ys[j].cpu().numpy().astype(np.float64) - c["y"].astype(np.float64))
        assert np.all(err <= c["bound"]), f"GEMV {j} ({c['n']} rows): outside the fp16 bound"


@pytest.mark.parametrize("m", [1, 2, 3])
def test_multi_unit_t5b_plans(m):
    # t5b: 32-byte blocks of 160 weights, one scale per tensor; the table and the table-free decode
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    _say(f"[gpu] multi-unit t5b plans m={m}: {COPIES} x {len(SHAPES)} GEMVs")
    cases = []
    for i, (n, k) in enumerate(SHAPES):
        seed = 9500 + 10 * i + m
        scale = 0.031 + 0.002 * i
        w = synth.ternary(n, k, 0.4, seed=seed)
        x = synth.activations(m, k, seed=seed)
        acc = O.gemv_acc_blocks(w, x)
        cases.append(dict(n=n, acc=acc, scale=scale, y=O.combine_tensor(acc, scale),
                          dw=B.DeviceWeights(B.pack_t5b(w, scale), dev), x=torch.from_numpy(x).to(dev)))
        del w
    order = [c for _ in range(COPIES) for c in cases]
    decodes = [B.DECODE_BYTE] + ([B.DECODE_ARITH] if m == 1 else [])
    for decode in decodes:
        ys = [torch.full((m, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
        B.Plan([c["dw"] for c in order], [c["x"] for c in order], ys=ys).set_decode(decode).run()
        torch.cuda.synchronize()
        for j, c in enumerate(order):
            ok, ndiff = bounds.tensor_y_ok(ys[j].cpu().numpy(), c["y"], c["acc"], c["scale"])
            assert ok, f"GEMV {j} ({c['n']} rows), decode {decode}: outside the bound ({ndiff} differ)"
