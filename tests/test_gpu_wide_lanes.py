"""GPU parity of BITCOS rows of 5120 weights at m = 1 with fp32 outputs, which the kernel runs with a
lane per 80 weights (ten presence bytes) so that a row fills the wave; a lane's weights lie in one
128-weight group or straddle two, and the two parts take their own group scales ("Breaking the
1.58-bit Barrier for Ternary LLMs", Sec. II-C: int32 group sums, the scale applied once per group).

Every output is checked against the oracle: plain fp32 outputs bit for bit (the kernel adds exact fp64
products, as the oracle does before its one rounding), outputs with activation group scales within the
stated bound. The same plans with the nibble-keyed decode, which keeps a lane per group, must give
identical outputs. Cases: one row, ragged row counts, all-non-zero weights (a lane's 80 signs fill its
window), all-zero weights (every row empty), sparse rows, empty rows among full ones, extreme
activations; and plans that mix these rows with rows of other lengths in one launch.
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

K = 5120
# (rows, zero density, empty rows)
CASES = [(1, 0.4, 0), (3, 0.0, 0), (130, 0.47, 7), (2, 1.0, 0), (257, 0.33, 0), (64, 0.95, 0), (1000, 0.42, 50)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def _case(n, k, z, dead, seed, dev, x_fill=None):
    w = synth.ternary(n, k, z, seed=seed)
    if dead:
        w[synth.dead_rows(n, dead, seed=seed)] = 0
    x = synth.activations(1, k, seed=seed)
    if x_fill is not None:
        x[:] = x_fill
    xf = synth.float_activations(1, k, seed=seed)
    s = synth.scales(n, k // 128, seed=seed)
    acc = O.gemv_acc(w, x)
    xq_ref, xs_ref = O.quantize_x(xf)
    acc_q = O.gemv_acc(w, xq_ref)
    xq, xs = B.quantize_x(torch.from_numpy(xf).to(dev))
    return dict(n=n, k=k, s=s, acc=acc, y=O.combine(acc, s), acc_q=acc_q, xs_ref=xs_ref,
                y_xs=O.combine_xs(acc_q, s, xs_ref), dw=B.DeviceWeights(B.pack_bitcos(w), dev),
                x=torch.from_numpy(x).to(dev), st=torch.from_numpy(s).to(dev), xq=xq, xs=xs)


def _check(c, y, yxs, label):
    y = y.cpu().numpy()
    ok, ndiff = bounds.int8_y_ok(y, c["y"], c["acc"], c["s"])
    assert ok and ndiff == 0, f"{label}: y outside the bound or not bit-identical ({ndiff} differ)"
    if yxs is not None:
        ok, ndiff = bounds.int8_y_ok(yxs.cpu().numpy(), c["y_xs"], c["acc_q"], c["s"], c["xs_ref"])
        assert ok, f"{label}: y with activation scales outside the bound ({ndiff} differ)"


def test_wide_lane_single_calls():
    dev = _dev()
    fills = {1: 127, 3: -128}
    for i, (n, z, dead) in enumerate(CASES):
        _say(f"[gpu] wide-lane single call {n}x{K} z={z} empty={dead}")
        c = _case(n, K, z, dead, 2100 + i, dev, fills.get(i))
        y = B.ternary_gemv(c["dw"], c["st"], c["x"])
        yxs = B.ternary_gemv_xs(c["dw"], c["st"], c["xq"], c["xs"])
        torch.cuda.synchronize()
        _check(c, y, yxs, f"{n}x{K} z={z}")


@pytest.mark.parametrize("mixed", [False, True], ids=["wide-only", "mixed"])
def test_wide_lane_plans(mixed):
    # several copies of every case in one launch (ranges cross rows, units and GEMVs); `mixed` adds rows
    # of 32, 112 and 200 groups (group lanes, chunked rows) to the same launch
    dev = _dev()
    shapes = [(n, K, z, dead) for n, z, dead in CASES]
    if mixed:
        shapes += [(4096, 4096, 0.4, 0), (512, 14336, 0.44, 3), (256, 25600, 0.47, 0), (2048, 4096, 0.4, 11)]
    _say(f"[gpu] wide-lane plan mixed={mixed}: 4 x {len(shapes)} GEMVs")
    cases = [_case(n, k, z, dead, 2200 + 10 * i + int(mixed), dev) for i, (n, k, z, dead) in enumerate(shapes)]
    order = [c for _ in range(4) for c in cases]
    dws = [c["dw"] for c in order]
    out = {}
    for decode in (B.DECODE_BYTE, B.DECODE_NIBBLE):
        ys = [torch.full((1, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
        B.Plan(dws, [c["x"] for c in order], scales=[c["st"] for c in order], ys=ys).set_decode(decode).run()
        out[decode] = ys
    yxs = [torch.full((1, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in order]
    B.Plan(dws, [c["xq"] for c in order], scales=[c["st"] for c in order], ys=yxs, x_scales=[c["xs"] for c in order]).run()
    torch.cuda.synchronize()
    for j, c in enumerate(order):
        label = f"GEMV {j} ({c['n']}x{c['k']})"
        _check(c, out[B.DECODE_BYTE][j], yxs[j], label)
        assert torch.equal(out[B.DECODE_BYTE][j], out[B.DECODE_NIBBLE][j]), f"{label}: differs from the group lanes"
