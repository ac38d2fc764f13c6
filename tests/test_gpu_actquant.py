"""GPU parity of the per-group activation quantisation and the GEMV with activation group scales.

The quantiser decides every code in fp32 on both sides, so the int8 codes and the fp32 group scales
must match the oracle bit for bit. The scaled GEMV is compared with the oracle's fp64 definition
y = sum_g (scale * acc) * xs (every term exact, one rounding): element by element within
|y - y_ref| <= 1e-5 * max(|y_ref|, sum_g |scale * xs * acc| / sqrt(ng)), the same bound as the plain
GEMV. The thin-batch matrix-core path adds the terms in the oracle's order and must be bit-identical.
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
FMTS = [B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def _quantize_gpu(xf):
    dev = _dev()
    xq, xs = B.quantize_x(torch.from_numpy(np.ascontiguousarray(xf)).to(dev))
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def _edge_activations(k):
    """Rows built to hit the quantiser's special cases, one group per case (k >= 128 * 6)."""
    x = synth.float_activations(1, k, seed=77)[0].copy()
    x[0:128] = 0.0                                    # all-zero group: sigma 0, codes 0
    x[128:256] = 0.0
    x[200] = -3.25                                    # one non-zero, negative: code -127
    x[256:384] = np.arange(128, dtype=np.float32) - 63.5  # sigma = 0.5 exactly: codes -127 .. 127, odd
    x[384:512] = np.float32(127.0) * np.sign(np.arange(128) - 63.5).astype(np.float32)
    x[384:448] = 2.0 * np.arange(64, dtype=np.float32) - 63.5  # sigma = 1: every ratio a tie, to even
    x[384] = -127.0
    x[512:640] = np.float32(1e-30) * (np.arange(128, dtype=np.float32) - 64.0)  # tiny but normal
    x[640:768] = np.float32(3e38) * np.cos(np.arange(128, dtype=np.float32))  # near the fp32 top
    return x[None, :]


QSHAPES = [(1, 128), (1, 2560), (3, 4096), (16, 14336), (2, 5120), (5, 384)]


@pytest.mark.parametrize("m,k", QSHAPES, ids=[f"m{m}_k{k}" for m, k in QSHAPES])
def test_quantize_matches_oracle_bit_exact(m, k):
    _say(f"[gpu] quantize m={m} k={k}")
    xf = synth.float_activations(m, k, seed=m * 31 + k)
    xq, xs = _quantize_gpu(xf)
    xq_ref, xs_ref = O.quantize_x(xf)
    assert np.array_equal(xq, xq_ref), f"int8 codes differ in {(xq != xq_ref).sum()} places"
    assert np.array_equal(xs.view(np.uint32), xs_ref.view(np.uint32)), "group scales differ"


def test_quantize_special_groups_bit_exact():
    _say("[gpu] quantize special groups")
    xf = _edge_activations(1024)
    xq, xs = _quantize_gpu(xf)
    xq_ref, xs_ref = O.quantize_x(xf)
    assert xs_ref[0, 0] == 0.0 and np.all(xq_ref[0, :128] == 0)
    assert np.array_equal(xq, xq_ref)
    assert np.array_equal(xs.view(np.uint32), xs_ref.view(np.uint32))


def y_xs_tolerance_ok(y, y_ref, acc, scales, xs):
    return bounds.int8_y_ok(y, y_ref, acc, scales, xs)


def run_xs_case(w, xf, scales, fmts=FMTS, label="", exact=False):
    """float activations -> GPU quantiser -> scaled GEMV, against the oracle's quantiser and definition."""
    dev = _dev()
    xq_ref, xs_ref = O.quantize_x(xf)
    acc_ref = O.gemv_acc(w, xq_ref)
    y_ref = O.combine_xs(acc_ref, scales, xs_ref)
    xq, xs = B.quantize_x(torch.from_numpy(np.ascontiguousarray(xf)).to(dev))
    st = torch.from_numpy(np.ascontiguousarray(scales)).to(dev)
    for fmt in fmts:
        _say(f"[gpu] {label} fmt={B.FMT_NAMES[fmt]} n={w.shape[0]} k={w.shape[1]} m={xf.shape[0]}")
        dw = B.DeviceWeights(B.pack(fmt, w), dev)
        y = B.ternary_gemv_xs(dw, st, xq, xs)
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), xq_ref), f"{label}: quantised activations differ"
        y_np = y.cpu().numpy()
        ok, ndiff = y_xs_tolerance_ok(y_np, y_ref, acc_ref, scales, xs_ref)
        assert ok, f"{label} {B.FMT_NAMES[fmt]}: y outside tolerance ({ndiff} differ)"
        if exact:
            assert ndiff == 0, f"{label} {B.FMT_NAMES[fmt]}: {ndiff} y values not bit-identical"


XS_SMALL = [(1, 128, 0.42, 1), (37, 4096, 0.4, 1), (129, 5120, 0.47, 2), (17, 14336, 0.44, 3), (130, 1024, 0.515, 2),
            (33, 2560, 0.42, 4), (20, 14336, 0.44, 16), (9, 384, 0.3, 7)]


@pytest.mark.parametrize("n,k,z,m", XS_SMALL, ids=[f"{n}x{k}_z{z}_m{m}" for n, k, z, m in XS_SMALL])
def test_gemv_xs_small_shapes(n, k, z, m):
    seed = n * 1000 + k + m
    w = synth.ternary(n, k, z, seed=seed)
    xf = synth.float_activations(m, k, seed=seed)
    s = synth.scales(n, k // 128, seed=seed)
    run_xs_case(w, xf, s, label=f"xs small {n}x{k}")


def test_gemv_xs_special_activation_groups():
    n, k = 70, 1024
    w = synth.ternary(n, k, 0.4, seed=5)
    xf = _edge_activations(k)[:, :]
    xf[0, 640:768] = synth.float_activations(1, 128, seed=6)[0]  # keep y finite
    s = synth.scales(n, k // 128, seed=5)
    run_xs_case(w, xf, s, label="xs special groups")


@pytest.mark.parametrize("m", [4, 8, 16])
@pytest.mark.parametrize("name,n,k", [("gate", 14336, 4096), ("down", 4096, 14336)])
def test_gemv_xs_thin_batch_bit_identical(name, n, k, m):
    w = synth.ternary(n, k, 0.44, seed=0, tid=synth.tensor_id(0, 1 if name == "gate" else 2, synth.STREAM_W))
    xf = synth.float_activations(m, k, seed=m)
    s = synth.scales(n, k // 128, seed=0)
    run_xs_case(w, xf, s, fmts=[B.FMT_BITCOS], label=f"xs thin {name} m={m}", exact=True)


@pytest.mark.parametrize("name,n,k", [("q", 4096, 4096), ("gate", 14336, 4096), ("down", 4096, 14336)])
def test_gemv_xs_llama3_8b_layer(name, n, k):
    w = synth.ternary(n, k, 0.40, seed=0, tid=synth.tensor_id(0, 3, synth.STREAM_W))
    xf = synth.float_activations(1, k, seed=0)
    s = synth.scales(n, k // 128, seed=0)
    run_xs_case(w, xf, s, label=f"xs llama3-8b {name}")


def test_gemv_xs_unit_scales_equal_plain_gemv():
    """With every activation group scale 1 the scaled GEMV is the plain GEMV, value for value."""
    dev = _dev()
    n, k = 300, 4096
    w = synth.ternary(n, k, 0.4, seed=12)
    x = torch.from_numpy(synth.activations(2, k, seed=12)).to(dev)
    s = torch.from_numpy(synth.scales(n, k // 128, seed=12)).to(dev)
    ones = torch.ones((2, k // 128), dtype=torch.float32, device=dev)
    for fmt in FMTS:
        dw = B.DeviceWeights(B.pack(fmt, w), dev)
        assert torch.equal(B.ternary_gemv_xs(dw, s, x, ones), B.ternary_gemv(dw, s, x)), B.FMT_NAMES[fmt]


PLAN_SHAPES = [(96, 4096), (40, 5120), (33, 14336), (7, 2560), (130, 1024), (1, 128), (9, 25600)]
PLAN_CASES = [(f, m) for f in FMTS for m in (1, 3)] + [(B.FMT_BITCOS, m) for m in (4, 16)]


@pytest.mark.parametrize("fmt,m", PLAN_CASES, ids=[f"{B.FMT_NAMES[f]}-m{m}" for f, m in PLAN_CASES])
def test_plan_xs_matches_oracle(fmt, m):
    dev = _dev()
    _say(f"[gpu] plan xs fmt={B.FMT_NAMES[fmt]} m={m}")
    dws, xqs, xss, ss, refs = [], [], [], [], []
    for i, (n, k) in enumerate(PLAN_SHAPES):
        w = synth.ternary(n, k, 0.4 + 0.01 * i, seed=100 + i)
        xf = synth.float_activations(m, k, seed=200 + i)
        s = synth.scales(n, k // 128, seed=300 + i)
        xq_ref, xs_ref = O.quantize_x(xf)
        acc_ref = O.gemv_acc(w, xq_ref)
        refs.append((O.combine_xs(acc_ref, s, xs_ref), acc_ref, s, xs_ref))
        dws.append(B.DeviceWeights(B.pack(fmt, w), dev))
        xq, xs = B.quantize_x(torch.from_numpy(xf).to(dev))
        xqs.append(xq)
        xss.append(xs)
        ss.append(torch.from_numpy(s).to(dev))
    ys = [torch.full((m, w.n), float("nan"), dtype=torch.float32, device=dev) for w in dws]
    B.Plan(dws, xqs, scales=ss, ys=ys, x_scales=xss).run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(PLAN_SHAPES):
        y_ref, acc_ref, s, xs_ref = refs[i]
        ok, ndiff = y_xs_tolerance_ok(ys[i].cpu().numpy(), y_ref, acc_ref, s, xs_ref)
        assert ok, f"plan xs {n}x{k}: outside tolerance ({ndiff} differ)"
