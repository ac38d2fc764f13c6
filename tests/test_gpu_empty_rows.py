"""GPU parity for BITCOS matrices with rows that hold no non-zero weight (the dead FFN neurons of
"Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract). The packer
records their count in the descriptor, and the m = 1 launches with fp32 outputs then walk only the
other rows of GEMVs with one row per step (32 < k/128 <= 64), storing 0 for the empty ones. Every
output is compared with the oracle: bit-identical, the empty rows exactly 0 (outputs are pre-filled
with NaN, so a row the kernel forgot shows). The patterns cover a sparse random set, long runs (a
64-row index window with fewer than four non-empty rows), the first and last rows, all rows empty,
a single non-empty row, and plans whose per-wave ranges cut through them.
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


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def _matrix(n, k, pattern, seed):
    w = synth.ternary(n, k, 0.45, seed=seed)
    if pattern == "random":
        w[synth.dead_rows(n, max(1, n // 20), seed=seed)] = 0
    elif pattern == "runs":
        w[3:80] = 0          # 77 consecutive empty rows: windows with fewer than four non-empty rows
        w[150:290] = 0
        w[-5:] = 0
    elif pattern == "edges":
        w[0] = 0
        w[1] = 0
        w[-1] = 0
    elif pattern == "all":
        w[:] = 0
    elif pattern == "one":
        w[:] = 0
        w[n // 2, 7] = -1
    elif pattern == "alternate":
        w[::2] = 0
    return w


PATTERNS = ["random", "runs", "edges", "all", "one", "alternate"]
SHAPES = [(301, 5120), (64, 8192), (257, 4224)]  # 40, 64 and 33 groups per row: one row per step


def _check(y, y_ref, acc_ref, s, w, label, xs=None):
    empty = ~w.any(axis=1)
    assert not np.isnan(y).any(), f"{label}: outputs not written"
    assert np.all(y[:, empty] == 0), f"{label}: empty rows not zero"
    ok, ndiff = bounds.int8_y_ok(y, y_ref, acc_ref, s, xs)
    assert ok and ndiff == 0, f"{label}: within the bound {ok}, {ndiff} outputs differ"


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("n,k", SHAPES, ids=[f"{n}x{k}" for n, k in SHAPES])
def test_single_call_skips_empty_rows(n, k, pattern):
    dev = _dev()
    seed = n + k + PATTERNS.index(pattern)
    w = _matrix(n, k, pattern, seed)
    x = synth.activations(1, k, seed=seed)
    s = synth.scales(n, k // 128, seed=seed)
    acc_ref = O.gemv_acc(w, x)
    y_ref = O.combine(acc_ref, s)
    p = B.pack_bitcos(w)
    assert p.desc.empty_rows == int((~w.any(axis=1)).sum())
    _say(f"[gpu] empty rows {pattern} {n}x{k}: {p.desc.empty_rows} empty")
    dw = B.DeviceWeights(p, dev)
    xt, st = torch.from_numpy(x).to(dev), torch.from_numpy(s).to(dev)
    y = torch.full((1, n), float("nan"), dtype=torch.float32, device=dev)
    B.ternary_gemv(dw, st, xt, y)
    acc = B.ternary_gemv_acc(dw, xt)
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), y_ref, acc_ref, s, w, f"{pattern} {n}x{k}")
    assert np.array_equal(acc.cpu().numpy(), acc_ref), f"{pattern} {n}x{k}: accumulators differ"
    # quantised activations with group scales take the same walk
    xf = synth.float_activations(1, k, seed=seed)
    xq_ref, xs_ref = O.quantize_x(xf)
    acc_q = O.gemv_acc(w, xq_ref)
    xq, xs = B.quantize_x(torch.from_numpy(xf).to(dev))
    yq = torch.full((1, n), float("nan"), dtype=torch.float32, device=dev)
    B.ternary_gemv_xs(dw, st, xq, xs, yq)
    torch.cuda.synchronize()
    _check(yq.cpu().numpy(), O.combine_xs(acc_q, s, xs_ref), acc_q, s, w, f"xs {pattern} {n}x{k}", xs_ref)


def test_plan_mixing_empty_rows_with_other_shapes():
    # one launch over GEMVs with and without empty rows, one-row steps, several rows per step and
    # chunked rows, in enough copies that the per-wave ranges cut through the empty runs
    dev = _dev()
    cases = [(_matrix(301, 5120, "runs", 1), 1), (_matrix(1024, 5120, "random", 2), 3),
             (_matrix(77, 8192, "alternate", 3), 2), (synth.ternary(130, 4096, 0.4, seed=4), 2),
             (_matrix(96, 2048, "random", 5), 1), (_matrix(40, 14336, "edges", 6), 2),
             (synth.ternary(512, 5120, 0.4, seed=7), 2)]
    dws, xs, ss, ys, refs = [], [], [], [], []
    for i, (w, copies) in enumerate(cases):
        n, k = w.shape
        x = synth.activations(1, k, seed=40 + i)
        s = synth.scales(n, k // 128, seed=50 + i)
        acc_ref = O.gemv_acc(w, x)
        p = B.pack_bitcos(w)
        for c in range(copies):
            dws.append(B.DeviceWeights(p, dev))
            xs.append(torch.from_numpy(x).to(dev))
            ss.append(torch.from_numpy(s).to(dev))
            ys.append(torch.full((1, n), float("nan"), dtype=torch.float32, device=dev))
            refs.append((w, s, acc_ref, O.combine(acc_ref, s)))
    plan = B.Plan(dws, xs, scales=ss, ys=ys)
    assert plan.plan.live_rows == 1
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        _say(f"[gpu] empty rows, mixed plan run {rep}")
        plan.run()
        torch.cuda.synchronize()
        for i, ((w, s, acc_ref, y_ref), y) in enumerate(zip(refs, ys)):
            _check(y.cpu().numpy(), y_ref, acc_ref, s, w, f"plan GEMV {i} run {rep}")
    # the same GEMVs with accumulator outputs take the plain walk
    accs = [torch.empty((1, d.n, d.k // 128), dtype=torch.int32, device=dev) for d in dws]
    pa = B.Plan(dws, xs, accs=accs)
    assert pa.plan.live_rows == 0
    pa.run()
    torch.cuda.synchronize()
    for (w, s, acc_ref, y_ref), a in zip(refs, accs):
        assert np.array_equal(a.cpu().numpy(), acc_ref)
