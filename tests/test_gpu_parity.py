"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Int32 per-group accumulators must match bit for bit. fp32 outputs must satisfy, element by element,
|y - y_ref| <= 1e-5 * max(|y_ref|, sum_g |s * acc| / sqrt(ng)): a 1e-5 relative bound, measured
against the size of the terms when cancellation makes y_ref itself tiny. Both sides sum exact
fp64 products (fp16 * int32 needs at most 26 bits), so for the scale ranges used here the fp64 sums
are exact and y is expected to be bit-identical; the test also reports how many elements differ.
"""
import itertools
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


def y_tolerance_ok(y, y_ref, acc, scales):
    return bounds.int8_y_ok(y, y_ref, acc, scales)


def run_case(w, x, scales, fmts=FMTS, label=""):
    dev = _dev()
    acc_ref = O.gemv_acc(w, x)
    y_ref = O.combine(acc_ref, scales)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    st = torch.from_numpy(np.ascontiguousarray(scales)).to(dev)
    for fmt in fmts:
        _say(f"[gpu] {label} fmt={B.FMT_NAMES[fmt]} n={w.shape[0]} k={w.shape[1]} m={x.shape[0]}")
        dw = B.DeviceWeights(B.pack(fmt, w), dev)
        acc = B.ternary_gemv_acc(dw, xt)
        y = B.ternary_gemv(dw, st, xt)
        torch.cuda.synchronize()
        acc_np = acc.cpu().numpy()
        y_np = y.cpu().numpy()
        assert np.array_equal(acc_np, acc_ref), f"{label} {B.FMT_NAMES[fmt]}: int32 accumulators differ"
        ok, ndiff = y_tolerance_ok(y_np, y_ref, acc_ref, scales)
        assert ok, f"{label} {B.FMT_NAMES[fmt]}: y outside tolerance"
        assert ndiff == 0, f"{label} {B.FMT_NAMES[fmt]}: {ndiff} y values not bit-identical"


SMALL = [(1, 128, 0.42, 1), (3, 256, 0.0, 2), (4, 640, 1.0, 1), (5, 2176, 0.42, 3), (37, 4096, 0.4, 4),
         (129, 5120, 0.47, 1), (64, 2560, 0.95, 5), (17, 14336, 0.44, 16), (9, 384, 0.3, 7), (130, 1024, 0.515, 2)]


@pytest.mark.parametrize("n,k,z,m", SMALL, ids=[f"{n}x{k}_z{z}_m{m}" for n, k, z, m in SMALL])
def test_small_shapes(n, k, z, m):
    seed = n * 1000 + k + m
    w = synth.ternary(n, k, z, seed=seed)
    x = synth.activations(m, k, seed=seed)
    s = synth.scales(n, k // 128, seed=seed)
    run_case(w, x, s, label=f"small {n}x{k}")


@pytest.mark.parametrize("k,start", [(128, 60), (256, 124)])
def test_brute_force_patterns(k, start):
    pats = np.array(list(itertools.product([-1, 0, 1], repeat=8)), np.int8)
    w = np.zeros((len(pats), k), np.int8)
    w[:, start:start + 8] = pats
    x = np.concatenate([synth.activations(2, k, seed=9), np.full((1, k), -128, np.int8), np.full((1, k), 127, np.int8)])
    s = synth.scales(len(pats), k // 128, seed=9)
    run_case(w, x, s, label=f"brute k={k} start={start}")


def test_extreme_activations_and_structure():
    n, k = 70, 2048
    w = synth.ternary(n, k, 0.4, seed=31)
    w[0] = 0            # empty row
    w[1] = 1            # full positive row
    w[2] = -1           # full negative row
    w[3, :] = 0
    w[3, 2047] = -1     # single non-zero at the very end
    w[4, :64] = 0       # leading empty word
    x = np.stack([np.full(k, -128, np.int8), np.full(k, 127, np.int8), synth.activations(1, k, seed=31)[0]])
    s = synth.scales(n, k // 128, seed=31)
    s[5, 3] = np.float16(0.0)
    s[6, :] = np.float16(65504.0)
    s[7, 0] = np.float16(-0.5)
    run_case(w, x, s, label="extremes")


def test_non_default_stream():
    dev = _dev()
    n, k = 96, 4096
    w = synth.ternary(n, k, 0.4, seed=41)
    x = synth.activations(1, k, seed=41)
    s = synth.scales(n, k // 128, seed=41)
    y_ref = O.gemv(w, s, x)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        dw = B.DeviceWeights(B.pack_bitcos(w), dev)
        y = B.ternary_gemv(dw, torch.from_numpy(s).to(dev), torch.from_numpy(x).to(dev), stream=st)
    st.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_ref)


# ----- grouped launch (one persistent kernel over a table of GEMVs) ------------------------------------

# Shapes cover: full 4096-weight chunks only (4096), full chunks plus power-of-two tails of 2, 4 and 8
# rows per step (14336, 5120, 25600 -> 32, 16 and 8 lanes per row), tails only (1024, 384: 8 and 6
# lanes), a non-power-of-two tail (2560: 40 lanes) and single-row and odd-row matrices.
PLAN_SHAPES = [(96, 4096), (40, 5120), (33, 14336), (7, 2560), (130, 1024), (1, 128), (64, 384), (9, 25600)]


PLAN_CASES = [(f, m) for f in FMTS for m in (1, 2, 3)] + [(B.FMT_BITCOS, m) for m in (4, 7, 16)]


@pytest.mark.parametrize("fmt,m", PLAN_CASES, ids=[f"{B.FMT_NAMES[f]}-m{m}" for f, m in PLAN_CASES])
def test_plan_matches_oracle(fmt, m):
    dev = _dev()
    _say(f"[gpu] plan fmt={B.FMT_NAMES[fmt]} m={m} shapes={PLAN_SHAPES}")
    ws, xs, ss, refs, accrefs, dws = [], [], [], [], [], []
    for i, (n, k) in enumerate(PLAN_SHAPES):
        w = synth.ternary(n, k, 0.4 + 0.01 * i, seed=100 + i)
        x = synth.activations(m, k, seed=200 + i)
        s = synth.scales(n, k // 128, seed=300 + i)
        acc_ref = O.gemv_acc(w, x)
        accrefs.append(acc_ref)
        refs.append(O.combine(acc_ref, s))
        dws.append(B.DeviceWeights(B.pack(fmt, w), dev))
        xs.append(torch.from_numpy(x).to(dev))
        ss.append(torch.from_numpy(s).to(dev))
    ys = [torch.full((m, w.n), float("nan"), dtype=torch.float32, device=dev) for w in dws]
    accs = [torch.full((m, w.n, w.k // 128), -7, dtype=torch.int32, device=dev) for w in dws]
    B.Plan(dws, xs, scales=ss, ys=ys).run()
    B.Plan(dws, xs, accs=accs).run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(PLAN_SHAPES):
        assert np.array_equal(accs[i].cpu().numpy(), accrefs[i]), f"plan acc {n}x{k}"
        y = ys[i].cpu().numpy()
        ok, ndiff = y_tolerance_ok(y, refs[i], accrefs[i], ss[i].cpu().numpy())
        assert ok and ndiff == 0, f"plan y {n}x{k}: within tolerance {ok}, {ndiff} differ"


def test_plan_equals_per_call_and_replays():
    dev = _dev()
    shapes = [(4096, 4096), (1024, 4096), (512, 14336)]
    dws, xs, ss, ys1 = [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.4, seed=7 + i)
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        xs.append(torch.from_numpy(synth.activations(1, k, seed=8 + i)).to(dev))
        ss.append(torch.from_numpy(synth.scales(n, k // 128, seed=9 + i)).to(dev))
        ys1.append(B.ternary_gemv(dws[-1], ss[-1], xs[-1]))
    ys = [torch.empty((1, w.n), dtype=torch.float32, device=dev) for w in dws]
    plan = B.Plan(dws, xs, scales=ss, ys=ys)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        for a, b in zip(ys, ys1):
            assert torch.equal(a, b), f"replay {rep}"


# ----- the benchmark workloads at full size ---------------------------------------------------------

LLAMA = {"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
         "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336)}


def test_single_gemv_2560():
    n = k = 2560
    w = synth.ternary(n, k, 0.42, seed=0)
    run_case(w, synth.activations(1, k, seed=0), synth.scales(n, k // 128, seed=0), label="2560x2560")


@pytest.mark.parametrize("name", list(LLAMA))
def test_llama3_8b_layer(name):
    n, k = LLAMA[name]
    role = list(LLAMA).index(name)
    w = synth.ternary(n, k, 0.40, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
    x = synth.activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_X))
    s = synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))
    run_case(w, x, s, label=f"llama3-8b {name}")


@pytest.mark.parametrize("z", [0.30, 0.375, 0.42, 0.47, 0.515])
def test_zero_density_sweep_8192(z):
    n = k = 8192
    w = synth.ternary(n, k, z, seed=0)
    run_case(w, synth.activations(1, k, seed=0), synth.scales(n, k // 128, seed=0), label=f"8192 z={z}")


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("name", ["gate", "down"])
def test_thin_batch(name, m):
    n, k = LLAMA[name]
    w = synth.ternary(n, k, 0.44, seed=0, tid=synth.tensor_id(0, 1 if name == "gate" else 2, synth.STREAM_W))
    x = synth.activations(m, k, seed=m)
    s = synth.scales(n, k // 128, seed=0)
    run_case(w, x, s, fmts=[B.FMT_BITCOS], label=f"thin {name} m={m}")


def test_dead_rows_layer_5120():
    # Four point seven six percent of FFN neurons identically zero at the same indices in gate and up.
    n, k = 25600, 5120
    dead = synth.dead_rows(n, round(0.0476 * n), seed=0)
    assert dead.size == 1219
    for role in (4, 5):
        w = synth.ternary(n, k, 0.47, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        w[dead] = 0
        x = synth.activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_X))
        s = synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))
        run_case(w, x, s, fmts=[B.FMT_BITCOS], label=f"dead-rows role={role}")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: B.FMT_NAMES[f])
def test_graph_replays_match_eager(fmt):
    """Launches captured in a HIP graph: every replay (with eager work and synchronisation between
    replays) reproduces the eager results exactly."""
    dev = _dev()
    shapes = [(1024, 4096), (4096, 4096), (14336, 4096), (512, 14336)]
    items = []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.4, seed=50 + i)
        dw = B.DeviceWeights(B.pack(fmt, w), dev)
        x = torch.from_numpy(synth.activations(1, k, seed=60 + i)).to(dev)
        s = torch.from_numpy(synth.scales(n, k // 128, seed=70 + i)).to(dev)
        items.append((dw, x, s, B.ternary_gemv(dw, s, x)))
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    ys = [torch.empty((1, dw.n), dtype=torch.float32, device=dev) for dw, _, _, _ in items]
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for (dw, x, s, _), y in zip(items, ys):
            B.ternary_gemv(dw, s, x, y, stream=st)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (dw, _, _, ref), y in zip(items, ys):
            assert torch.equal(y, ref), f"{B.FMT_NAMES[fmt]} replay {rep} n={dw.n} k={dw.k}"


# Plans of long rows only (k > 8192) at m = 2 take the thin-batch matrix-core path; mixed with shorter
# rows that hold most of the weights they stay on the vector kernels; without chunked rows they take
# the 12-wave vector build with two-step units. All must match the oracle.
@pytest.mark.parametrize("shapes,path", [([(33, 14336), (9, 25600), (20, 16384)], 1),
                                          ([(33, 14336), (300, 4096)], 0),
                                          ([(300, 4096), (77, 2560), (130, 8192), (5, 128), (64, 1024)], 4)],
                         ids=["long-rows", "mixed", "single-chunk"])
def test_plan_m2_path_choice(shapes, path):
    dev = _dev()
    m = 2
    _say(f"[gpu] plan m=2 path={path} shapes={shapes}")
    dws, xs, ss, ys, refs = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.44, seed=500 + i)
        x = synth.activations(m, k, seed=600 + i)
        s = synth.scales(n, k // 128, seed=700 + i)
        acc_ref = O.gemv_acc(w, x)
        refs.append((O.combine(acc_ref, s), acc_ref, s))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        xs.append(torch.from_numpy(x).to(dev))
        ss.append(torch.from_numpy(s).to(dev))
        ys.append(torch.full((m, n), float("nan"), dtype=torch.float32, device=dev))
    plan = B.Plan(dws, xs, scales=ss, ys=ys)
    assert plan.plan.path == path
    plan.run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(shapes):
        y_ref, acc_ref, s = refs[i]
        ok, ndiff = y_tolerance_ok(ys[i].cpu().numpy(), y_ref, acc_ref, s)
        assert ok and ndiff == 0, f"plan m=2 {n}x{k}: within tolerance {ok}, {ndiff} differ"


def test_plan_coarse_chunked_units():
    """A plan with more work units than the launch has waves keeps 8-row units for chunked rows (small
    plans and single calls use 2-row units): one 4096x4096 matrix referenced often enough to exceed
    the wave count, plus chunked 14336- and 25600-long rows, all against the oracle."""
    dev = _dev()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    reps = (cus * 16) // 512 + 1  # 512 units per 4096x4096 GEMV at m = 1
    _say(f"[gpu] coarse plan: {reps} x 4096x4096 + chunked rows")
    big = synth.ternary(4096, 4096, 0.4, seed=800)
    xb = synth.activations(1, 4096, seed=801)
    sb = synth.scales(4096, 32, seed=802)
    refs = [(O.combine(O.gemv_acc(big, xb), sb))]
    dw_big = B.DeviceWeights(B.pack_bitcos(big), dev)
    xbt, sbt = torch.from_numpy(xb).to(dev), torch.from_numpy(sb).to(dev)
    dws, xs, ss = [dw_big] * reps, [xbt] * reps, [sbt] * reps
    chunked = []
    for i, (n, k) in enumerate([(37, 14336), (11, 25600)]):
        w = synth.ternary(n, k, 0.45, seed=810 + i)
        x = synth.activations(1, k, seed=820 + i)
        s = synth.scales(n, k // 128, seed=830 + i)
        acc_ref = O.gemv_acc(w, x)
        chunked.append((O.combine(acc_ref, s), acc_ref, s))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        xs.append(torch.from_numpy(x).to(dev))
        ss.append(torch.from_numpy(s).to(dev))
    ys = [torch.full((1, d.n), float("nan"), dtype=torch.float32, device=dev) for d in dws]
    plan = B.Plan(dws, xs, scales=ss, ys=ys)
    assert plan.plan.units >= cus * 16 and plan.plan.rows_per_unit == 8
    plan.run()
    torch.cuda.synchronize()
    for i in range(reps):
        assert np.array_equal(ys[i].cpu().numpy(), refs[0]), f"coarse plan copy {i}"
    for (y_ref, acc_ref, s), y in zip(chunked, ys[reps:]):
        ok, ndiff = y_tolerance_ok(y.cpu().numpy(), y_ref, acc_ref, s)
        assert ok and ndiff == 0, f"coarse plan chunked: within tolerance {ok}, {ndiff} differ"


@pytest.mark.parametrize("m", [1, 3, 4])
def test_very_long_rows(m):
    """k = 65664: 513 groups, nine chunk passes with a one-group tail; every format (t5b: 411 blocks,
    seven passes, a 27-block tail), the vector path and (BITCOS, m = 3, 4) the matrix-core path."""
    n, k = 96, 65664
    w = synth.ternary(n, k, 0.41, seed=1313)
    x = synth.activations(m, k, seed=1314)
    s = synth.scales(n, k // 128, seed=1315)
    run_case(w, x, s, label=f"long rows m={m}")
    dev = _dev()
    acc_ref = O.gemv_acc_blocks(w, x)
    dw = B.DeviceWeights(B.pack_t5b(w, 0.02), dev)
    xt = torch.from_numpy(x).to(dev)
    acc = B.ternary_gemv_acc(dw, xt)
    y = B.ternary_gemv(dw, None, xt)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref), "t5b long rows: block sums differ"
    y_ref = O.combine_tensor(acc_ref, 0.02)
    ok, ndiff = bounds.tensor_y_ok(y.cpu().numpy(), y_ref, acc_ref, 0.02)
    assert ok and ndiff == 0, f"t5b long rows: within the bound {ok}, {ndiff} outputs differ"

