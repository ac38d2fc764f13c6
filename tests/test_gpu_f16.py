"""GPU parity of the BITCOS GEMV against fp16 activations ("Breaking the 1.58-bit Barrier for Ternary
LLMs", Sec. II-B and II-D: ternary weights rebuilt as +-1 or 0 in fp16 and multiplied with fp16
activations).

The oracle computes y = (float) sum_g s_g * sum_{k in g} W x exactly up to the final rounding. The
kernel sums each group in fp32 (exact products, at most two roundings per pair of weights, partial
sums no larger than S_g = sum_{k in g} |W x|), applies the scale and sums the groups exactly in fp64,
and rounds once to fp32; so element by element
    |y - y_ref| <= 2^-22 |y_ref| + 2^-17 * sum_g |s_g| * S_g
(128 roundings of at most 2^-24 S_g per group, plus the two fp32 output roundings).
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


def f16_bound(w, s, x16, y_ref):
    return bounds.f16_bound(w, s, x16, y_ref)


def run_f16(w, s, x16, label="", exact_check=True):
    dev = _dev()
    _say(f"[gpu] f16 {label} n={w.shape[0]} k={w.shape[1]} m={x16.shape[0]}")
    y_ref = O.gemv_f16(w, s, x16)
    dw = B.DeviceWeights(B.pack_bitcos(w), dev)
    st = torch.from_numpy(np.ascontiguousarray(s)).to(dev)
    xt = torch.from_numpy(np.ascontiguousarray(x16)).to(dev)
    y = B.ternary_gemv_f16(dw, st, xt)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(np.isfinite(y)), f"f16 {label}: non-finite outputs"
    if exact_check:
        bound = f16_bound(w, s, x16, y_ref)
        err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
        assert np.all(err <= bound), f"f16 {label}: {(err > bound).sum()} outputs outside the bound, worst " \
                                     f"{np.max(err / np.maximum(bound, 1e-300)):.3g}x"
    return y, y_ref


# (n, k, zero density, m): single-chunk rows (k <= 8192, R = 64 / ng rows per step) with ragged row
# counts, chunked rows (k > 8192: coarse 8-row units, fine 2-row units when the units are few), one
# and two activation rows per launch on the vector kernel; from m = 3 the matrix-core kernel (16-row
# tiles, 8-group chunks: ragged tiles, a partial last chunk, m up to 16).
SHAPES = [(1, 128, 0.42, 1), (3, 256, 0.0, 2), (5, 640, 1.0, 1), (37, 4096, 0.4, 1), (129, 5120, 0.47, 2),
          (17, 14336, 0.44, 1), (9, 25600, 0.47, 2), (64, 2560, 0.95, 1), (130, 1024, 0.515, 3),
          (600, 14336, 0.4, 1), (301, 8320, 0.3, 2), (2051, 4096, 0.44, 1),
          (1, 128, 0.4, 3), (33, 1152, 0.44, 4), (70, 4096, 0.0, 5), (97, 14336, 0.44, 8), (40, 2560, 1.0, 16),
          (300, 4224, 0.47, 16), (15, 25600, 0.47, 7), (50, 14336, 0.44, 2), (33, 8320, 0.4, 2)]


@pytest.mark.parametrize("n,k,z,m", SHAPES, ids=[f"{n}x{k}_z{z}_m{m}" for n, k, z, m in SHAPES])
def test_f16_shapes(n, k, z, m):
    seed = n * 1000 + k + m
    w = synth.ternary(n, k, z, seed=seed)
    s = synth.scales(n, k // 128, seed=seed)
    x16 = synth.float_activations(m, k, seed=seed).astype(np.float16)
    run_f16(w, s, x16, label="shape")


def test_f16_integer_activations_match_the_int8_gemv():
    # integer-valued fp16 activations: every group sum is exact in fp32 (|sum| <= 128 * 128 < 2^24),
    # so y equals the int8 GEMV's y bit for bit
    n, k = 333, 6144
    w = synth.ternary(n, k, 0.4, seed=41)
    s = synth.scales(n, k // 128, seed=41)
    x8 = synth.activations(2, k, seed=41)
    dev = _dev()
    y16, y_ref = run_f16(w, s, x8.astype(np.float16), label="integer")
    assert np.array_equal(y_ref, O.gemv(w, s, x8))
    dw = B.DeviceWeights(B.pack_bitcos(w), dev)
    y8 = B.ternary_gemv(dw, torch.from_numpy(s).to(dev), torch.from_numpy(x8).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(y16, y8.cpu().numpy())


def test_f16_integer_activations_match_the_int8_thin_batch():
    # the same on the matrix-core kernels (m = 4): fp32 group sums of integers are exact, and both
    # paths add the same fp64 terms in the same order
    n, k = 77, 14336
    w = synth.ternary(n, k, 0.44, seed=43)
    s = synth.scales(n, k // 128, seed=43)
    x8 = synth.activations(4, k, seed=43)
    dev = _dev()
    y16, y_ref = run_f16(w, s, x8.astype(np.float16), label="integer m=4")
    dw = B.DeviceWeights(B.pack_bitcos(w), dev)
    y8 = B.ternary_gemv(dw, torch.from_numpy(s).to(dev), torch.from_numpy(x8).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(y16, y8.cpu().numpy())


def test_f16_whole_range_values():
    # fp16 activations drawn over every finite bit pattern (subnormals, the largest normal), with
    # weight rows of all-zero, all +1, all -1 and a single -1 at the last column
    n, k = 70, 1280
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 0x7C00, size=(2, k), dtype=np.uint16)
    bits[0, :8] = [0x0001, 0x0002, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0x0000, 0x7BFE]
    bits |= rng.integers(0, 2, size=(2, k), dtype=np.uint16) << 15
    x16 = bits.view(np.float16)
    w = synth.ternary(n, k, 0.4, seed=12)
    w[0] = 0
    w[1] = 1
    w[2] = -1
    w[3, :] = 0
    w[3, k - 1] = -1
    s = synth.scales(n, k // 128, seed=12)
    y, y_ref = run_f16(w, s, x16, label="whole range")
    assert np.all(y[:, 0] == 0.0)
    x4 = np.concatenate([x16, -x16[::-1]])  # the matrix-core path
    y, y_ref = run_f16(w, s, x4, label="whole range m=4")
    assert np.all(y[:, 0] == 0.0)


@pytest.mark.parametrize("name,n,k", [("q", 4096, 4096), ("gate", 14336, 4096), ("down", 4096, 14336)])
def test_f16_llama3_8b_layer(name, n, k):
    w = synth.ternary(n, k, 0.40, seed=0, tid=synth.tensor_id(0, 5, synth.STREAM_W))
    s = synth.scales(n, k // 128, seed=0)
    x16 = synth.float_activations(1, k, seed=0).astype(np.float16)
    run_f16(w, s, x16, label=f"llama3-8b {name}")


def test_f16_rejects_other_formats_and_bad_arguments():
    dev = _dev()
    w = synth.ternary(8, 256, 0.4, seed=3)
    s = torch.from_numpy(synth.scales(8, 2, seed=3)).to(dev)
    x16 = torch.zeros((1, 256), dtype=torch.float16, device=dev)
    for fmt in (B.FMT_5TRIT, B.FMT_2BIT):
        with pytest.raises(B.TgError):
            B.ternary_gemv_f16(B.DeviceWeights(B.pack(fmt, w), dev), s, x16)
    dw = B.DeviceWeights(B.pack_bitcos(w), dev)
    with pytest.raises(B.TgError):
        B.ternary_gemv_f16(dw, s, torch.zeros((B.TG_MAX_M + 1, 256), dtype=torch.float16, device=dev))


def test_thin_batch_xs_after_f16_kernel():
    # The thin-batch kernel with activation group scales once read its scale stage for the pipeline-fill
    # steps before writing it, so Inf/NaN bit patterns left in LDS by an earlier kernel (the fp16 one
    # leaves fp64 tile terms there) could turn whole output rows into NaN. Run it right after the fp16
    # kernel on the same GPU and check it against the oracle.
    dev = _dev()
    n, k = 17, 14336
    w = synth.ternary(n, k, 0.44, seed=17)
    s = synth.scales(n, k // 128, seed=17)
    run_f16(w, s, synth.float_activations(2, k, seed=17).astype(np.float16), label="before thin batch")
    xf = synth.float_activations(3, k, seed=18)
    xq_ref, xs_ref = O.quantize_x(xf)
    acc_ref = O.gemv_acc(w, xq_ref)
    y_ref = O.combine_xs(acc_ref, s, xs_ref)
    dw = B.DeviceWeights(B.pack_bitcos(w), dev)
    st = torch.from_numpy(s).to(dev)
    for _ in range(3):
        B.ternary_gemv_f16(dw, st, torch.from_numpy(xf[:2].astype(np.float16)).to(dev))
        xq, xs = B.quantize_x(torch.from_numpy(xf).to(dev))
        y = B.ternary_gemv_xs(dw, st, xq, xs)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        assert np.all(np.isfinite(y))
        assert bounds.int8_y_ok(y, y_ref, acc_ref, s, xs_ref)[0]


@pytest.mark.parametrize("m", [1, 2, 4])
def test_f16_plan_matches_oracle(m):
    # at m = 2 the long rows (k > 8192) hold most of the weights: the matrix-core path
    # one grouped launch over GEMVs of mixed shapes (single-chunk, chunked, ragged), fp16 activations
    dev = _dev()
    shapes = [(96, 4096), (40, 5120), (33, 14336), (7, 2560), (130, 1024), (1, 128), (9, 25600), (300, 14336)]
    _say(f"[gpu] f16 plan m={m}")
    dws, ss, xs, ys, refs = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.4 + 0.01 * i, seed=700 + i)
        s = synth.scales(n, k // 128, seed=700 + i)
        x16 = synth.float_activations(m, k, seed=750 + i).astype(np.float16)
        refs.append((w, s, x16, O.gemv_f16(w, s, x16)))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        ss.append(torch.from_numpy(s).to(dev))
        xs.append(torch.from_numpy(x16).to(dev))
        ys.append(torch.full((m, n), float("nan"), dtype=torch.float32, device=dev))
    plan = B.Plan(dws, xs, scales=ss, ys=ys, f16=True)
    assert plan.plan.path == (2 if m == 1 else 3)
    plan.run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(shapes):
        w, s, x16, y_ref = refs[i]
        y = ys[i].cpu().numpy()
        err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
        assert np.all(err <= f16_bound(w, s, x16, y_ref)), f"f16 plan {n}x{k}"


def test_f16_plan_m2_vector_path_with_chunked_rows():
    # short rows hold most of the weights: the plan stays on the vector kernel, whose two-row chunked
    # path then runs the long-row GEMV
    dev = _dev()
    m = 2
    shapes = [(2000, 4096), (900, 2560), (60, 14336), (13, 8320)]
    _say("[gpu] f16 plan m=2 vector")
    dws, ss, xs, ys, refs = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.42, seed=800 + i)
        s = synth.scales(n, k // 128, seed=800 + i)
        x16 = synth.float_activations(m, k, seed=850 + i).astype(np.float16)
        refs.append((w, s, x16, O.gemv_f16(w, s, x16)))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        ss.append(torch.from_numpy(s).to(dev))
        xs.append(torch.from_numpy(x16).to(dev))
        ys.append(torch.full((m, n), float("nan"), dtype=torch.float32, device=dev))
    plan = B.Plan(dws, xs, scales=ss, ys=ys, f16=True)
    assert plan.plan.path == 2
    plan.run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(shapes):
        w, s, x16, y_ref = refs[i]
        err = np.abs(ys[i].cpu().numpy().astype(np.float64) - y_ref.astype(np.float64))
        assert np.all(err <= f16_bound(w, s, x16, y_ref)), f"f16 plan m=2 {n}x{k}"
