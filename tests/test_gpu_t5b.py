"""GPU parity of the t5b format (five-trit bytes in 160-weight blocks, one scale per tensor).

The int32 block sums must match the oracle bit for bit. fp32 outputs are compared with the oracle's
y = (float)(scale * exact row sum) element by element within
|y - y_ref| <= 1e-5 * max(|y_ref|, sum_b |scale * acc_b| / sqrt(blocks)), the bound of the other
formats; the kernel adds exact fp64 block terms, so y is expected to be identical.
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


def y_ok(y, y_ref, acc, scale):
    return bounds.tensor_y_ok(y, y_ref, acc, scale)


def run_t5b(w, x, scale, label=""):
    dev = _dev()
    _say(f"[gpu] t5b {label} n={w.shape[0]} k={w.shape[1]} m={x.shape[0]}")
    acc_ref = O.gemv_acc_blocks(w, x)
    y_ref = O.combine_tensor(acc_ref, scale)
    dw = B.DeviceWeights(B.pack_t5b(w, scale), dev)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    acc = B.ternary_gemv_acc(dw, xt)
    y = B.ternary_gemv(dw, None, xt)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref), f"t5b {label}: block sums differ"
    ok, ndiff = y_ok(y.cpu().numpy(), y_ref, acc_ref, scale)
    assert ok, f"t5b {label}: y outside tolerance ({ndiff} differ)"


SHAPES = [(1, 128, 0.42, 1), (3, 256, 0.0, 2), (5, 640, 1.0, 1), (37, 4096, 0.4, 1), (129, 5120, 0.47, 3),
          (17, 14336, 0.44, 2), (9, 25600, 0.47, 1), (64, 2560, 0.95, 1), (130, 1024, 0.515, 16), (20, 14336, 0.4, 4)]


@pytest.mark.parametrize("n,k,z,m", SHAPES, ids=[f"{n}x{k}_z{z}_m{m}" for n, k, z, m in SHAPES])
def test_t5b_small_shapes(n, k, z, m):
    seed = n * 1000 + k + m
    w = synth.ternary(n, k, z, seed=seed)
    x = synth.activations(m, k, seed=seed)
    run_t5b(w, x, 0.03125 + 0.001 * m, label="small")


def test_t5b_extremes():
    n, k = 70, 2560
    w = synth.ternary(n, k, 0.4, seed=31)
    w[0] = 0
    w[1] = 1
    w[2] = -1
    w[3, :] = 0
    w[3, k - 1] = -1
    x = np.stack([np.full(k, -128, np.int8), np.full(k, 127, np.int8), synth.activations(1, k, seed=31)[0]])
    run_t5b(w, x, 1.0, label="extremes")
    run_t5b(w, x, -0.75, label="negative scale")


@pytest.mark.parametrize("name,n,k", [("q", 4096, 4096), ("gate", 14336, 4096), ("down", 4096, 14336)])
def test_t5b_llama3_8b_layer(name, n, k):
    w = synth.ternary(n, k, 0.40, seed=0, tid=synth.tensor_id(0, 5, synth.STREAM_W))
    run_t5b(w, synth.activations(1, k, seed=0), 0.0213, label=f"llama3-8b {name}")


@pytest.mark.parametrize("m", [1, 3])
def test_t5b_plan_matches_oracle(m):
    dev = _dev()
    shapes = [(96, 4096), (40, 5120), (33, 14336), (7, 2560), (130, 1024), (1, 128), (9, 25600)]
    _say(f"[gpu] t5b plan m={m}")
    dws, xs, ys, accs, refs = [], [], [], [], []
    for i, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.4 + 0.01 * i, seed=900 + i)
        x = synth.activations(m, k, seed=950 + i)
        scale = 0.01 * (i + 1)
        acc_ref = O.gemv_acc_blocks(w, x)
        refs.append((acc_ref, O.combine_tensor(acc_ref, scale), scale))
        dws.append(B.DeviceWeights(B.pack_t5b(w, scale), dev))
        xs.append(torch.from_numpy(x).to(dev))
        ys.append(torch.full((m, n), float("nan"), dtype=torch.float32, device=dev))
        accs.append(torch.full((m, n, B.groups_per_row(B.FMT_T5B, k)), -7, dtype=torch.int32, device=dev))
    B.Plan(dws, xs, ys=ys).run()
    B.Plan(dws, xs, accs=accs).run()
    torch.cuda.synchronize()
    for i, (n, k) in enumerate(shapes):
        acc_ref, y_ref, scale = refs[i]
        assert np.array_equal(accs[i].cpu().numpy(), acc_ref), f"t5b plan acc {n}x{k}"
        ok, ndiff = y_ok(ys[i].cpu().numpy(), y_ref, acc_ref, scale)
        assert ok, f"t5b plan y {n}x{k}: {ndiff} differ"
