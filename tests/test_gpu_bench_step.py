"""Parity of the launches bench.py times, at their full size: one grouped plan over the Llama3-8B-shaped
layer set stored 32 times (224 GEMVs, 1.51 GB of BITCOS), with the default byte-keyed decode, the
nibble-keyed decode and fp16 activations. The 32 copies hold the same bytes, so the oracle computes
the 7 distinct GEMVs and every output of every copy is checked against them: y within
|y - y_ref| <= 1e-5 * max(|y_ref|, sum_g |s * acc| / sqrt(ng)) and bit-identical in practice (exact
fp64 terms); the fp16 step within 2^-22 |y_ref| + 2^-17 sum_g |s_g| sum_{k in g} |W x|.
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


@pytest.fixture(scope="module")
def layer_set():
    import bench

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    _say("[gpu] bench layer set: packing and storing 32 copies")
    ls = bench.LayerSet(B, synth, torch, dev, B.FMT_BITCOS)
    refs = []
    for role, (name, n, k) in enumerate(bench.LAYER):
        w = synth.ternary(n, k, bench.Z, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        h = ls.host[role]
        acc = O.gemv_acc(w, h["x"])
        xf = synth.float_activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_XF))
        x16 = xf.astype(np.float16)
        refs.append(dict(w=w, s=h["s"], acc=acc, y=O.combine(acc, h["s"]), x16=x16, y16=O.gemv_f16(w, h["s"], x16)))
    yield bench, ls, refs, dev
    del ls
    torch.cuda.empty_cache()


def _reset(ls):
    for m in ls.flat():
        m["y"].fill_(float("nan"))


@pytest.mark.parametrize("decode", [B.DECODE_BYTE, B.DECODE_NIBBLE], ids=["byte", "nibble"])
def test_bench_step_every_output(layer_set, decode):
    bench, ls, refs, dev = layer_set
    _say(f"[gpu] bench step, decode={decode}")
    plan = ls.plan(B).set_decode(decode)
    assert plan.plan.count == 7 * bench.LAYERS and plan.plan.path == 0
    _reset(ls)
    plan.run()
    torch.cuda.synchronize()
    for role, (name, n, k) in enumerate(bench.LAYER):
        r = refs[role]
        for layer in range(bench.LAYERS):
            y = ls.mats[layer][role]["y"].cpu().numpy()
            assert bounds.int8_y_ok(y, r["y"], r["acc"], r["s"])[0], f"{name} copy {layer}"
            assert np.array_equal(y, r["y"]), f"{name} copy {layer}: not bit-identical"


def test_bench_fp16_step_every_output(layer_set):
    bench, ls, refs, dev = layer_set
    _say("[gpu] bench fp16 step")
    mats = [(role, m) for row in ls.mats for role, m in enumerate(row)]
    x16 = [torch.from_numpy(r["x16"]).to(dev) for r in refs]
    plan = B.Plan([m["w"] for _, m in mats], [x16[r] for r, _ in mats], scales=[m["s"] for _, m in mats],
                  ys=[m["y"] for _, m in mats], f16=True)
    assert plan.plan.path == 2
    _reset(ls)
    plan.run()
    torch.cuda.synchronize()
    for role, (name, n, k) in enumerate(bench.LAYER):
        r = refs[role]
        bound = bounds.f16_bound(r["w"], r["s"], r["x16"], r["y16"])
        for layer in range(bench.LAYERS):
            y = ls.mats[layer][role]["y"].cpu().numpy()
            assert np.all(np.abs(y.astype(np.float64) - r["y16"].astype(np.float64)) <= bound), f"{name} copy {layer}"


@pytest.mark.parametrize("mode", ["byte", "nibble", "fp16"])
def test_per_layer_plans_every_output(layer_set, mode):
    # the bench's per-layer mode: 32 launches of the 7 GEMVs of one layer each. A one-layer plan gives
    # its chunked 4096 x 14336 rows 4-row units (8-row ones would each cost over 1.5 times a wave's
    # share), and every range starts with the pass whose activation wait follows the first bitmaps.
    bench, ls, refs, dev = layer_set
    _say(f"[gpu] per-layer plans, {mode}")
    if mode == "fp16":
        x16 = [torch.from_numpy(r["x16"]).to(dev) for r in refs]
        plans = [B.Plan([m["w"] for m in row], x16, scales=[m["s"] for m in row], ys=[m["y"] for m in row], f16=True)
                 for row in ls.mats]
    else:
        plans = [ls.plan(B, row).set_decode(B.DECODE_NIBBLE if mode == "nibble" else B.DECODE_BYTE) for row in ls.mats]
    _reset(ls)
    for p in plans:
        p.run()
    torch.cuda.synchronize()
    for role, (name, n, k) in enumerate(bench.LAYER):
        r = refs[role]
        bound = bounds.f16_bound(r["w"], r["s"], r["x16"], r["y16"]) if mode == "fp16" else None
        for layer in range(bench.LAYERS):
            y = ls.mats[layer][role]["y"].cpu().numpy()
            if mode == "fp16":
                err = np.abs(y.astype(np.float64) - r["y16"].astype(np.float64))
                assert np.all(err <= bound), f"{name} copy {layer}"
            else:
                assert np.array_equal(y, r["y"]), f"{name} copy {layer}: not bit-identical"
