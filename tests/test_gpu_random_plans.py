"""GPU parity of grouped launches over seeded random mixes of shapes: each plan draws 4-10 GEMVs with
row counts from 1 to a few thousand, row lengths from one group to 224 groups (single-chunk rows of
every width, chunked rows with ragged last passes, the wide-lane rows of 5120 weights), zero
densities from 0 to 1 and, for some, empty rows; over every format, activation-row count, output kind
and decode a plan can take. Every output is compared with the oracle ("Breaking the 1.58-bit Barrier
for Ternary LLMs", Sec. II-C: int32 group sums, fp16 group scales applied once per group): int32
sums bit for bit, fp32 outputs within the stated bounds (plain int8 BITCOS outputs bit for bit).
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

# (format, m, output kind, decode); output kinds: y (fp32), acc (int32 group sums), xs (quantised
# activations with group scales), f16 (fp16 activations)
PLANS = [
    (B.FMT_BITCOS, 1, "y", B.DECODE_BYTE), (B.FMT_BITCOS, 1, "acc", B.DECODE_BYTE),
    (B.FMT_BITCOS, 1, "xs", B.DECODE_BYTE), (B.FMT_BITCOS, 1, "y", B.DECODE_NIBBLE),
    (B.FMT_BITCOS, 2, "y", B.DECODE_BYTE), (B.FMT_BITCOS, 3, "acc", B.DECODE_BYTE),
    (B.FMT_BITCOS, 5, "y", B.DECODE_BYTE), (B.FMT_BITCOS, 16, "xs", B.DECODE_BYTE),
    (B.FMT_BITCOS, 1, "f16", B.DECODE_BYTE), (B.FMT_BITCOS, 7, "f16", B.DECODE_BYTE),
    (B.FMT_5TRIT, 1, "y", B.DECODE_ARITH), (B.FMT_5TRIT, 2, "acc", B.DECODE_BYTE),
    (B.FMT_5TRIT, 3, "xs", B.DECODE_BYTE), (B.FMT_2BIT, 1, "acc", B.DECODE_ARITH),
    (B.FMT_2BIT, 3, "y", B.DECODE_BYTE), (B.FMT_T5B, 1, "y", B.DECODE_BYTE),
    (B.FMT_T5B, 1, "acc", B.DECODE_ARITH), (B.FMT_T5B, 2, "y", B.DECODE_BYTE),
]
WEIGHT_BUDGET = 3_000_000  # weights per GEMV at most, so that the oracle stays fast


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _draw(rng):
    ng = int(rng.choice([1, 2, 3, 5, 8, 20, 25, 31, 32, 33, 40, 40, 47, 64, 65, 112, 127, 128, 129, 200, 224]))
    k = 128 * ng
    n = int(rng.integers(1, max(2, min(3000, WEIGHT_BUDGET // k))))
    z = float(rng.choice([0.0, 0.2, 0.4, 0.47, 0.6, 0.9, 1.0]))
    dead = int(rng.integers(1, max(2, n // 8))) if rng.random() < 0.3 else 0
    return n, k, z, dead


@pytest.mark.parametrize("fmt,m,out,decode", PLANS,
                         ids=[f"{B.FMT_NAMES[f]}-m{m}-{o}-d{d}" for f, m, o, d in PLANS])
def test_random_plan(fmt, m, out, decode):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    seed = 4000 + 97 * PLANS.index((fmt, m, out, decode))
    rng = np.random.default_rng(seed)
    shapes = [_draw(rng) for _ in range(int(rng.integers(4, 11)))]
    _say(f"[gpu] random plan fmt={B.FMT_NAMES[fmt]} m={m} out={out} decode={decode}: {shapes}")
    t5b = fmt == B.FMT_T5B
    cases = []
    for i, (n, k, z, dead) in enumerate(shapes):
        s_ = seed + 10 * i
        w = synth.ternary(n, k, z, seed=s_)
        if dead:
            w[synth.dead_rows(n, dead, seed=s_)] = 0
        c = dict(n=n, k=k)
        if t5b:
            scale = 0.017 + 0.003 * i
            c["dw"] = B.DeviceWeights(B.pack_t5b(w, scale), dev)
            c["scale"] = scale
        else:
            c["s"] = synth.scales(n, k // 128, seed=s_)
            c["st"] = torch.from_numpy(c["s"]).to(dev)
            c["dw"] = B.DeviceWeights(B.pack(fmt, w), dev)
        if out == "f16":
            x16 = synth.float_activations(m, k, seed=s_).astype(np.float16)
            c["x"] = torch.from_numpy(x16).to(dev)
            c["y_ref"] = O.gemv_f16(w, c["s"], x16)
            c["bound"] = bounds.f16_bound(w, c["s"], x16, c["y_ref"])
        elif out == "xs":
            xf = synth.float_activations(m, k, seed=s_)
            xq_ref, c["xs_ref"] = O.quantize_x(xf)
            c["acc"] = O.gemv_acc(w, xq_ref)
            c["y_ref"] = O.combine_xs(c["acc"], c["s"], c["xs_ref"])
            c["x"], c["xs"] = B.quantize_x(torch.from_numpy(xf).to(dev))
        else:
            x = synth.activations(m, k, seed=s_)
            c["x"] = torch.from_numpy(x).to(dev)
            if t5b:
                c["acc"] = O.gemv_acc_blocks(w, x)
                c["y_ref"] = O.combine_tensor(c["acc"], c["scale"])
            else:
                c["acc"] = O.gemv_acc(w, x)
                c["y_ref"] = O.combine(c["acc"], c["s"])
        cases.append(c)
        del w
    dws, xs = [c["dw"] for c in cases], [c["x"] for c in cases]
    if out == "acc":
        res = [torch.full((m, c["n"], B.groups_per_row(fmt, c["k"])), -7, dtype=torch.int32, device=dev) for c in cases]
        plan = B.Plan(dws, xs, accs=res)
    else:
        res = [torch.full((m, c["n"]), float("nan"), dtype=torch.float32, device=dev) for c in cases]
        sc = None if t5b else [c["st"] for c in cases]
        plan = B.Plan(dws, xs, scales=sc, ys=res, x_scales=[c["xs"] for c in cases] if out == "xs" else None,
                      f16=out == "f16")
    if out != "f16":
        plan.set_decode(decode)
    for _ in range(2):  # twice: nothing may depend on what the previous launch left
        plan.run()
    torch.cuda.synchronize()
    for j, (c, r) in enumerate(zip(cases, res)):
        label = f"GEMV {j} ({c['n']}x{c['k']}, {shapes[j]})"
        got = r.cpu().numpy()
        if out == "acc":
            assert np.array_equal(got, c["acc"]), f"{label}: int32 sums differ"
        elif out == "f16":
            err = np.abs(got.astype(np.float64) - c["y_ref"].astype(np.float64))
            assert np.all(err <= c["bound"]), f"{label}: outside the fp16 bound"
        elif out == "xs":
            ok, nd = bounds.int8_y_ok(got, c["y_ref"], c["acc"], c["s"], c["xs_ref"])
            assert ok, f"{label}: outside the bound ({nd} differ)"
        elif t5b:
            ok, nd = bounds.tensor_y_ok(got, c["y_ref"], c["acc"], c["scale"])
            assert ok, f"{label}: outside the bound ({nd} differ)"
        else:
            ok, nd = bounds.int8_y_ok(got, c["y_ref"], c["acc"], c["s"])
            assert ok, f"{label}: outside the bound ({nd} differ)"
            if fmt == B.FMT_BITCOS:
                assert nd == 0, f"{label}: {nd} outputs not bit-identical"
