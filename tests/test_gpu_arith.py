"""GPU parity of the table-free decode (TG_DECODE_ARITH): for the five-trit code (26-byte groups) and t5b
(32-byte blocks) each base-3 digit of a code byte by multiply and shift (the depth-one decode of
"Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract); for 2-bit the codes
isolated by shift and mask and contracted as they are ("Breaking the 1.58-bit Barrier for Ternary LLMs",
Sec. II-C: 2-bit expansion by shift, mask and subtract).

The int32 group (block) sums must match the oracle bit for bit, and the fp32 outputs must be
identical to the table decode's (both add the same exact fp64 terms in the same order) and within the
stated bound of the oracle. Random weights at these sizes produce every one of the 243 code bytes;
all-zero, all-non-zero and extreme activations pin the digit ends (codes 0, 121, 242).
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


# single-chunk rows of several step widths, ragged row counts, chunked rows (more than 64 groups or
# blocks: 14336 and 25600), all-zero and all-non-zero weights
SHAPES = [(96, 4096, 0.4), (40, 5120, 0.47), (33, 14336, 0.44), (7, 2560, 0.0), (130, 1024, 1.0),
          (1, 128, 0.42), (9, 25600, 0.47), (300, 8192, 0.515), (5, 640, 0.95), (257, 4224, 0.33)]


def _case(fmt, n, k, z, i):
    w = synth.ternary(n, k, z, seed=1700 + i)
    x = synth.activations(1, k, seed=1750 + i)
    if i == 3:
        x[:] = -128
    elif i == 4:
        x[:] = 127
    if fmt in (B.FMT_5TRIT, B.FMT_2BIT):
        s = synth.scales(n, k // 128, seed=1700 + i)
        acc_ref = O.gemv_acc(w, x)
        return w, x, s, acc_ref, O.combine(acc_ref, s), B.pack_5trit(w) if fmt == B.FMT_5TRIT else B.pack_2bit(w)
    scale = 0.0213 + 0.001 * i
    acc_ref = O.gemv_acc_blocks(w, x)
    return w, x, scale, acc_ref, O.combine_tensor(acc_ref, scale), B.pack_t5b(w, scale)


@pytest.mark.parametrize("fmt", [B.FMT_5TRIT, B.FMT_T5B, B.FMT_2BIT], ids=["5trit", "t5b", "2bit"])
def test_arith_decode_matches_oracle_and_table_decode(fmt):
    dev = _dev()
    _say(f"[gpu] table-free decode plan, fmt={fmt}, {len(SHAPES)} GEMVs")
    cases = [_case(fmt, n, k, z, i) for i, (n, k, z) in enumerate(SHAPES)]
    dws = [B.DeviceWeights(c[5], dev) for c in cases]
    xs = [torch.from_numpy(c[1]).to(dev) for c in cases]
    ss = None if fmt == B.FMT_T5B else [torch.from_numpy(c[2]).to(dev) for c in cases]
    out = {}
    for decode in (B.DECODE_BYTE, B.DECODE_ARITH):
        ys = [torch.full((1, n), float("nan"), dtype=torch.float32, device=dev) for n, _, _ in SHAPES]
        accs = [torch.full((1, n, B.groups_per_row(fmt, k)), -7, dtype=torch.int32, device=dev) for n, k, _ in SHAPES]
        py = B.Plan(dws, xs, scales=ss, ys=ys).set_decode(decode)
        pa = B.Plan(dws, xs, accs=accs).set_decode(decode)
        for rep in range(2):  # twice: nothing may depend on what the previous launch left
            py.run()
            pa.run()
        torch.cuda.synchronize()
        out[decode] = ([y.cpu().numpy() for y in ys], [a.cpu().numpy() for a in accs])
    for i, (n, k, z) in enumerate(SHAPES):
        w, x, s, acc_ref, y_ref, _ = cases[i]
        y_a, acc_a = out[B.DECODE_ARITH][0][i], out[B.DECODE_ARITH][1][i]
        assert np.array_equal(acc_a, acc_ref), f"table-free acc {n}x{k}"
        if fmt == B.FMT_T5B:
            ok, _ = bounds.tensor_y_ok(y_a, y_ref, acc_ref, s)
        else:
            ok, _ = bounds.int8_y_ok(y_a, y_ref, acc_ref, s)
        assert ok, f"table-free y {n}x{k}"
        assert np.array_equal(y_a, out[B.DECODE_BYTE][0][i]), f"table-free y differs from table decode {n}x{k}"


def test_arith_decode_every_code_byte():
    # every code value 0..242 as a whole code byte: code c at slot c % 25 of group c // 25 (a 128-weight
    # group holds 25 whole codes and a three-weight one), its weights the code's base-3 digits minus 1;
    # the second row holds the negated weights (digits 2 - d), the third all zeros (code 121)
    dev = _dev()
    k = 10 * 128
    w = np.zeros((3, k), np.int8)
    for c in range(243):
        v, base = c, 128 * (c // 25) + 5 * (c % 25)
        for i in range(5):
            w[0, base + i] = v % 3 - 1
            v //= 3
    w[1] = -w[0]
    x = ((np.arange(k) * 37) % 255 - 127).astype(np.int8)[None, :]
    acc_ref = O.gemv_acc(w, x)
    dw = B.DeviceWeights(B.pack_5trit(w), dev)
    acc = torch.full((1, 3, k // 128), -7, dtype=torch.int32, device=dev)
    B.Plan([dw], [torch.from_numpy(x).to(dev)], accs=[acc]).set_decode(B.DECODE_ARITH).run()
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)


def test_2bit_plans_and_calls_default_to_the_table_free_decode():
    # a new 2-bit plan that may take the table-free decode starts with it (m = 1, fp32 or int32 outputs);
    # plans it cannot serve (m = 2, activation group scales) and the other formats start with the table;
    # single calls give the same results as the plans
    dev = _dev()
    n, k = 300, 4224
    w = synth.ternary(n, k, 0.4, seed=1901)
    x = synth.activations(2, k, seed=1901)
    s = synth.scales(n, k // 128, seed=1901)
    acc_ref = O.gemv_acc(w, x[:1])
    y_ref = O.combine(acc_ref, s)
    dw = B.DeviceWeights(B.pack_2bit(w), dev)
    xt, st = torch.from_numpy(x[:1].copy()).to(dev), torch.from_numpy(s).to(dev)
    y = torch.full((1, n), float("nan"), dtype=torch.float32, device=dev)
    acc = torch.full((1, n, k // 128), -7, dtype=torch.int32, device=dev)
    py = B.Plan([dw], [xt], scales=[st], ys=[y])
    pa = B.Plan([dw], [xt], accs=[acc])
    assert py.plan.decode == B.DECODE_ARITH and pa.plan.decode == B.DECODE_ARITH
    y2 = torch.empty((2, n), dtype=torch.float32, device=dev)
    assert B.Plan([dw], [torch.from_numpy(x).to(dev)], scales=[st], ys=[y2]).plan.decode == B.DECODE_BYTE
    xq, xs = B.quantize_x(torch.from_numpy(synth.float_activations(1, k, seed=1901)).to(dev))
    assert B.Plan([dw], [xq], scales=[st], ys=[y], x_scales=[xs]).plan.decode == B.DECODE_BYTE
    dw5 = B.DeviceWeights(B.pack_5trit(w), dev)
    assert B.Plan([dw5], [xt], scales=[st], ys=[y]).plan.decode == B.DECODE_BYTE
    py.run()
    pa.run()
    y_call = B.ternary_gemv(dw, st, xt)
    acc_call = B.ternary_gemv_acc(dw, xt)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref) and np.array_equal(acc_call.cpu().numpy(), acc_ref)
    assert bounds.int8_y_ok(y.cpu().numpy(), y_ref, acc_ref, s)[0]
    assert np.array_equal(y_call.cpu().numpy(), y.cpu().numpy())
