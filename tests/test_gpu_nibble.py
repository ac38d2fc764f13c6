"""GPU parity of the nibble-keyed BITCOS decode ("Breaking the 1.58-bit Barrier for Ternary LLMs",
Sec. II-D, Eq. 4), selected per plan with tg_plan_set_decode.

Its int32 group sums must match the oracle bit for bit, and its fp32 outputs must be identical to the
byte-keyed decode's (both add the same exact fp64 terms in the same order) and within the stated
tolerance of the oracle.
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


def y_ok(y, y_ref, acc, scales):
    return bounds.int8_y_ok(y, y_ref, acc, scales)[0]


# single-chunk rows of every step width (k = 128 .. 8192), ragged row counts, chunked rows (k > 8192)
# with a one-group last pass, all-zero and all-nonzero weights
SHAPES_A = [(96, 4096, 0.4), (40, 5120, 0.47), (33, 14336, 0.44), (7, 2560, 0.0), (130, 1024, 1.0),
            (1, 128, 0.42), (9, 25600, 0.47), (65, 8320, 0.3), (300, 8192, 0.515), (5, 640, 0.95)]
# a small plan of chunked rows only: fewer coarse units than waves, so the fine 2-row units
SHAPES_B = [(17, 14336, 0.44), (5, 16512, 0.4)]


@pytest.mark.parametrize("shapes", [SHAPES_A, SHAPES_B], ids=["mixed", "chunked_fine"])
def test_nibble_decode_matches_oracle_and_byte_decode(shapes):
    dev = _dev()
    _say(f"[gpu] nibble decode plan, {len(shapes)} GEMVs")
    dws, ss, xs, refs = [], [], [], []
    for i, (n, k, z) in enumerate(shapes):
        w = synth.ternary(n, k, z, seed=1300 + i)
        s = synth.scales(n, k // 128, seed=1300 + i)
        x = synth.activations(1, k, seed=1350 + i)
        acc_ref = O.gemv_acc(w, x)
        refs.append((acc_ref, O.combine(acc_ref, s), s))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        ss.append(torch.from_numpy(s).to(dev))
        xs.append(torch.from_numpy(x).to(dev))
    out = {}
    for decode in (B.DECODE_BYTE, B.DECODE_NIBBLE):
        ys = [torch.full((1, n), float("nan"), dtype=torch.float32, device=dev) for n, _, _ in shapes]
        accs = [torch.full((1, n, k // 128), -7, dtype=torch.int32, device=dev) for n, k, _ in shapes]
        B.Plan(dws, xs, scales=ss, ys=ys).set_decode(decode).run()
        B.Plan(dws, xs, accs=accs).set_decode(decode).run()
        torch.cuda.synchronize()
        out[decode] = ([y.cpu().numpy() for y in ys], [a.cpu().numpy() for a in accs])
    for i, (n, k, z) in enumerate(shapes):
        acc_ref, y_ref, s = refs[i]
        y_nib, acc_nib = out[B.DECODE_NIBBLE][0][i], out[B.DECODE_NIBBLE][1][i]
        assert np.array_equal(acc_nib, acc_ref), f"nibble acc {n}x{k}"
        assert y_ok(y_nib, y_ref, acc_ref, s), f"nibble y {n}x{k}"
        assert np.array_equal(y_nib, out[B.DECODE_BYTE][0][i]), f"nibble y differs from byte decode {n}x{k}"


def test_nibble_decode_llama3_8b_layer():
    dev = _dev()
    _say("[gpu] nibble decode, one Llama3-8B layer")
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
    dws, ss, xs, ys, refs = [], [], [], [], []
    for role, (n, k) in enumerate(shapes):
        w = synth.ternary(n, k, 0.40, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        s = synth.scales(n, k // 128, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_SCALE))
        x = synth.activations(1, k, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_X))
        refs.append(O.gemv_acc(w, x))
        dws.append(B.DeviceWeights(B.pack_bitcos(w), dev))
        xs.append(torch.from_numpy(x).to(dev))
        ys.append(torch.empty((1, n, k // 128), dtype=torch.int32, device=dev))
    B.Plan(dws, xs, accs=ys).set_decode(B.DECODE_NIBBLE).run()
    torch.cuda.synchronize()
    for role, (n, k) in enumerate(shapes):
        assert np.array_equal(ys[role].cpu().numpy(), refs[role]), f"role {role}"
