"""GPU parity of GEMVs whose rows hold one, two or four 128-weight groups (k = 128, 256, 512), in
grouped launches large enough that every wave's range holds several units.

A step of the vector kernels covers R = 64 / (k / 128) rows, one group per lane, and a unit is a fixed
number of steps whose row sums are reduced together at its end. Each of the 64 GEMVs here has its own
output, so that a row left unwritten in one of them cannot be covered by another; outputs start as NaN.
Every output must equal the oracle's ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C:
int32 group sums, the scale applied once per group), bit for bit in practice and within the stated
bound in any case.
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

N, COPIES = 8192, 64


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("m", [1, 2, 3])
@pytest.mark.parametrize("k", [128, 256, 512])
@pytest.mark.parametrize("fmt", [B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT], ids=["bitcos", "5trit", "2bit"])
def test_short_rows_in_multi_unit_ranges(fmt, k, m):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    seed = 7000 + k + 10 * m + fmt
    w = synth.ternary(N, k, 0.4, seed=seed)
    x = synth.activations(m, k, seed=seed)
    s = synth.scales(N, k // 128, seed=seed)
    acc_ref = O.gemv_acc(w, x)
    y_ref = O.combine(acc_ref, s)
    _say(f"[gpu] short rows fmt={B.FMT_NAMES[fmt]} k={k} m={m}: {COPIES} x {N} rows, one launch")
    dw = B.DeviceWeights(B.pack(fmt, w), dev)
    xt = torch.from_numpy(x).to(dev)
    st = torch.from_numpy(s).to(dev)
    ys = [torch.full((m, N), float("nan"), dtype=torch.float32, device=dev) for _ in range(COPIES)]
    B.Plan([dw] * COPIES, [xt] * COPIES, scales=[st] * COPIES, ys=ys).run()
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        y_np = y.cpu().numpy()
        missing = int(np.isnan(y_np).sum())
        assert missing == 0, f"GEMV {i}: {missing} outputs never written"
        ok, ndiff = bounds.int8_y_ok(y_np, y_ref, acc_ref, s)
        assert ok, f"GEMV {i}: outputs outside the bound ({ndiff} differ)"
