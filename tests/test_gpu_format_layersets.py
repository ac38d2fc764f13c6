"""Parity of the fixed-code formats' layer-set launches that bench.py times: the Llama3-8B-shaped layer
set stored 32 times (224 GEMVs in one grouped launch, every wave's range holding many units, the
4096 x 14336 rows chunked) in five-trit, 2-bit and t5b, each with the LDS-table decode and with the
table-free decode. The copies hold the same bytes, so the oracle computes the 7 distinct GEMVs and
every output of every copy is checked against them ("Breaking the 1.58-bit Barrier for Ternary
LLMs", Sec. II-C: int32 group sums, the scale applied once per group; t5b: one scale per tensor, the
sub-two-bit page's block code), within the stated bound and bit-identical in practice.
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


@pytest.mark.parametrize("fmt", [B.FMT_5TRIT, B.FMT_2BIT, B.FMT_T5B], ids=["5trit", "2bit", "t5b"])
def test_format_layer_set_every_output(fmt):
    import bench

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    _say(f"[gpu] {B.FMT_NAMES[fmt]} layer set: packing and storing 32 copies")
    ls = bench.LayerSet(B, synth, torch, dev, fmt)
    refs = []
    for role, (name, n, k) in enumerate(bench.LAYER):
        w = synth.ternary(n, k, bench.Z, seed=0, tid=synth.tensor_id(0, role, synth.STREAM_W))
        x = ls.host[role]["x"]
        if fmt == B.FMT_T5B:
            acc = O.gemv_acc_blocks(w, x)
            refs.append((acc, O.combine_tensor(acc, bench.T5B_SCALE), None))
        else:
            acc = O.gemv_acc(w, x)
            s = ls.host[role]["s"]
            refs.append((acc, O.combine(acc, s), s))
        del w
    for decode in (B.DECODE_BYTE, B.DECODE_ARITH):
        _say(f"[gpu] {B.FMT_NAMES[fmt]} layer set, decode={decode}, one launch of {7 * bench.LAYERS} GEMVs")
        plan = ls.plan(B).set_decode(decode)
        for m in ls.flat():
            m["y"].fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        for role, (name, n, k) in enumerate(bench.LAYER):
            acc, y_ref, s = refs[role]
            for layer in range(bench.LAYERS):
                y = ls.mats[layer][role]["y"].cpu().numpy()
                if fmt == B.FMT_T5B:
                    ok = bounds.tensor_y_ok(y, y_ref, acc, bench.T5B_SCALE)[0]
                else:
                    ok = bounds.int8_y_ok(y, y_ref, acc, s)[0]
                assert ok, f"{name} copy {layer}, decode {decode}: outside the bound"
                assert np.array_equal(y, y_ref), f"{name} copy {layer}, decode {decode}: not bit-identical"
        del plan
    del ls
    torch.cuda.empty_cache()
