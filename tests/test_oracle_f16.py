"""Pins of the oracle's GEMV against fp16 activations ("Breaking the 1.58-bit Barrier for Ternary
LLMs", Sec. II-B: the weights are rebuilt as +-s or 0 in 16-bit floating point and multiplied with the
activations; Sec. II-D: the Xe2 lookup entries hold fp16 weights).

The oracle computes y = (float) sum_g s_g * sum_{k in g} W x exactly up to the final rounding. The
checks pin it by reduction to the int8 GEMV, a closed form for one activation, exact rational
arithmetic on tiny inputs and symmetry.
"""
from fractions import Fraction

import numpy as np

import oracle as O
from bit_gemv_decode_amd import synth


def test_integer_activations_reduce_to_the_int8_gemv():
    w = synth.ternary(33, 1024, 0.4, seed=1)
    s = synth.scales(33, 8, seed=1)
    x8 = synth.activations(3, 1024, seed=1)
    assert np.array_equal(O.gemv_f16(w, s, x8.astype(np.float16)), O.gemv(w, s, x8))


def test_unit_scales_give_the_integer_matvec():
    w = synth.ternary(20, 640, 0.3, seed=2)
    x = synth.activations(2, 640, seed=2).astype(np.float16)
    s = np.ones((20, 5), np.float16)
    dense = (x.astype(np.int64) @ w.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(O.gemv_f16(w, s, x), dense)


def test_single_activation_closed_form():
    w = synth.ternary(9, 256, 0.4, seed=3)
    s = synth.scales(9, 2, seed=3)
    x = np.zeros((1, 256), np.float16)
    x[0, 200] = np.float16(-3.140625)
    want = (s[:, 1].astype(np.float64) * w[:, 200].astype(np.float64) * -3.140625).astype(np.float32)
    assert np.array_equal(O.gemv_f16(w, s, x)[0], want)


def test_exact_sums_over_the_whole_fp16_range():
    # subnormals, the largest normal and values in between: the definition is computed with exact
    # rationals and rounded once
    rng = np.random.default_rng(4)
    n, k = 5, 256
    w = synth.ternary(n, k, 0.2, seed=4)
    bits = rng.integers(0, 0x7C00, size=(1, k), dtype=np.uint16)  # every finite non-negative fp16
    bits[0, :8] = [0x0001, 0x0002, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0x0000, 0x7BFE]
    sign = rng.integers(0, 2, size=(1, k), dtype=np.uint16) << 15
    x = (bits | sign).view(np.float16)
    s = synth.scales(n, 2, seed=4)
    y = O.gemv_f16(w, s, x)
    for r in range(n):
        tot = Fraction(0)
        for g in range(2):
            grp = sum(Fraction(int(w[r, c])) * Fraction(float(x[0, c])) for c in range(128 * g, 128 * g + 128))
            tot += Fraction(float(s[r, g])) * grp
        assert y[0, r] == np.float32(float(tot))


def test_odd_symmetry_and_power_of_two_scaling():
    w = synth.ternary(17, 2048, 0.4, seed=5)
    s = synth.scales(17, 16, seed=5)
    x = (synth.float_activations(2, 2048, seed=5)).astype(np.float16)
    y = O.gemv_f16(w, s, x)
    assert np.array_equal(O.gemv_f16(w, s, -x), -y)
    assert np.array_equal(O.gemv_f16(w, s, (x.astype(np.float32) * 4).astype(np.float16)), y * 4)
