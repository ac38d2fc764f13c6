"""Pins of the oracle's per-group int8 activation quantisation and of the GEMV that applies the
activation group scales (no GPU).

The int8 path of "Breaking the 1.58-bit Barrier for Ternary LLMs" (Sec. II-C, discussion after
Fig. 5) quantises activations to int8 per group of 128 and applies group scales once per group; the
quantiser itself is not spelled out. The reading pinned here: symmetric absmax per group, sigma =
max|x| / 127 and codes x / sigma rounded to nearest-even (both in fp32), clamped to [-127, 127].
Closed forms (sigma = 1 and sigma = 2 exactly, ties to even), invariants, and reduction to the
pinned integer GEMV catch a wrong divisor, a wrong rounding rule, a per-row instead of per-group
scale, a transposed group index or a misapplied activation scale.
"""
import numpy as np

import oracle as O
from bit_gemv_decode_amd import synth


def _group(vals, fill=0.0):
    g = np.full(128, fill, np.float32)
    g[: len(vals)] = vals
    return g


def test_sigma_one_codes_are_round_half_even_of_x():
    # max|x| = 127 gives sigma = 127 / 127 = 1 exactly, so every code is x rounded to nearest-even.
    x = _group([127.0, -3.5, 2.5, 0.49, -0.5, 100.2, -126.5, 1.5, -127.0])[None, :]
    q, s = O.quantize_x(x)
    assert s.tolist() == [[1.0]]
    assert q[0, :9].tolist() == [127, -4, 2, 0, 0, 100, -126, 2, -127]
    assert not q[0, 9:].any()


def test_sigma_two_halves_the_codes():
    # max|x| = 254 gives sigma = 2 exactly; x / 2 is exact, then rounded to nearest-even.
    x = _group([254.0, 5.0, 7.0, -3.0, 1.0, -254.0, 9.0])[None, :]
    q, s = O.quantize_x(x)
    assert s.tolist() == [[2.0]]
    assert q[0, :7].tolist() == [127, 2, 4, -2, 0, -127, 4]


def test_zero_group_has_zero_scale_and_codes():
    x = np.concatenate([_group([]), _group([-0.0, 0.0]), _group([127.0])])[None, :]
    q, s = O.quantize_x(x)
    assert s.tolist() == [[0.0, 0.0, 1.0]]
    assert not q[0, :256].any() and q[0, 256] == 127


def test_group_and_row_boundaries():
    # group g covers k in [128 g, 128 g + 128) of one activation row and nothing else
    x = np.zeros((2, 384), np.float32)
    x[0, 127] = 127.0   # last element of group 0
    x[0, 128] = 254.0   # first element of group 1
    x[0, 200] = 3.0
    x[1, 300] = -127.0  # group 2 of row 1
    q, s = O.quantize_x(x)
    assert s.tolist() == [[1.0, 2.0, 0.0], [0.0, 0.0, 1.0]]
    assert q[0, 127] == 127 and q[0, 128] == 127 and q[0, 200] == 2 and q[1, 300] == -127
    assert np.count_nonzero(q) == 4


def test_invariants_on_seeded_activations():
    x = synth.float_activations(3, 4096, seed=1)
    q, s = O.quantize_x(x)
    g = x.reshape(3, 32, 128).astype(np.float64)
    qg = q.reshape(3, 32, 128).astype(np.int64)
    sg = s.astype(np.float64)[..., None]
    assert (np.abs(qg) <= 127).all()
    # the largest magnitude of every group lands on +-127, with its sign
    amax = np.abs(g).argmax(-1)
    top = np.take_along_axis(qg, amax[..., None], -1)[..., 0]
    assert (np.abs(top) == 127).all()
    assert (np.sign(top) == np.sign(np.take_along_axis(g, amax[..., None], -1)[..., 0])).all()
    # each code is within half a step of x / sigma (plus fp32 rounding of the quotient)
    err = np.abs(g - qg * sg)
    assert (err <= sg * (0.5 + 1e-6)).all()
    # codes never flip sign
    assert (qg * np.sign(g) >= 0).all()
    # sigma is the group's max magnitude over 127, within fp32 rounding
    ref = np.abs(g).max(-1) / 127.0
    assert np.allclose(s, ref, rtol=2**-23, atol=0)


def test_power_of_two_scaling_keeps_codes():
    x = synth.float_activations(2, 1024, seed=2)
    q, s = O.quantize_x(x)
    for j in (-3, 5):
        q2, s2 = O.quantize_x(x * np.float32(2.0**j))
        assert (q2 == q).all()
        assert (s2 == s * np.float32(2.0**j)).all()


def test_gemv_xs_reduces_to_integer_gemv_when_sigma_is_one():
    # integer-valued activations whose every group holds a +-127 quantise to themselves with sigma 1,
    # so the activation-scaled GEMV equals the pinned integer-activation GEMV bit for bit
    n, k = 40, 1024
    w = synth.ternary(n, k, 0.4, seed=3)
    sc = synth.scales(n, k // 128, seed=3)
    xi = synth.activations(2, k, seed=3).astype(np.int16)
    xi[:, ::128] = 127
    xi[1, 5::128] = -127
    xf = xi.astype(np.float32)
    q, s = O.quantize_x(xf)
    assert (s == 1.0).all() and (q == xi).all()
    assert (O.gemv_xs(w, sc, xf) == O.gemv(w, sc, xi.astype(np.int8))).all()


def test_gemv_xs_close_to_dequantised_dense_product():
    # y differs from the dense product W (scale * x) by at most half a quantisation step per weight
    n, k = 24, 2048
    w = synth.ternary(n, k, 0.45, seed=4)
    sc = synth.scales(n, k // 128, seed=4)
    x = synth.float_activations(2, k, seed=4)
    _, s = O.quantize_x(x)
    y = O.gemv_xs(w, sc, x).astype(np.float64)
    wd = w.astype(np.float64) * np.repeat(sc.astype(np.float64), 128, axis=1)  # dequantised W
    dense = x.astype(np.float64) @ wd.T
    bound = (np.abs(wd).reshape(n, -1, 128).sum(-1)[None] * s.astype(np.float64)[:, None, :] * 0.5).sum(-1)
    assert (np.abs(y - dense) <= bound * (1 + 1e-5) + 1e-5 * np.abs(dense)).all()
    # and the quantisation error is a small fraction of the output scale
    assert np.abs(y - dense).max() < 0.05 * np.abs(dense).max()


def test_combine_xs_scales_each_group_independently():
    n, k = 8, 512
    w = synth.ternary(n, k, 0.3, seed=5)
    sc = synth.scales(n, k // 128, seed=5)
    xq = synth.activations(1, k, seed=5)
    acc = O.gemv_acc(w, xq)
    ones = np.ones((1, 4), np.float32)
    assert (O.combine_xs(acc, sc, ones) == O.combine(acc, sc)).all()
    # doubling every group scale doubles y exactly; scaling one group moves only that group's share
    assert (O.combine_xs(acc, sc, 2 * ones) == 2 * O.combine(acc, sc)).all()
    only2 = np.array([[0, 0, 1, 0]], np.float32)
    ref = (acc[0, :, 2].astype(np.float64) * sc[:, 2].astype(np.float64)).astype(np.float32)
    assert (O.combine_xs(acc, sc, only2)[0] == ref).all()
