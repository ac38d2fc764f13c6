"""Pins of the oracle's t5b format (five-trit bytes in blocks of 160 weights, one scale per tensor).

"Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract: the same base-3
construction as the five-trit code, at a block length of 160 weights, 1.600 bits per weight, with the
scale carried once per tensor. The oracle's readings: blocks run along each row; byte j of block b
holds weights 160b + 5j .. 160b + 5j + 4 as digits weight + 1, the first weight least significant;
positions past k are padding digits of value 1. The checks below fix them by the page's figures,
closed forms, exhaustive enumeration and agreement with independently computed quantities.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from bit_gemv_decode_amd import synth


def test_bits_per_weight_is_1_600():
    # 32 bytes per 160 weights: 256 / 160 = 1.6 exactly (the page's figure)
    for k in (160, 320, 2560, 6400):
        codes = O.t5b_pack(np.zeros((1, k), np.int8))
        assert codes.size * 8 / k == 1.6
    assert 3 ** 5 == 243 <= 256 and 160 // 5 == 32


def test_digit_order_worked_byte():
    # weights (+1, 0, -1, 0, 0): digits (2, 1, 0, 1, 1), first weight least significant:
    # 2 + 1*3 + 0*9 + 1*27 + 1*81 = 113
    w = np.zeros((1, 160), np.int8)
    w[0, :5] = [1, 0, -1, 0, 0]
    assert O.t5b_pack(w)[0, 0, 0] == 113
    # an all-zero block is 32 bytes of digit 1 everywhere: 1 + 3 + 9 + 27 + 81 = 121
    assert np.all(O.t5b_pack(np.zeros((1, 160), np.int8)) == 121)


def test_exhaustive_byte_values_round_trip():
    # every 5-weight pattern (3^5 = 243) placed at byte position j of a block, for every j
    pats = np.array(list(itertools.product([-1, 0, 1], repeat=5)), np.int8)  # 243 x 5
    vals = np.array([sum((int(p[i]) + 1) * 3 ** i for i in range(5)) for p in pats])
    assert sorted(vals) == list(range(243))
    for j in (0, 13, 31):
        w = np.zeros((243, 160), np.int8)
        w[:, 5 * j:5 * j + 5] = pats
        codes = O.t5b_pack(w)
        assert np.array_equal(codes[:, 0, j], vals)
        assert np.array_equal(O.t5b_unpack(codes, 243, 160), w)


def test_invalid_bytes_and_padding_rejected():
    codes = O.t5b_pack(np.zeros((1, 160), np.int8))
    for bad in (243, 250, 255):
        c = codes.copy()
        c[0, 0, 7] = bad
        with pytest.raises(ValueError):
            O.t5b_unpack(c, 1, 160)
    # k = 128: the block's last 32 positions are padding and must hold the weight-0 digit
    c = O.t5b_pack(np.zeros((1, 128), np.int8))
    assert np.all(c[0, 0, 26:] == 121)
    c2 = c.copy()
    c2[0, 0, 30] = 120  # first padding digit 0 instead of 1
    with pytest.raises(ValueError):
        O.t5b_unpack(c2, 1, 128)


@pytest.mark.parametrize("n,k,z", [(7, 128, 0.4), (5, 160, 0.0), (9, 4096, 0.42), (3, 14336, 1.0), (4, 640, 0.3)])
def test_round_trip_and_padding(n, k, z):
    w = synth.ternary(n, k, z, seed=n + k)
    codes = O.t5b_pack(w)
    assert codes.shape == (n, -(-k // 160), 32)
    assert np.array_equal(O.t5b_unpack(codes, n, k), w)


def test_same_bytes_as_the_128_block_code_where_spans_coincide():
    # both codes put weights 5j .. 5j + 4 of a row start into byte j: for j < 25 (weights < 125)
    # the bytes of t5b block 0 equal those of the five-trit 128-block 0
    w = synth.ternary(11, 1280, 0.4, seed=3)
    t5b = O.t5b_pack(w)
    t5 = O.t5_pack(w).reshape(11, 10, 26)
    assert np.array_equal(t5b[:, 0, :25], t5[:, 0, :25])


def test_block_sums_agree_with_group_sums_and_dense_product():
    w = synth.ternary(17, 4096, 0.4, seed=5)
    x = synth.activations(3, 4096, seed=5)
    accb = O.gemv_acc_blocks(w, x)
    assert accb.shape == (3, 17, 26)
    dense = x.astype(np.int64) @ w.T.astype(np.int64)  # [m, n]
    assert np.array_equal(accb.sum(-1), dense)
    assert np.array_equal(O.gemv_acc(w, x).sum(-1), dense)
    # a block's sum is the dense product over its columns (the last block is 96 wide)
    assert np.array_equal(accb[:, :, 25], x[:, 4000:].astype(np.int64) @ w[:, 4000:].T.astype(np.int64))


def test_per_tensor_scale_combine():
    w = synth.ternary(13, 2560, 0.42, seed=8)
    x = synth.activations(2, 2560, seed=8)
    acc = O.gemv_acc_blocks(w, x)
    dense = (x.astype(np.int64) @ w.T.astype(np.int64)).astype(np.float64)
    # scale 1: the integer matvec exactly
    assert np.array_equal(O.combine_tensor(acc, 1.0), dense.astype(np.float32))
    # any scale: the fp64 product of scale and the exact row sum, rounded once
    s = np.float32(0.0371)
    assert np.array_equal(O.combine_tensor(acc, s), (float(s) * dense).astype(np.float32))
    # linearity in the scale and odd symmetry in x
    assert np.array_equal(O.combine_tensor(O.gemv_acc_blocks(w, -x), s), -O.combine_tensor(acc, s))
