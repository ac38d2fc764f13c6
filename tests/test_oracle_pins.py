"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test checks the oracle against a value the pages print, a closed form, an invariant, a textbook
routine (numpy's integer matmul) or brute force, so that a dropped term, a wrong sign, a swapped bit
order or a transposed operand in the oracle fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from bit_gemv_decode_amd import synth
from tests.conftest import read_golden, read_table


def _bits_lsb(buf, count):
    return [(int(buf[i >> 3]) >> (i & 7)) & 1 for i in range(count)]


# --- Eq. (2)-(3) worked example (bit order, polarity, compaction) ---------------------------

def test_eq3_column_packs_to_printed_bitmap_and_signs():
    g = read_golden("eq3_column.txt")
    vals = np.array([[int(v) for v in g["values"].split()]], np.int8)
    b = O.bitcos_pack(vals)
    assert int(b.bitmap[0]) == int(g["bitmap"], 16)
    assert _bits_lsb(b.bitmap, 8) == [int(v) for v in g["p"].split()]
    stored = [int(v) for v in g["stored_signs"].split()]
    assert b.nnz == len(stored) == 7
    assert _bits_lsb(b.signs, b.nnz) == stored
    w, used = O.bitcos_unpack(b.bitmap, b.signs, 1, 8)
    assert used == 7
    assert bytes(w.view(np.uint8)[0]).hex(" ").upper() == g["unpacked_bytes"]


def test_eq3_predicates_match_unpacked_column():
    # w = p - 2n (Eq. 2) with the printed p and n gives the printed column.
    g = read_golden("eq3_column.txt")
    p = np.array([int(v) for v in g["p"].split()])
    n = np.array([int(v) for v in g["n"].split()])
    b = O.bitcos_pack(np.array([[int(v) for v in g["values"].split()]], np.int8))
    w, _ = O.bitcos_unpack(b.bitmap, b.signs, 1, 8)
    assert list(w[0]) == list(p - 2 * n)
    # n is the deposit of the stored signs onto the presence mask (the text after Eq. 3).
    stored = int("".join(reversed(g["stored_signs"].split())), 2)
    mask = int(g["bitmap"], 16)
    assert O.pdep64(stored, mask) == int("".join(reversed(g["n"].split())), 2)


# --- Fig. 4 pdep example ---------------------------------------------------------------------

def test_fig4_pdep_example():
    g = read_golden("fig4_pdep.txt")
    to_int = lambda s: sum(int(b) << i for i, b in enumerate(s.split()))
    mask, src, dst = to_int(g["mask_bits_lsb_first"]), to_int(g["src_bits_lsb_first"]), to_int(g["dst_bits_lsb_first"])
    assert O.pdep64(src, mask) == dst
    # Only popcount(mask) source bits are consumed: higher source bits change nothing.
    assert O.pdep64(src | (0xFFFF << 4), mask) == dst


def test_pdep_brute_force_small_masks():
    # pdep against its defining property on all 8-bit masks and sources: the j-th set bit of the mask
    # receives source bit j.
    for mask in range(256):
        pos = [i for i in range(8) if (mask >> i) & 1]
        for src in range(256):
            want = sum(((src >> j) & 1) << p for j, p in enumerate(pos))
            assert O.pdep64(src, mask) == want


# --- Eq. (4) / Fig. 7 / Fig. 9 LUT keys ------------------------------------------------------

def test_fig9_groups_unpack_to_printed_entries():
    g = read_golden("fig9_lut_keys.txt")
    k0, k1 = int(g["key0"], 16), int(g["key1"], 16)
    m0, s0, m1, s1 = k0 >> 4, k0 & 15, k1 >> 4, k1 & 15
    adv0 = int(g["advance0"])
    # Build one row of 8 weights: presence nibbles m0 then m1, sign stream s0's first adv0 bits, then s1.
    bitmap = np.array([m0 | (m1 << 4)], np.uint8)
    stream = [(s0 >> i) & 1 for i in range(adv0)] + [(s1 >> i) & 1 for i in range(4)]
    signs = np.array([sum(b << i for i, b in enumerate(stream))], np.uint8)
    w, used = O.bitcos_unpack(bitmap, signs, 1, 8)
    assert list(w[0, :4]) == [int(v) for v in g["entry0"].split()]
    assert list(w[0, 4:]) == [int(v) for v in g["entry1"].split()]
    assert bin(m0).count("1") == adv0 and bin(m1).count("1") == int(g["advance1"])
    assert used == adv0 + int(g["advance1"])


def test_eq4_table_matches_oracle_unpack_for_all_keys():
    # Eq. (4): c_i = 0 if m_i = 0, else +1/-1 by the compact sign at rank r_i = sum_{j<i} m_j.
    for key in range(256):
        m, s = key >> 4, key & 15
        ranks = [sum((m >> j) & 1 for j in range(i)) for i in range(4)]
        eq4 = [0 if not (m >> i) & 1 else (-1 if (s >> ranks[i]) & 1 else 1) for i in range(4)]
        w, used = O.bitcos_unpack(np.array([m], np.uint8), np.array([s], np.uint8), 1, 4)
        assert list(w[0]) == eq4, key
        assert used == bin(m).count("1")


# --- Fig. 2 counts and Eq. (1) -----------------------------------------------------------

def test_fig2_bit_counts():
    g = read_golden("fig2_counts.txt")
    n, k, zeros = int(g["rows"]), int(g["cols"]), int(g["zeros"])
    w = synth.exact_density_ternary(n, k, zeros, seed=7)
    b = O.bitcos_pack(w)
    assert n * k == int(g["presence_bits"]) and b.nnz == int(g["sign_bits"])
    assert round(b.symbol_bits() / (n * k), 3) == float(g["bits_per_weight"])
    assert round(zeros / (n * k), 3) == float(g["zero_density"])
    assert b.symbol_bits() / (n * k) < math.log2(3)


@pytest.mark.parametrize("z", [0.0, 0.1, 0.375, 0.42, 0.5148, 0.9, 1.0])
def test_eq1_symbol_bits_equal_two_minus_measured_z(z):
    n, k = 24, 256
    w = synth.ternary(n, k, z, seed=3)
    b = O.bitcos_pack(w)
    zm = float((w == 0).mean())
    assert b.symbol_bits() == n * k + int((w != 0).sum())
    assert b.symbol_bits() / (n * k) == pytest.approx(2 - zm, abs=1e-12)
    assert b.bitmap.size * 8 == n * k and b.signs.size == (b.nnz + 7) // 8


# --- Table I ----------------------------------------------------------------------------------

@pytest.mark.parametrize("row", read_table("table1_bitwidths.txt"), ids=lambda r: r[0])
def test_table1_bitwidths(row):
    name, zpct, sym, plus, two, red2, five, red5 = row
    zeros = int(round(float(zpct) * 100))  # zeros per 10000 weights, exact at the printed precision
    n, k = 10, 1000
    w = synth.exact_density_ternary(n, k, zeros, seed=11)
    b = O.bitcos_pack(w)
    assert abs(b.symbol_bits() / (n * k) - float(sym)) <= 0.0005 + 1e-12
    if plus != "-" and float(two) == 2.125:
        # group-128 fp16 checkpoints: measure every format with its fp16 scales, on a k=128-aligned tensor
        w2 = synth.exact_density_ternary(625, 128, zeros * 8, seed=11)  # 80000 weights, same density
        b2 = O.bitcos_pack(w2)
        nw = w2.size
        scale_bits = 16 * nw // 128
        bitcos = b2.symbol_bits() + scale_bits
        twobit = O.b2_pack(w2).size * 8 + scale_bits
        fivet = O.t5_pack(w2).size * 8 + scale_bits
        assert abs(bitcos / nw - float(plus)) <= 0.0005 + 1e-12
        assert abs(twobit / nw - float(two)) <= 0.0005 + 1e-12
        assert abs(fivet / nw - float(five)) <= 0.0005 + 1e-12
        assert abs(twobit / bitcos - float(red2)) <= 0.005 + 1e-12
        assert abs(fivet / bitcos - float(red5)) <= 0.005 + 1e-12


# --- five-trit arithmetic and the crossover -----------------------------------------------

def test_fivetrit_code_space_and_rate():
    g = read_golden("section1_fivetrit.txt")
    assert 3 ** 5 == int(g["codes"]) <= 256
    assert math.ceil(int(g["block"]) / 5) == int(g["block_bytes"])
    w = synth.ternary(3, 256, 0.3, seed=1)
    assert O.t5_pack(w).size * 8 / w.size == float(g["bits_per_weight"])


def test_fivetrit_all_codes_round_trip_and_invalid_bytes_rejected():
    # Every byte value < 243 is a valid code; its digits re-pack to the same byte.
    for v in range(243):
        digits = [(v // 3 ** i) % 3 for i in range(5)]
        w = np.zeros((1, 128), np.int8)
        w[0, :5] = np.array(digits) - 1
        codes = O.t5_pack(w)
        assert codes[0] == v
        assert list(O.t5_unpack(codes, 1, 128)[0, :5]) == [d - 1 for d in digits]
    base = O.t5_pack(np.zeros((1, 128), np.int8))
    for bad in range(243, 256):
        c = base.copy()
        c[3] = bad
        with pytest.raises(ValueError):
            O.t5_unpack(c, 1, 128)
    c = base.copy()
    c[25] = 0  # padding digits must encode weight 0
    with pytest.raises(ValueError):
        O.t5_unpack(c, 1, 128)


def test_fivetrit_tail_byte_layout():
    # byte 25 holds weights 125..127 as its first three digits, then two weight-0 pad digits.
    w = np.zeros((1, 128), np.int8)
    w[0, 125:128] = [1, -1, 1]
    codes = O.t5_pack(w)
    assert codes[25] == 2 + 0 * 3 + 2 * 9 + 1 * 27 + 1 * 81
    assert all(codes[:25] == 1 + 3 + 9 + 27 + 81)


def test_twobit_codes_and_invalid_code_rejected():
    w = np.array([[-1, 0, 1, 1] * 32], np.int8)
    codes = O.b2_pack(w)
    assert codes[0] == 0 | (1 << 2) | (2 << 4) | (2 << 6)
    bad = codes.copy()
    bad[5] |= 3 << 4
    with pytest.raises(ValueError):
        O.b2_unpack(bad, 1, 128)


def test_crossover_at_z_0375():
    g = read_golden("section1_fivetrit.txt")
    zc = float(g["crossover_z"])
    n, k = 8, 1024
    for zeros, sign in [(int(zc * n * k), 0), (int(zc * n * k) - 8, 1), (int(zc * n * k) + 8, -1)]:
        w = synth.exact_density_ternary(n, k, zeros, seed=5)
        bit = O.bitcos_pack(w).symbol_bits()
        five = O.t5_pack(w).size * 8
        two = O.b2_pack(w).size * 8
        assert np.sign(bit - five) == sign
        assert bit < two or zeros == 0


# --- Eq. (5) bytes per 32 weights ----------------------------------------------------------------

def test_eq5_bytes_per_iteration():
    g = read_golden("eq5_bytes.txt")
    z = float(g["z"])
    n, k = 10, 1280
    w = synth.exact_density_ternary(n, k, int(round(z * n * k)), seed=9)
    b = O.bitcos_pack(w)
    per32 = (b.bitmap.size + b.nnz / 8 + 2 * n * k / 128) * 32 / (n * k)
    assert per32 == pytest.approx(float(g["bytes_per_32"]), abs=1e-12)


# --- sign span of one 64-bit bitmap word ----------------------------------------------------------

def test_sign_span_of_a_word_fits_two_u64_words():
    w = synth.ternary(64, 1024, 0.05, seed=2)
    b = O.bitcos_pack(w)
    bm = np.frombuffer(b.bitmap.tobytes(), dtype="<u8").reshape(64, 16)
    for r in range(64):
        pos = int(b.rowoff[r])
        for j in range(16):
            c = bin(int(bm[r, j])).count("1")
            if c:
                assert (pos + c - 1) // 64 - pos // 64 <= 1
            pos += c
        assert pos == int(b.rowoff[r + 1])


# --- the textbook reduction ------------------------------------------------------------------------

def test_unit_scales_reduce_to_integer_matvec():
    n, k, m = 37, 640, 3
    w = synth.ternary(n, k, 0.42, seed=4)
    x = synth.activations(m, k, seed=4)
    ones = np.ones((n, k // 128), np.float16)
    y = O.gemv(w, ones, x)
    ref = (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), ref)
    acc = O.gemv_acc(w, x)
    ref_g = np.einsum("nk,mk->mnk", w.astype(np.int64), x.astype(np.int64)).reshape(m, n, k // 128, 128).sum(-1)
    assert np.array_equal(acc, ref_g)


def test_scaled_output_matches_float64_definition():
    n, k = 19, 512
    w = synth.ternary(n, k, 0.4, seed=8)
    x = synth.activations(2, k, seed=8)
    s = synth.scales(n, k // 128, seed=8)
    y = O.gemv(w, s, x)
    wd = w.astype(np.float64) * np.repeat(s.astype(np.float64), 128, axis=1)
    ref = (x.astype(np.float64) @ wd.T).astype(np.float32)
    assert np.array_equal(y, ref)  # all partial sums are exact in float64 for these scales


def test_half_decoding_matches_numpy():
    for h in [0, 1, 0x3C00, 0x3555, 0x7BFF, 0x8001, 0xC000, 0x0400, 0x03FF, 0x7C00, 0xFC00]:
        want = float(np.array([h], np.uint16).view(np.float16)[0])
        assert O.half_to_double(h) == want
    assert math.isnan(O.half_to_double(0x7E00))


# --- special cases -------------------------------------------------------------------------------------

def test_special_cases():
    n, k = 5, 256
    x = synth.activations(1, k, seed=6)
    s = synth.scales(n, 2, seed=6)
    # z = 0: 2 bits per weight; z = 1: 1 bit per weight, empty sign stream, y = 0
    w1 = synth.ternary(n, k, 0.0, seed=1)
    assert O.bitcos_pack(w1).symbol_bits() == 2 * n * k
    w0 = np.zeros((n, k), np.int8)
    b0 = O.bitcos_pack(w0)
    assert b0.symbol_bits() == n * k and b0.nnz == 0
    assert np.all(O.gemv(w0, s, x) == 0)
    # one non-zero per row: y = +-s * x[k]
    w = np.zeros((n, k), np.int8)
    cols = [3, 64, 127, 128, 255]
    for r, c in enumerate(cols):
        w[r, c] = 1 if r % 2 == 0 else -1
    y = O.gemv(w, s, x)[0]
    for r, c in enumerate(cols):
        want = np.float32(float(w[r, c]) * float(s[r, c // 128]) * float(x[0, c]))
        assert y[r] == want
    # x = e_k picks column k of the dequantised weights
    e = np.zeros((1, k), np.int8)
    e[0, 130] = 1
    y = O.gemv(w1, s, e)[0]
    assert np.array_equal(y, (w1[:, 130].astype(np.float64) * s[:, 1].astype(np.float64)).astype(np.float32))


# --- brute force over all local patterns -----------------------------------------------------------------

@pytest.mark.parametrize("k,start", [(128, 60), (256, 124)])
def test_brute_force_all_3pow8_patterns(k, start):
    pats = np.array(list(itertools.product([-1, 0, 1], repeat=8)), np.int8)  # 6561 rows
    w = np.zeros((len(pats), k), np.int8)
    w[:, start:start + 8] = pats
    xs = [synth.activations(1, k, seed=s) for s in range(3)]
    xs.append(np.full((1, k), -128, np.int8))
    xs.append(np.full((1, k), 127, np.int8))
    b = O.bitcos_pack(w)
    s = np.ones((len(pats), k // 128), np.float16)
    t5 = O.t5_pack(w)
    b2 = O.b2_pack(w)
    for x in xs:
        ref = (w.astype(np.int64) @ x[0].astype(np.int64))
        for fmt, a, sb, ro in [(O.FMT_BITCOS, b.bitmap, b.signs, b.rowoff), (O.FMT_5TRIT, t5, None, None),
                               (O.FMT_2BIT, b2, None, None)]:
            y = O.gemv_packed(fmt, a, sb, ro, s, len(pats), k, x)[0]
            assert np.array_equal(y.astype(np.int64), ref), fmt


# --- invariants ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("z", [0.0, 0.3, 0.47, 0.95])
def test_round_trips_and_cross_format_agreement(z):
    n, k = 33, 384
    w = synth.ternary(n, k, z, seed=12)
    b = O.bitcos_pack(w)
    w_b, used = O.bitcos_unpack(b.bitmap, b.signs, n, k)
    assert used == b.nnz and np.array_equal(w_b, w)
    assert np.array_equal(O.t5_unpack(O.t5_pack(w), n, k), w)
    assert np.array_equal(O.b2_unpack(O.b2_pack(w), n, k), w)
    x = synth.activations(2, k, seed=12)
    s = synth.scales(n, k // 128, seed=12)
    ref = O.gemv(w, s, x)
    for fmt, a, sb, ro in [(O.FMT_BITCOS, b.bitmap, b.signs, b.rowoff), (O.FMT_5TRIT, O.t5_pack(w), None, None),
                           (O.FMT_2BIT, O.b2_pack(w), None, None)]:
        assert np.array_equal(O.gemv_packed(fmt, a, sb, ro, s, n, k, x), ref)


def test_linearity_and_negation():
    n, k = 21, 256
    w = synth.ternary(n, k, 0.4, seed=13)
    x = synth.activations(1, k, seed=13).astype(np.int16)
    x = np.clip(x, -63, 63).astype(np.int8)
    acc1 = O.gemv_acc(w, x)
    acc2 = O.gemv_acc(w, (2 * x.astype(np.int16)).astype(np.int8))
    assert np.array_equal(acc2, 2 * acc1)
    s = synth.scales(n, 2, seed=13)
    assert np.array_equal(O.gemv(w, s, -x), -O.gemv(w, s, x))


def test_rejects_non_ternary():
    w = np.zeros((2, 128), np.int8)
    w[1, 7] = 2
    with pytest.raises(ValueError):
        O.bitcos_pack(w)
    with pytest.raises(ValueError):
        O.t5_pack(w)
    with pytest.raises(ValueError):
        O.b2_pack(w)
