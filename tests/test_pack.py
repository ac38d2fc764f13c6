"""Library packers vs the oracle's (CPU only): byte equality, round trips, accounting."""
import numpy as np
import pytest

import bit_gemv_decode_amd as B
import oracle as O
from bit_gemv_decode_amd import synth


def _check_bitcos(w):
    p = B.pack_bitcos(w)
    o = O.bitcos_pack(w)
    assert p.nnz == o.nnz
    # rows without non-zeros, as the oracle's index shows them (equal consecutive entries)
    assert p.desc.empty_rows == int((np.diff(o.rowoff.astype(np.int64)) == 0).sum()) == int((~w.any(axis=1)).sum())
    assert np.array_equal(p.section("codes"), o.bitmap)
    assert np.array_equal(p.sign_bytes(), o.signs)
    assert np.array_equal(p.rowoff(), o.rowoff)
    # padding after the sign stream is zero
    assert not p.section("signs")[(p.nnz + 7) // 8:].any()
    assert p.payload_bytes == o.bitmap.size + (o.nnz + 7) // 8 + 4 * (w.shape[0] + 1)
    return p


@pytest.mark.parametrize("n,k,z", [(1, 128, 0.42), (3, 256, 0.0), (5, 384, 1.0), (17, 640, 0.3), (64, 1024, 0.515),
                                   (33, 2560, 0.42), (7, 4096, 0.95)])
def test_packers_match_oracle_bytes(n, k, z):
    w = synth.ternary(n, k, z, seed=n * 7 + k)
    _check_bitcos(w)
    assert np.array_equal(B.pack_5trit(w).section("codes"), O.t5_pack(w))
    assert np.array_equal(B.pack_2bit(w).section("codes"), O.b2_pack(w))
    for fmt in (B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT):
        pk = B.pack(fmt, w)
        B.validate(pk.buf)
        assert np.array_equal(B.unpack(pk.buf), w)
        assert pk.desc.nnz == int((w != 0).sum())


def test_parallel_pack_row_boundaries():
    # Large enough for the multi-threaded packer; rows with odd non-zero counts put sign-word
    # boundaries inside rows, and the all-zero / all-non-zero rows test empty and full ranges.
    n, k = 1100, 8192
    w = synth.ternary(n, k, 0.47, seed=21)
    w[5] = 0
    w[6] = 1
    w[700, :] = -1
    w[701, 3] = 1
    p = _check_bitcos(w)
    assert np.array_equal(B.unpack(p.buf), w)


def test_bits_per_weight_accounting():
    n, k = 40, 1280
    w = synth.exact_density_ternary(n, k, int(0.4 * n * k), seed=3)
    p = B.pack_bitcos(w)
    sym_bits = p.desc.bytes_codes * 8 + p.nnz
    assert sym_bits / (n * k) == pytest.approx(1.6, abs=1e-12)
    assert B.pack_5trit(w).desc.bytes_codes * 8 / (n * k) == 1.625
    assert B.pack_2bit(w).desc.bytes_codes * 8 / (n * k) == 2.0


def test_descriptor_layout():
    w = synth.ternary(9, 512, 0.4, seed=2)
    for fmt in (B.FMT_BITCOS, B.FMT_5TRIT, B.FMT_2BIT):
        d = B.pack(fmt, w).desc
        assert d.magic == 0x53444754 and d.version == 1 and d.group == 128
        assert d.off_codes == 256 and d.off_codes % 256 == 0
        assert d.bytes_total % 256 == 0
        if fmt == B.FMT_BITCOS:
            assert d.off_signs % 256 == 0 and d.off_index % 256 == 0
            assert d.off_signs >= d.off_codes + d.bytes_codes
            assert d.off_index >= d.off_signs + d.bytes_signs
            assert d.bytes_signs >= (d.nnz + 7) // 8 + 16
        else:
            assert d.bytes_total >= d.off_codes + d.bytes_codes + 16


@pytest.mark.parametrize("n,k,z", [(1, 128, 0.42), (3, 256, 0.0), (5, 384, 1.0), (17, 640, 0.3), (33, 2560, 0.42),
                                   (7, 4096, 0.95), (4, 14336, 0.4), (300, 5120, 0.47)])
def test_t5b_packer_matches_oracle_bytes(n, k, z):
    w = synth.ternary(n, k, z, seed=n * 11 + k)
    p = B.pack_t5b(w, 0.0375)
    assert np.array_equal(p.section("codes").reshape(n, -1, 32), O.t5b_pack(w))
    assert p.desc.group == 160 and p.payload_bytes == n * (-(-k // 160)) * 32
    assert np.frombuffer(np.uint32(p.desc.tensor_scale).tobytes(), np.float32)[0] == np.float32(0.0375)
    B.validate(p.buf)
    assert np.array_equal(B.unpack(p.buf), w)
    assert p.desc.nnz == int((w != 0).sum())


def test_t5b_validate_rejects_bad_bytes_and_padding():
    w = synth.ternary(3, 128, 0.4, seed=2)
    p = B.pack_t5b(w, 1.0)
    off = p.desc.off_codes
    bad = p.buf.copy()
    bad[off + 5] = 250  # not a five-trit byte
    with pytest.raises(B.TgError):
        B.validate(bad)
    bad = p.buf.copy()
    bad[off + 31] = 120  # k = 128: byte 31 is all padding and must encode five weight-0 digits
    with pytest.raises(B.TgError):
        B.validate(bad)
