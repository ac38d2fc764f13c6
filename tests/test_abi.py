"""C ABI: exported symbols, error codes and corrupt-buffer detection (CPU only, no compute calls)."""
import ctypes
import re

import numpy as np
import pytest

import bit_gemv_decode_amd as B
from bit_gemv_decode_amd import binding, synth
from tests.conftest import ROOT


def _declared_functions():
    src = open(f"{ROOT}/include/ternary_gemv.h").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(binding.EXPORTS), declared
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert binding.lib().tg_version() == 1


def test_strerror_names_every_code():
    for code in range(0, -8, -1):
        assert binding.strerror(code) != "unknown error"
    assert binding.strerror(-99) == "unknown error"


def _raw(fn, w, n, k, out=None, cap=0):
    need = ctypes.c_size_t(0)
    ptr = None if w is None else w.ctypes.data_as(ctypes.c_void_p)
    outp = None if out is None else out.ctypes.data_as(ctypes.c_void_p)
    return fn(ptr, n, k, outp, cap, ctypes.byref(need)), need.value


@pytest.mark.parametrize("name", ["tg_pack_bitcos", "tg_pack_5trit", "tg_pack_2bit"])
def test_packer_errors(name):
    fn = getattr(binding.lib(), name)
    w = np.zeros((4, 256), np.int8)
    assert _raw(fn, None, 4, 256)[0] == -1
    assert _raw(fn, w, 4, 200)[0] == -3  # k % 128
    assert _raw(fn, w, 0, 256)[0] == -3
    assert _raw(fn, w, 4, 0)[0] == -3
    bad = w.copy()
    bad[2, 100] = 2
    assert _raw(fn, bad, 4, 256)[0] == -2
    bad[2, 100] = -128
    assert _raw(fn, bad, 4, 256)[0] == -2
    code, need = _raw(fn, w, 4, 256)
    assert code == 0 and need > 0
    small = np.zeros(need - 1, np.uint8)
    assert _raw(fn, w, 4, 256, small, small.size)[0] == -6
    assert not small.any()  # nothing written on error
    with pytest.raises(B.TgError):
        B.pack(1 if "bitcos" in name else 2 if "5trit" in name else 3, bad)


def test_describe_rejects_foreign_and_truncated_buffers():
    w = synth.ternary(8, 256, 0.4, seed=1)
    p = B.pack_bitcos(w)
    with pytest.raises(B.TgError) as e:
        B.describe(p.buf[:100])
    assert e.value.code == -4
    bad = p.buf.copy()
    bad[0] ^= 1  # magic
    with pytest.raises(B.TgError) as e:
        B.describe(bad)
    assert e.value.code == -4
    with pytest.raises(B.TgError) as e:
        B.describe(p.buf[: p.desc.bytes_total - 256])  # sections past the end
    assert e.value.code == -5


def _poke_desc(buf, field, value):
    out = buf.copy()
    d = binding.TgDesc.from_buffer(out)
    setattr(d, field, value)
    return out


def test_describe_rejects_inconsistent_descriptors():
    w = synth.ternary(8, 256, 0.4, seed=1)
    p = B.pack_bitcos(w)
    for field, value, code in [("fmt", 9, -4), ("group", 64, -4), ("version", 2, -4), ("k", 200, -5),
                               ("n", 0, -5), ("nnz", 8 * 256 + 1, -5), ("bytes_codes", 1, -5),
                               ("off_signs", 300, -5), ("bytes_index", 4, -5), ("bytes_payload", 1, -5)]:
        with pytest.raises(B.TgError) as e:
            B.describe(_poke_desc(p.buf, field, value))
        assert e.value.code == code, field
    t = B.pack_5trit(w)
    with pytest.raises(B.TgError) as e:
        B.describe(_poke_desc(t.buf, "bytes_total", t.desc.off_codes + t.desc.bytes_codes))
    assert e.value.code == -5


def test_validate_detects_corrupt_contents():
    w = synth.ternary(8, 256, 0.4, seed=1)
    p = B.pack_bitcos(w)
    bad = p.buf.copy()
    bad[p.desc.off_index + 4 * 3] += 1  # rowoff[3] no longer matches the bitmap
    with pytest.raises(B.TgError) as e:
        B.validate(bad)
    assert e.value.code == -5
    bad = p.buf.copy()
    bad[p.desc.off_codes] ^= 1  # bitmap popcount of row 0 changes
    with pytest.raises(B.TgError) as e:
        B.unpack(bad)
    assert e.value.code == -5
    t = B.pack_5trit(w)
    bad = t.buf.copy()
    bad[t.desc.off_codes + 7] = 243
    with pytest.raises(B.TgError):
        B.validate(bad)
    bad = t.buf.copy()
    bad[t.desc.off_codes + 25] = 0  # padding digits must be weight 0
    with pytest.raises(B.TgError):
        B.validate(bad)
    b = B.pack_2bit(w)
    bad = b.buf.copy()
    bad[b.desc.off_codes + 3] |= 0xC0  # code 3
    with pytest.raises(B.TgError):
        B.validate(bad)
    bad = b.buf.copy()
    bad[b.desc.off_codes + 3] ^= 0x01  # still valid codes, but the non-zero count changes
    with pytest.raises(B.TgError):
        B.validate(bad)


def test_gemv_argument_errors_before_any_gpu_work():
    L = binding.lib()
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    dummy = ctypes.c_void_p(256)
    # null descriptor / pointers, m out of range, misalignment: rejected on the host
    assert L.ternary_gemv(None, dummy, dummy, dummy, dummy, 1, None) == -1
    assert L.ternary_gemv(ctypes.byref(d), None, dummy, dummy, dummy, 1, None) == -1
    assert L.ternary_gemv(ctypes.byref(d), dummy, dummy, dummy, dummy, 0, None) == -1
    assert L.ternary_gemv(ctypes.byref(d), dummy, dummy, dummy, dummy, 17, None) == -1
    assert L.ternary_gemv(ctypes.byref(d), ctypes.c_void_p(264), dummy, dummy, dummy, 1, None) == -1
    assert L.ternary_gemv(ctypes.byref(d), dummy, None, dummy, dummy, 1, None) == -1
    assert L.ternary_gemv_acc(ctypes.byref(d), dummy, dummy, None, 1, None) == -1
    d2 = binding.TgDesc.from_buffer_copy(d)
    d2.magic = 0
    assert L.ternary_gemv(ctypes.byref(d2), dummy, dummy, dummy, dummy, 1, None) == -4
    d2 = binding.TgDesc.from_buffer_copy(d)
    d2.bytes_signs = 4
    assert L.ternary_gemv_acc(ctypes.byref(d2), dummy, dummy, dummy, 1, None) == -5


def test_plan_argument_errors_before_any_gpu_work():
    L = binding.lib()
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    descs = (binding.TgDesc * 1)(d)
    dummy = ctypes.c_void_p(256)
    P1 = ctypes.c_void_p * 1
    ptrs = P1(256)
    plan = binding.TgPlan()
    nbytes = L.tg_plan_table_bytes(1)
    assert nbytes > 0 and L.tg_plan_table_bytes(0) == 0
    # null plan / table / descriptors, bad count or m, misaligned or short table: TG_EINVAL
    assert L.tg_plan_init(None, dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    assert L.tg_plan_init(ctypes.byref(plan), None, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 0, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 17) == -1
    # m above 3 is for BITCOS (thin-batch path) only
    d5one = (binding.TgDesc * 1)(B.pack_5trit(w).desc)
    d2one = (binding.TgDesc * 1)(B.pack_2bit(w).desc)
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, d5one, ptrs, ptrs, ptrs, ptrs, None, 4) == -1
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, d2one, ptrs, ptrs, ptrs, ptrs, None, 4) == -1
    assert L.tg_plan_init(ctypes.byref(plan), ctypes.c_void_p(264), nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs,
                          None, 1) == -1
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes - 1, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    # value mode without y
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, None, None, 1) == -1
    # a corrupt descriptor is reported as such
    bad = (binding.TgDesc * 1)(binding.TgDesc.from_buffer_copy(d))
    bad[0].magic = 0
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, bad, ptrs, ptrs, ptrs, ptrs, None, 1) == -4
    # mixed formats
    d5 = B.pack_5trit(w).desc
    two = (binding.TgDesc * 2)(d, d5)
    P2 = ctypes.c_void_p * 2
    p2 = P2(256, 256)
    assert L.tg_plan_init(ctypes.byref(plan), dummy, L.tg_plan_table_bytes(2), 2, two, p2, p2, p2, p2, None,
                          1) == -1
    # running a plan that was never initialised
    assert L.ternary_gemv_plan(ctypes.byref(binding.TgPlan()), None) == -1
    assert L.ternary_gemv_plan(None, None) == -1


def test_activation_quantisation_argument_errors_before_any_gpu_work():
    L = binding.lib()
    dummy = ctypes.c_void_p(256)
    # tg_quantize_x: null or misaligned pointers, m out of range -> TG_EINVAL; bad k -> TG_ESHAPE
    assert L.tg_quantize_x(None, 1, 128, dummy, dummy, None) == -1
    assert L.tg_quantize_x(dummy, 1, 128, None, dummy, None) == -1
    assert L.tg_quantize_x(dummy, 1, 128, dummy, None, None) == -1
    assert L.tg_quantize_x(dummy, 0, 128, dummy, dummy, None) == -1
    assert L.tg_quantize_x(dummy, 17, 128, dummy, dummy, None) == -1
    assert L.tg_quantize_x(ctypes.c_void_p(260), 1, 128, dummy, dummy, None) == -1
    assert L.tg_quantize_x(dummy, 1, 128, ctypes.c_void_p(257), dummy, None) == -1
    assert L.tg_quantize_x(dummy, 1, 128, dummy, ctypes.c_void_p(258), None) == -1
    assert L.tg_quantize_x(dummy, 1, 0, dummy, dummy, None) == -3
    assert L.tg_quantize_x(dummy, 1, 192, dummy, dummy, None) == -3
    assert L.tg_quantize_x(dummy, 1, (1 << 30) + 128, dummy, dummy, None) == -3
    # ternary_gemv_xs: the ternary_gemv checks plus a null or misaligned activation-scale pointer
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    assert L.ternary_gemv_xs(ctypes.byref(d), dummy, dummy, dummy, None, dummy, 1, None) == -1
    assert L.ternary_gemv_xs(ctypes.byref(d), dummy, dummy, dummy, ctypes.c_void_p(258), dummy, 1, None) == -1
    assert L.ternary_gemv_xs(ctypes.byref(d), dummy, dummy, dummy, dummy, dummy, 0, None) == -1
    assert L.ternary_gemv_xs(ctypes.byref(d), dummy, None, dummy, dummy, dummy, 1, None) == -1
    d2 = binding.TgDesc.from_buffer_copy(d)
    d2.magic = 0
    assert L.ternary_gemv_xs(ctypes.byref(d2), dummy, dummy, dummy, dummy, dummy, 1, None) == -4
    # tg_plan_init_xs: a null activation-scale array or entry, or a misaligned entry
    descs = (binding.TgDesc * 1)(d)
    P1 = ctypes.c_void_p * 1
    ptrs = P1(256)
    plan = binding.TgPlan()
    nbytes = L.tg_plan_table_bytes(1)
    assert L.tg_plan_init_xs(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, None, ptrs, 1) == -1
    assert L.tg_plan_init_xs(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, P1(None), ptrs, 1) == -1
    assert L.tg_plan_init_xs(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, P1(258), ptrs, 1) == -1
    assert L.tg_plan_init_xs(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    bad = (binding.TgDesc * 1)(d2)
    assert L.tg_plan_init_xs(ctypes.byref(plan), dummy, nbytes, 1, bad, ptrs, ptrs, ptrs, ptrs, ptrs, 1) == -4


def test_t5b_argument_errors_before_any_gpu_work():
    L = binding.lib()
    w = synth.ternary(8, 256, 0.4, seed=1)
    sz = ctypes.c_size_t(0)
    wp = w.ctypes.data_as(ctypes.c_void_p)
    assert L.tg_pack_t5b(wp, 8, 256, ctypes.c_float(float("nan")), None, 0, ctypes.byref(sz)) == -1
    assert L.tg_pack_t5b(wp, 8, 256, ctypes.c_float(float("inf")), None, 0, ctypes.byref(sz)) == -1
    assert L.tg_pack_t5b(wp, 8, 200, ctypes.c_float(1.0), None, 0, ctypes.byref(sz)) == -3
    bad = w.copy()
    bad[0, 0] = 2
    assert L.tg_pack_t5b(bad.ctypes.data_as(ctypes.c_void_p), 8, 256, ctypes.c_float(1.0), None, 0,
                         ctypes.byref(sz)) == -2
    d = B.pack_t5b(w, 0.5).desc
    dummy = ctypes.c_void_p(256)
    # t5b takes no per-group scales and no activation group scales
    assert L.ternary_gemv(ctypes.byref(d), dummy, dummy, dummy, dummy, 1, None) == -1
    assert L.ternary_gemv_xs(ctypes.byref(d), dummy, None, dummy, dummy, dummy, 1, None) == -1
    descs = (binding.TgDesc * 1)(d)
    P1 = ctypes.c_void_p * 1
    plan = binding.TgPlan()
    nbytes = L.tg_plan_table_bytes(1)
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, descs, P1(256), P1(256), P1(256), P1(256), None,
                          1) == -1
    # a t5b descriptor with the other formats' group size is not a valid descriptor
    d2 = binding.TgDesc.from_buffer_copy(d)
    d2.group = 128
    assert L.ternary_gemv(ctypes.byref(d2), dummy, None, dummy, dummy, 1, None) == -4


def test_f16_gemv_argument_errors_before_any_gpu_work():
    L = binding.lib()
    dummy = ctypes.c_void_p(256)
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    # null or misaligned pointers, m out of range -> TG_EINVAL
    assert L.ternary_gemv_f16(None, dummy, dummy, dummy, dummy, 1, None) == -1
    for i in range(4):
        args = [dummy] * 4
        args[i] = None
        assert L.ternary_gemv_f16(ctypes.byref(d), *args, 1, None) == -1
    assert L.ternary_gemv_f16(ctypes.byref(d), dummy, dummy, dummy, dummy, 0, None) == -1
    assert L.ternary_gemv_f16(ctypes.byref(d), dummy, dummy, dummy, dummy, B.TG_MAX_M + 1, None) == -1
    assert L.ternary_gemv_f16(ctypes.byref(d), dummy, dummy, ctypes.c_void_p(264), dummy, 1, None) == -1
    assert L.ternary_gemv_f16(ctypes.byref(d), dummy, ctypes.c_void_p(257), dummy, dummy, 1, None) == -1
    assert L.ternary_gemv_f16(ctypes.byref(d), dummy, dummy, dummy, ctypes.c_void_p(258), 1, None) == -1
    # BITCOS only
    for fmt in (B.FMT_5TRIT, B.FMT_2BIT):
        d5 = B.pack(fmt, w).desc
        assert L.ternary_gemv_f16(ctypes.byref(d5), dummy, dummy, dummy, dummy, 1, None) == -1
    d2 = binding.TgDesc.from_buffer_copy(d)
    d2.magic = 0
    assert L.ternary_gemv_f16(ctypes.byref(d2), dummy, dummy, dummy, dummy, 1, None) == -4


def test_f16_plan_argument_errors_before_any_gpu_work():
    L = binding.lib()
    dummy = ctypes.c_void_p(256)
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    descs = (binding.TgDesc * 1)(d)
    P1 = ctypes.c_void_p * 1
    ptrs = P1(256)
    plan = binding.TgPlan()
    nbytes = L.tg_plan_table_bytes(1)
    # m outside [1, 16], null arrays or entries, misaligned activations
    for m in (0, 17):
        assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, m) == -1
    assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, None, ptrs, 1) == -1
    assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, P1(None), ptrs, 1) == -1
    assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, P1(264), ptrs, 1) == -1
    assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, None, ptrs, ptrs, 1) == -1
    # BITCOS only
    for fmt in (B.FMT_5TRIT, B.FMT_2BIT):
        other = (binding.TgDesc * 1)(B.pack(fmt, w).desc)
        assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, other, ptrs, ptrs, ptrs, ptrs, 1) == -1
    # a plan claiming the fp16 path with another format, m or output mode is refused before launching
    forged = binding.TgPlan(magic=0x4E4C5054, fmt=B.FMT_5TRIT, m=1, count=1, units=1, rows_per_unit=1,
                            acc_mode=0, waves=8, path=2, table=256)
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
    forged.fmt, forged.acc_mode = B.FMT_BITCOS, 1
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
    forged.acc_mode, forged.m = 0, 3
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
    forged.m, forged.path = 1, 3  # the fp16 matrix-core path takes m >= 2
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
    forged.m, forged.acc_mode = 4, 2
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
    forged.acc_mode, forged.path = 0, 4
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1


def test_plan_struct_layout_and_decode_selection_errors():
    L = binding.lib()
    # the C layout: twelve 32-bit fields, then the table pointer
    assert ctypes.sizeof(binding.TgPlan) == 56 and binding.TgPlan.table.offset == 48
    assert binding.TgPlan.decode.offset == 36 and binding.TgPlan.live_rows.offset == 40
    assert binding.TgPlan.table_gen.offset == 44
    assert L.tg_plan_set_decode(None, 1) == -1
    assert L.tg_plan_set_decode(ctypes.byref(binding.TgPlan()), 1) == -1  # never initialised
    ok = dict(magic=0x4E4C5054, fmt=B.FMT_BITCOS, m=1, count=1, units=1, rows_per_unit=1, acc_mode=0, waves=8,
              path=0, table=256)
    for bad in (dict(fmt=B.FMT_5TRIT), dict(m=2), dict(path=1), dict(path=2), dict(acc_mode=2)):
        p = binding.TgPlan(**{**ok, **bad})
        assert L.tg_plan_set_decode(ctypes.byref(p), 1) == -1 and p.decode == 0
        assert L.tg_plan_set_decode(ctypes.byref(p), 0) == 0
        p.decode = 1  # a forged plan claiming the nibble decode is refused before launching
        assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
    p = binding.TgPlan(**ok)
    assert L.tg_plan_set_decode(ctypes.byref(p), 2) == -1 and p.decode == 0
    for acc_mode in (0, 1):
        p.acc_mode = acc_mode
        assert L.tg_plan_set_decode(ctypes.byref(p), 1) == 0 and p.decode == 1
        assert L.tg_plan_set_decode(ctypes.byref(p), 0) == 0 and p.decode == 0
    p.decode = 5
    assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
    # the table-free decode: five-trit, t5b and 2-bit plans at m = 1 on the vector path, y or accumulators
    for fmt in (B.FMT_5TRIT, B.FMT_T5B, B.FMT_2BIT):
        for acc_mode in (0, 1):
            p = binding.TgPlan(**{**ok, "fmt": fmt, "acc_mode": acc_mode})
            assert L.tg_plan_set_decode(ctypes.byref(p), 2) == 0 and p.decode == 2
            assert L.tg_plan_set_decode(ctypes.byref(p), 1) == -1 and p.decode == 2  # nibble: BITCOS only
            assert L.tg_plan_set_decode(ctypes.byref(p), 0) == 0 and p.decode == 0
        for bad in (dict(m=2), dict(path=1), dict(acc_mode=2)):
            p = binding.TgPlan(**{**ok, "fmt": fmt, **bad})
            assert L.tg_plan_set_decode(ctypes.byref(p), 2) == -1 and p.decode == 0
            p.decode = 2  # forged: refused before launching
            assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
    for fmt in (B.FMT_BITCOS,):
        p = binding.TgPlan(**{**ok, "fmt": fmt})
        assert L.tg_plan_set_decode(ctypes.byref(p), 2) == -1 and p.decode == 0
        p.decode = 2
        assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
    # a forged plan claiming the live-row walk where no kernel has it is refused before launching
    for bad in (dict(live_rows=2), dict(live_rows=1, fmt=B.FMT_5TRIT), dict(live_rows=1, m=2),
                dict(live_rows=1, acc_mode=1), dict(live_rows=1, path=1), dict(live_rows=1, m=2, path=4)):
        p = binding.TgPlan(**{**ok, **bad})
        assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
    # path 4 (the 12-wave build with two-step units) exists for BITCOS at m = 2 only; no path 5
    for bad in (dict(path=4), dict(path=4, m=3), dict(path=4, m=2, fmt=B.FMT_5TRIT), dict(path=4, m=2, fmt=B.FMT_2BIT),
                dict(path=5, m=2)):
        p = binding.TgPlan(**{**ok, **bad})
        assert L.ternary_gemv_plan(ctypes.byref(p), None) == -1
        assert L.tg_plan_set_decode(ctypes.byref(p), 1) == -1


def test_empty_rows_field_checked():
    # tg_desc.empty_rows: BITCOS rows without non-zeros (a hint for the kernel); at most n, zero for the
    # other formats, and tg_validate compares it with the index.
    w = synth.ternary(9, 256, 0.4, seed=4)
    w[[1, 5, 6]] = 0
    p = B.pack_bitcos(w)
    assert p.desc.empty_rows == 3
    B.validate(p.buf)
    for value, code in ((10, -5), (2, -5), (4, -5)):
        bad = _poke_desc(p.buf, "empty_rows", value)
        with pytest.raises(B.TgError) as e:
            B.validate(bad)
        assert e.value.code == code
    for fmt in (B.FMT_5TRIT, B.FMT_2BIT):
        q = B.pack(fmt, w)
        assert q.desc.empty_rows == 0
        with pytest.raises(B.TgError) as e:
            B.describe(_poke_desc(q.buf, "empty_rows", 1))
        assert e.value.code == -5


def _bitcos_desc(n, k, nnz):
    """A consistent BITCOS descriptor of an n x k matrix with nnz non-zeros (the packer's layout),
    for shapes too large to pack here."""
    d = binding.TgDesc.from_buffer_copy(B.pack_bitcos(np.zeros((1, 128), np.int8)).desc)
    up = lambda v, a=256: (v + a - 1) // a * a
    sign_bytes = (nnz + 7) // 8
    d.n, d.k, d.nnz = n, k, nnz
    d.bytes_codes = n * k // 8
    d.off_signs = up(d.off_codes + d.bytes_codes)
    d.bytes_signs = up(sign_bytes + 16, 8)
    d.off_index = up(d.off_signs + d.bytes_signs)
    d.bytes_index = 4 * (n + 1)
    d.bytes_total = up(d.off_index + d.bytes_index)
    d.bytes_payload = d.bytes_codes + sign_bytes + d.bytes_index
    return d


def test_offset_limits_refused_before_any_gpu_work():
    # The kernels address each section with 32-bit offsets (switched-off accesses use offsets from
    # 2^31): bitmaps, scales and outputs must stay below 1 GiB, sign windows below 512 MiB, and fp16
    # activation rows (2 m k bytes) at most 1 GiB. Descriptors past a limit are TG_ESHAPE.
    L = binding.lib()
    dummy = ctypes.c_void_p(256)
    at_bitmap_limit = _bitcos_desc(65536, 131072, 1 << 20)   # bitmap exactly 1 GiB
    at_sign_limit = _bitcos_desc(65535, 131072, (1 << 32) - 1)  # 512 MiB of signs
    big_out = _bitcos_desc(65535, 131072, 1 << 20)          # n * k/128 * 4 * m > 1 GiB from m = 5
    long_rows = _bitcos_desc(1, 1 << 28, 1 << 20)            # 2 m k > 2^30 at m = 3
    for d in (at_bitmap_limit, at_sign_limit):
        assert L.ternary_gemv(ctypes.byref(d), dummy, dummy, dummy, dummy, 1, None) == -3
        assert L.ternary_gemv_acc(ctypes.byref(d), dummy, dummy, dummy, 1, None) == -3
        assert L.ternary_gemv_f16(ctypes.byref(d), dummy, dummy, dummy, dummy, 1, None) == -3
    assert L.ternary_gemv_acc(ctypes.byref(big_out), dummy, dummy, dummy, 5, None) == -3
    assert L.ternary_gemv(ctypes.byref(big_out), dummy, dummy, dummy, dummy, 5, None) == -3
    assert L.ternary_gemv_f16(ctypes.byref(long_rows), dummy, dummy, dummy, dummy, 3, None) == -3
    descs = (binding.TgDesc * 1)(at_bitmap_limit)
    P1 = ctypes.c_void_p * 1
    ptrs = P1(256)
    plan = binding.TgPlan()
    nbytes = L.tg_plan_table_bytes(1)
    assert L.tg_plan_init(ctypes.byref(plan), dummy, nbytes, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -3
    assert L.tg_plan_init_f16(ctypes.byref(plan), dummy, nbytes, 1, (binding.TgDesc * 1)(long_rows), ptrs, ptrs,
                              ptrs, ptrs, 3) == -3


@pytest.mark.parametrize("fmt", [B.FMT_5TRIT, B.FMT_2BIT, B.FMT_T5B], ids=["5trit", "2bit", "t5b"])
def test_multi_launch_calls_check_everything_before_enqueuing(fmt):
    # Five-trit, 2-bit and t5b with m > 3 run several launches of at most three activation rows. All of
    # them are set up and checked before the first is enqueued, so every bad argument comes back as its
    # own code (on a machine without a GPU, reaching the HIP runtime would give TG_EHIP instead).
    L = binding.lib()
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = (B.pack_t5b(w, 0.5) if fmt == B.FMT_T5B else B.pack(fmt, w)).desc
    dummy = ctypes.c_void_p(256)
    sc = None if fmt == B.FMT_T5B else dummy
    for m in (4, 7, 16):
        assert L.ternary_gemv(ctypes.byref(d), dummy, sc, dummy, ctypes.c_void_p(258), m, None) == -1  # y
        assert L.ternary_gemv(ctypes.byref(d), dummy, sc, ctypes.c_void_p(264), dummy, m, None) == -1  # x
        assert L.ternary_gemv(ctypes.byref(d), ctypes.c_void_p(264), sc, dummy, dummy, m, None) == -1  # W
        assert L.ternary_gemv_acc(ctypes.byref(d), dummy, dummy, ctypes.c_void_p(258), m, None) == -1
        if fmt != B.FMT_T5B:
            assert L.ternary_gemv(ctypes.byref(d), dummy, ctypes.c_void_p(257), dummy, dummy, m, None) == -1
        d2 = binding.TgDesc.from_buffer_copy(d)
        d2.magic = 0
        assert L.ternary_gemv(ctypes.byref(d2), dummy, sc, dummy, dummy, m, None) == -4
        d2 = binding.TgDesc.from_buffer_copy(d)
        d2.bytes_codes = 4
        assert L.ternary_gemv_acc(ctypes.byref(d2), dummy, dummy, dummy, m, None) == -5
    assert L.ternary_gemv(ctypes.byref(d), dummy, sc, dummy, dummy, 17, None) == -1


def test_noalloc_plan_argument_errors_before_any_gpu_work():
    # tg_plan_init_noalloc: the same checks as tg_plan_init; a count whose table exceeds the static
    # array is TG_ENOSPACE before anything else happens
    L = binding.lib()
    w = synth.ternary(8, 256, 0.4, seed=1)
    d = B.pack_bitcos(w).desc
    descs = (binding.TgDesc * 1)(d)
    P1 = ctypes.c_void_p * 1
    ptrs = P1(256)
    plan = binding.TgPlan()
    assert L.tg_plan_init_noalloc(None, 1, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    assert L.tg_plan_init_noalloc(ctypes.byref(plan), 0, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -1
    big = 1
    while L.tg_plan_table_bytes(big) <= binding.NOALLOC_TABLE_BYTES:
        big *= 2
    assert L.tg_plan_init_noalloc(ctypes.byref(plan), big, descs, ptrs, ptrs, ptrs, ptrs, None, 1) == -6
    # a plan claiming a static-table generation that is not the current one is refused
    forged = binding.TgPlan(magic=0x4E4C5054, fmt=B.FMT_BITCOS, m=1, count=1, units=1, rows_per_unit=1, acc_mode=0,
                            waves=8, path=0, table_gen=7, table=256)
    assert L.ternary_gemv_plan(ctypes.byref(forged), None) == -1
