"""Thin Python binding of the C ABI in include/ternary_gemv.h (argument marshalling only).

Every numeric step runs in libternary_gemv.so: the host packers in C++ and the GEMV in HIP kernels
on the GPU. PyTorch supplies device memory and streams; numpy supplies host arrays. There is no
fallback: if the library is missing or the GPU path is unavailable the call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# TG_LIB_PATH selects another build of the library (e.g. one with sanitized host code)
LIB_PATH = os.environ.get("TG_LIB_PATH") or os.path.join(PKG, "libternary_gemv.so")

TG_GROUP = 128
TG_MAX_M = 16
TG_HEADER_BYTES = 256
FMT_BITCOS, FMT_5TRIT, FMT_2BIT, FMT_T5B = 1, 2, 3, 4
FMT_NAMES = {FMT_BITCOS: "bitcos", FMT_5TRIT: "5trit", FMT_2BIT: "2bit", FMT_T5B: "t5b"}
T5B_BLOCK = 160
DECODE_BYTE, DECODE_NIBBLE, DECODE_ARITH = 0, 1, 2
ERRORS = {0: "TG_OK", -1: "TG_EINVAL", -2: "TG_ENOTTERNARY", -3: "TG_ESHAPE", -4: "TG_EFORMAT",
          -5: "TG_ECORRUPT", -6: "TG_ENOSPACE", -7: "TG_EHIP"}

# Every symbol include/ternary_gemv.h declares.
EXPORTS = ["tg_pack_bitcos", "tg_pack_5trit", "tg_pack_2bit", "tg_pack_t5b", "tg_describe", "tg_validate", "tg_unpack",
           "ternary_gemv", "ternary_gemv_acc", "tg_quantize_x", "ternary_gemv_xs", "ternary_gemv_f16",
           "tg_plan_table_bytes",
           "tg_plan_init", "tg_plan_init_xs", "tg_plan_init_f16", "ternary_gemv_plan", "tg_plan_init_noalloc",
           "tg_plan_set_decode", "tg_stream_read", "tg_clock_probe", "tg_strerror", "tg_version"]
NOALLOC_TABLE_BYTES = 256 * 1024


class TgError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({strerror(code)})")


class TgDesc(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("fmt", ctypes.c_int32),
                ("group", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("nnz", ctypes.c_uint64),
                ("off_codes", ctypes.c_uint64), ("bytes_codes", ctypes.c_uint64),
                ("off_signs", ctypes.c_uint64), ("bytes_signs", ctypes.c_uint64),
                ("off_index", ctypes.c_uint64), ("bytes_index", ctypes.c_uint64),
                ("bytes_total", ctypes.c_uint64), ("bytes_payload", ctypes.c_uint64),
                ("tensor_scale", ctypes.c_uint32), ("empty_rows", ctypes.c_uint32), ("reserved", ctypes.c_uint64)]


class TgPlan(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("fmt", ctypes.c_int32), ("m", ctypes.c_int32),
                ("count", ctypes.c_int32), ("units", ctypes.c_int32), ("rows_per_unit", ctypes.c_int32),
                ("acc_mode", ctypes.c_int32), ("waves", ctypes.c_int32), ("path", ctypes.c_int32),
                ("decode", ctypes.c_int32), ("live_rows", ctypes.c_int32), ("table_gen", ctypes.c_uint32),
                ("table", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libternary_gemv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_gemv_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        for name in ("tg_pack_bitcos", "tg_pack_5trit", "tg_pack_2bit"):
            f = getattr(L, name)
            f.argtypes = [p, i64, i64, p, sz, ctypes.POINTER(sz)]
            f.restype = ctypes.c_int
        L.tg_pack_t5b.argtypes = [p, i64, i64, ctypes.c_float, p, sz, ctypes.POINTER(sz)]
        L.tg_pack_t5b.restype = ctypes.c_int
        L.tg_describe.argtypes = [p, sz, ctypes.POINTER(TgDesc)]
        L.tg_describe.restype = ctypes.c_int
        L.tg_validate.argtypes = [p, sz]
        L.tg_validate.restype = ctypes.c_int
        L.tg_unpack.argtypes = [p, sz, p]
        L.tg_unpack.restype = ctypes.c_int
        L.ternary_gemv.argtypes = [ctypes.POINTER(TgDesc), p, p, p, p, ctypes.c_int32, p]
        L.ternary_gemv.restype = ctypes.c_int
        L.ternary_gemv_acc.argtypes = [ctypes.POINTER(TgDesc), p, p, p, ctypes.c_int32, p]
        L.ternary_gemv_acc.restype = ctypes.c_int
        L.tg_quantize_x.argtypes = [p, ctypes.c_int32, i64, p, p, p]
        L.tg_quantize_x.restype = ctypes.c_int
        L.ternary_gemv_xs.argtypes = [ctypes.POINTER(TgDesc), p, p, p, p, p, ctypes.c_int32, p]
        L.ternary_gemv_xs.restype = ctypes.c_int
        L.ternary_gemv_f16.argtypes = [ctypes.POINTER(TgDesc), p, p, p, p, ctypes.c_int32, p]
        L.ternary_gemv_f16.restype = ctypes.c_int
        L.tg_plan_init_xs.argtypes = [ctypes.POINTER(TgPlan), p, sz, ctypes.c_int32, ctypes.POINTER(TgDesc), p, p,
                                      p, p, p, ctypes.c_int32]
        L.tg_plan_init_xs.restype = ctypes.c_int
        L.tg_plan_init_f16.argtypes = [ctypes.POINTER(TgPlan), p, sz, ctypes.c_int32, ctypes.POINTER(TgDesc), p, p,
                                       p, p, ctypes.c_int32]
        L.tg_plan_init_f16.restype = ctypes.c_int
        L.tg_plan_set_decode.argtypes = [ctypes.POINTER(TgPlan), ctypes.c_int32]
        L.tg_plan_set_decode.restype = ctypes.c_int
        L.tg_plan_table_bytes.argtypes = [ctypes.c_int32]
        L.tg_plan_table_bytes.restype = sz
        L.tg_plan_init.argtypes = [ctypes.POINTER(TgPlan), p, sz, ctypes.c_int32, ctypes.POINTER(TgDesc), p, p, p, p,
                                   p, ctypes.c_int32]
        L.tg_plan_init.restype = ctypes.c_int
        L.tg_plan_init_noalloc.argtypes = [ctypes.POINTER(TgPlan), ctypes.c_int32, ctypes.POINTER(TgDesc), p, p, p,
                                           p, p, ctypes.c_int32]
        L.tg_plan_init_noalloc.restype = ctypes.c_int
        L.ternary_gemv_plan.argtypes = [ctypes.POINTER(TgPlan), p]
        L.ternary_gemv_plan.restype = ctypes.c_int
        L.tg_clock_probe.argtypes = [p, ctypes.c_uint32, ctypes.c_uint32, p]
        L.tg_clock_probe.restype = ctypes.c_int
        L.tg_stream_read.argtypes = [p, sz, p, ctypes.c_int32, ctypes.c_int32, p]
        L.tg_stream_read.restype = ctypes.c_int
        L.tg_strerror.argtypes = [ctypes.c_int]
        L.tg_strerror.restype = ctypes.c_char_p
        L.tg_version.argtypes = []
        L.tg_version.restype = ctypes.c_uint32
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().tg_strerror(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise TgError(code, what)


def _host_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Packed:
    """A host packed buffer (descriptor + sections) as produced by the library's packers."""

    def __init__(self, buf: np.ndarray):
        self.buf = buf
        self.desc = describe(buf)

    fmt = property(lambda self: self.desc.fmt)
    n = property(lambda self: self.desc.n)
    k = property(lambda self: self.desc.k)
    nnz = property(lambda self: self.desc.nnz)
    payload_bytes = property(lambda self: self.desc.bytes_payload)

    def section(self, name: str) -> np.ndarray:
        off = getattr(self.desc, "off_" + name)
        nbytes = getattr(self.desc, "bytes_" + name)
        return self.buf[off:off + nbytes]

    def sign_bytes(self) -> np.ndarray:
        return self.section("signs")[: (self.nnz + 7) // 8]

    def rowoff(self) -> np.ndarray:
        return self.section("index").view(np.uint32)


def _pack(fn_name: str, w: np.ndarray, *extra) -> Packed:
    w = np.ascontiguousarray(w, dtype=np.int8)
    if w.ndim != 2:
        raise ValueError("weights must be a 2-D [n, k] int8 array")
    n, k = w.shape
    fn = getattr(lib(), fn_name)
    need = ctypes.c_size_t(0)
    _check(fn(_host_ptr(w), n, k, *extra, None, 0, ctypes.byref(need)), fn_name)
    buf = np.empty(need.value, dtype=np.uint8)
    got = ctypes.c_size_t(0)
    _check(fn(_host_ptr(w), n, k, *extra, _host_ptr(buf), buf.size, ctypes.byref(got)), fn_name)
    return Packed(buf)


def pack_bitcos(w: np.ndarray) -> Packed:
    return _pack("tg_pack_bitcos", w)


def pack_5trit(w: np.ndarray) -> Packed:
    return _pack("tg_pack_5trit", w)


def pack_2bit(w: np.ndarray) -> Packed:
    return _pack("tg_pack_2bit", w)


def pack_t5b(w: np.ndarray, scale: float = 1.0) -> Packed:
    """t5b: five-trit bytes in 160-weight blocks, with the per-tensor scale in the descriptor."""
    return _pack("tg_pack_t5b", w, ctypes.c_float(scale))


PACKERS = {FMT_BITCOS: pack_bitcos, FMT_5TRIT: pack_5trit, FMT_2BIT: pack_2bit, FMT_T5B: pack_t5b}


def pack(fmt: int, w: np.ndarray, **kw) -> Packed:
    return PACKERS[fmt](w, **kw)


def groups_per_row(fmt: int, k: int) -> int:
    """Per-row count of the GEMV's group sums: 128-weight groups, or t5b's 160-weight blocks."""
    return -(-k // T5B_BLOCK) if fmt == FMT_T5B else k // TG_GROUP


def describe(buf: np.ndarray) -> TgDesc:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    d = TgDesc()
    _check(lib().tg_describe(_host_ptr(buf), buf.size, ctypes.byref(d)), "tg_describe")
    return d


def validate(buf: np.ndarray) -> None:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    _check(lib().tg_validate(_host_ptr(buf), buf.size), "tg_validate")


def unpack(buf: np.ndarray) -> np.ndarray:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    d = describe(buf)
    w = np.empty((d.n, d.k), dtype=np.int8)
    _check(lib().tg_unpack(_host_ptr(buf), buf.size, _host_ptr(w)), "tg_unpack")
    return w


# ----------------------------------------------------------------------------------------------- GPU

class DeviceWeights:
    """A packed buffer resident in GPU memory (a torch uint8 tensor) plus its host descriptor."""

    def __init__(self, packed: Packed, device="cuda"):
        import torch

        self.desc = packed.desc
        self.tensor = torch.from_numpy(packed.buf).to(device)

    @classmethod
    def from_tensor(cls, desc: TgDesc, tensor):
        obj = cls.__new__(cls)
        obj.desc = desc
        obj.tensor = tensor
        return obj

    fmt = property(lambda self: self.desc.fmt)
    n = property(lambda self: self.desc.n)
    k = property(lambda self: self.desc.k)
    payload_bytes = property(lambda self: self.desc.bytes_payload)


def _stream_handle(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require_cuda(t, dtype, name):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ternary_gemv(w: DeviceWeights, scales, x, y=None, stream=None):
    """y[m, n] = sum_g scales[n, g] * acc[m, n, g] (see include/ternary_gemv.h); for t5b weights
    scales is None and y = tensor scale * W x. Asynchronous."""
    import torch

    _require_cuda(w.tensor, torch.uint8, "weights")
    _require_cuda(x, torch.int8, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    m = x.shape[0]
    if w.fmt == FMT_T5B:
        if scales is not None:
            raise ValueError("t5b weights carry their scale; pass scales=None")
    else:
        _require_cuda(scales, torch.float16, "scales")
        if tuple(scales.shape) != (w.n, w.k // TG_GROUP):
            raise ValueError("shape mismatch between weights and scales")
    if x.shape[1] != w.k:
        raise ValueError("shape mismatch between weights and x")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    _require_cuda(y, torch.float32, "y")
    if tuple(y.shape) != (m, w.n):
        raise ValueError("y has the wrong shape")
    _check(lib().ternary_gemv(ctypes.byref(w.desc), ctypes.c_void_p(w.tensor.data_ptr()),
                              ctypes.c_void_p(scales.data_ptr() if scales is not None else None),
                              ctypes.c_void_p(x.data_ptr()),
                              ctypes.c_void_p(y.data_ptr()), m, _stream_handle(stream)), "ternary_gemv")
    return y


def ternary_gemv_acc(w: DeviceWeights, x, acc=None, stream=None):
    """int32 per-group accumulators acc[m, n, groups] (bit-exact entry point; groups = k/128, or
    ceil(k/160) blocks for t5b). Asynchronous."""
    import torch

    _require_cuda(w.tensor, torch.uint8, "weights")
    _require_cuda(x, torch.int8, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    m = x.shape[0]
    if x.shape[1] != w.k:
        raise ValueError("x has the wrong length")
    if acc is None:
        acc = torch.empty((m, w.n, groups_per_row(w.fmt, w.k)), dtype=torch.int32, device=x.device)
    _require_cuda(acc, torch.int32, "acc")
    _check(lib().ternary_gemv_acc(ctypes.byref(w.desc), ctypes.c_void_p(w.tensor.data_ptr()),
                                  ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(acc.data_ptr()), m,
                                  _stream_handle(stream)), "ternary_gemv_acc")
    return acc


def quantize_x(x, xq=None, x_scales=None, stream=None):
    """Per-group int8 quantisation of float32 activations [m, k] (tg_quantize_x): returns (xq int8
    [m, k], x_scales float32 [m, k/128]). Asynchronous."""
    import torch

    _require_cuda(x, torch.float32, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scales is None:
        x_scales = torch.empty((m, k // TG_GROUP), dtype=torch.float32, device=x.device)
    _require_cuda(xq, torch.int8, "xq")
    _require_cuda(x_scales, torch.float32, "x_scales")
    if tuple(xq.shape) != (m, k) or tuple(x_scales.shape) != (m, k // TG_GROUP):
        raise ValueError("xq or x_scales has the wrong shape")
    _check(lib().tg_quantize_x(ctypes.c_void_p(x.data_ptr()), m, k, ctypes.c_void_p(xq.data_ptr()),
                               ctypes.c_void_p(x_scales.data_ptr()), _stream_handle(stream)), "tg_quantize_x")
    return xq, x_scales


def ternary_gemv_xs(w: DeviceWeights, scales, xq, x_scales, y=None, stream=None):
    """y[m, n] = sum_g scales[n, g] * x_scales[m, g] * acc[m, n, g] on quantised activations
    (ternary_gemv_xs). Asynchronous."""
    import torch

    _require_cuda(w.tensor, torch.uint8, "weights")
    _require_cuda(scales, torch.float16, "scales")
    _require_cuda(xq, torch.int8, "xq")
    _require_cuda(x_scales, torch.float32, "x_scales")
    if xq.dim() == 1:
        xq = xq.view(1, -1)
    if x_scales.dim() == 1:
        x_scales = x_scales.view(1, -1)
    m = xq.shape[0]
    if (xq.shape[1] != w.k or tuple(scales.shape) != (w.n, w.k // TG_GROUP)
            or tuple(x_scales.shape) != (m, w.k // TG_GROUP)):
        raise ValueError("shape mismatch between weights, scales, xq and x_scales")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=xq.device)
    _require_cuda(y, torch.float32, "y")
    if tuple(y.shape) != (m, w.n):
        raise ValueError("y has the wrong shape")
    _check(lib().ternary_gemv_xs(ctypes.byref(w.desc), ctypes.c_void_p(w.tensor.data_ptr()),
                                 ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(xq.data_ptr()),
                                 ctypes.c_void_p(x_scales.data_ptr()), ctypes.c_void_p(y.data_ptr()), m,
                                 _stream_handle(stream)), "ternary_gemv_xs")
    return y


def ternary_gemv_f16(w: DeviceWeights, scales, x16, y=None, stream=None):
    """y[m, n] = sum_g scales[n, g] * sum_{k in g} W[n, k] * x16[m, k] for fp16 activations on BITCOS
    weights (ternary_gemv_f16). Asynchronous."""
    import torch

    _require_cuda(w.tensor, torch.uint8, "weights")
    _require_cuda(scales, torch.float16, "scales")
    _require_cuda(x16, torch.float16, "x16")
    if x16.dim() == 1:
        x16 = x16.view(1, -1)
    m = x16.shape[0]
    if x16.shape[1] != w.k or tuple(scales.shape) != (w.n, w.k // TG_GROUP):
        raise ValueError("shape mismatch between weights, scales and x16")
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device=x16.device)
    _require_cuda(y, torch.float32, "y")
    if tuple(y.shape) != (m, w.n):
        raise ValueError("y has the wrong shape")
    _check(lib().ternary_gemv_f16(ctypes.byref(w.desc), ctypes.c_void_p(w.tensor.data_ptr()),
                                  ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(x16.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), m, _stream_handle(stream)), "ternary_gemv_f16")
    return y


class Plan:
    """Several GEMVs of one format run as one launch (tg_plan_init / ternary_gemv_plan).

    weights: list of DeviceWeights; xs: int8 [m, k] device tensors; scales and ys (fp16 [n, k/128],
    float32 [m, n]) for fp32 outputs, or accs (int32 [m, n, k/128]) for accumulator outputs. With
    x_scales (float32 [m, k/128] per GEMV) the xs are quantised activations and every group term is
    also multiplied by its activation group scale (tg_plan_init_xs). With f16=True the xs are fp16
    [m, k] activations of BITCOS GEMVs with fp32 outputs, m <= 16 (tg_plan_init_f16). The plan keeps
    references to every tensor it names, and its device table, for its lifetime.
    """

    def __init__(self, weights, xs, scales=None, ys=None, accs=None, x_scales=None, f16=False, noalloc=False):
        import torch

        count = len(weights)
        if count < 1 or len(xs) != count:
            raise ValueError("one x per weight matrix is required")
        acc_mode = accs is not None
        if acc_mode:
            if len(accs) != count or x_scales is not None:
                raise ValueError("one acc per weight matrix is required (and no x_scales)")
        elif ys is None or len(ys) != count:
            raise ValueError("ys (one per matrix) are required for fp32 outputs")
        t5b = weights[0].fmt == FMT_T5B
        if not acc_mode and (t5b != (scales is None) or (scales is not None and len(scales) != count)):
            raise ValueError("scales (one per matrix) are required for fp32 outputs, and must be None for t5b")
        if x_scales is not None and len(x_scales) != count:
            raise ValueError("one x_scales per weight matrix is required")
        m = xs[0].shape[0] if xs[0].dim() == 2 else 1
        for i, w in enumerate(weights):
            _require_cuda(w.tensor, torch.uint8, "weights")
            _require_cuda(xs[i], torch.float16 if f16 else torch.int8, "x")
            if xs[i].shape[-1] != w.k or (xs[i].shape[0] if xs[i].dim() == 2 else 1) != m:
                raise ValueError("every x must be [m, k] with the same m")
            if acc_mode:
                _require_cuda(accs[i], torch.int32, "acc")
                if tuple(accs[i].shape) != (m, w.n, groups_per_row(w.fmt, w.k)):
                    raise ValueError("acc has the wrong shape")
            else:
                _require_cuda(ys[i], torch.float32, "y")
                if tuple(ys[i].shape) != (m, w.n):
                    raise ValueError("y has the wrong shape")
                if scales is not None:
                    _require_cuda(scales[i], torch.float16, "scales")
                    if tuple(scales[i].shape) != (w.n, w.k // TG_GROUP):
                        raise ValueError("scales has the wrong shape")
                if x_scales is not None:
                    _require_cuda(x_scales[i], torch.float32, "x_scales")
                    if tuple(x_scales[i].reshape(m, -1).shape) != (m, w.k // TG_GROUP):
                        raise ValueError("x_scales has the wrong shape")
        L = lib()
        descs = (TgDesc * count)(*[w.desc for w in weights])
        P = ctypes.c_void_p * count
        ptr = lambda ts: P(*[t.data_ptr() for t in ts]) if ts is not None else None
        self.plan = TgPlan()
        self._keep = (list(weights), list(xs), scales, ys, accs, x_scales)
        if noalloc:
            # the table goes to the library's static device array (tg_plan_init_noalloc)
            if f16 or x_scales is not None:
                raise ValueError("tg_plan_init_noalloc takes int8 activations (fp32 y or int32 accumulators)")
            self.table = None
            _check(L.tg_plan_init_noalloc(ctypes.byref(self.plan), count, descs, ptr([w.tensor for w in weights]),
                                          ptr(scales), ptr(xs), ptr(ys), ptr(accs), m), "tg_plan_init_noalloc")
            return
        nbytes = L.tg_plan_table_bytes(count)
        self.table = torch.empty(nbytes, dtype=torch.uint8, device=xs[0].device)
        if f16:
            if acc_mode or x_scales is not None:
                raise ValueError("fp16 plans write fp32 y only")
            _check(L.tg_plan_init_f16(ctypes.byref(self.plan), ctypes.c_void_p(self.table.data_ptr()), nbytes, count,
                                      descs, ptr([w.tensor for w in weights]), ptr(scales), ptr(xs), ptr(ys), m),
                   "tg_plan_init_f16")
        elif x_scales is not None:
            _check(L.tg_plan_init_xs(ctypes.byref(self.plan), ctypes.c_void_p(self.table.data_ptr()), nbytes, count,
                                     descs, ptr([w.tensor for w in weights]), ptr(scales), ptr(xs), ptr(x_scales),
                                     ptr(ys), m), "tg_plan_init_xs")
        else:
            _check(L.tg_plan_init(ctypes.byref(self.plan), ctypes.c_void_p(self.table.data_ptr()), nbytes, count,
                                  descs, ptr([w.tensor for w in weights]), ptr(scales), ptr(xs), ptr(ys), ptr(accs),
                                  m), "tg_plan_init")

    def set_decode(self, decode: int):
        """Decode strategy: DECODE_BYTE, DECODE_NIBBLE (BITCOS) or DECODE_ARITH (five-trit, t5b, 2-bit)
        (tg_plan_set_decode). A new plan decodes by table (DECODE_BYTE), except 2-bit plans that may take
        DECODE_ARITH, which start with it."""
        _check(lib().tg_plan_set_decode(ctypes.byref(self.plan), decode), "tg_plan_set_decode")
        return self

    def run(self, stream=None):
        _check(lib().ternary_gemv_plan(ctypes.byref(self.plan), _stream_handle(stream)), "ternary_gemv_plan")


def stream_read(buf, sink, blocks: int, unroll: int, stream=None):
    """Bandwidth reference: read all of `buf` (a uint8 device tensor) with the stream-read kernel."""
    import torch

    _require_cuda(buf, torch.uint8, "buf")
    _require_cuda(sink, torch.int32, "sink")
    if sink.numel() < blocks * 4:
        raise ValueError("sink needs blocks * 4 words")
    _check(lib().tg_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), ctypes.c_void_p(sink.data_ptr()),
                                blocks, unroll, _stream_handle(stream)), "tg_stream_read")


def clock_probe(out, slot: int, spin_ticks: int = 100, stream=None):
    """Counter samples into out[4 slot .. 4 slot + 3] (an int64 device tensor): constant 100 MHz counter
    and shader-clock counter, at the start and after spin_ticks of the constant counter (tg_clock_probe)."""
    import torch

    _require_cuda(out, torch.int64, "out")
    if out.numel() < 4 * (slot + 1):
        raise ValueError("out needs 4 * (slot + 1) values")
    _check(lib().tg_clock_probe(ctypes.c_void_p(out.data_ptr()), slot, spin_ticks, _stream_handle(stream)),
           "tg_clock_probe")
