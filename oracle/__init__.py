"""CPU oracle for the ternary GEMV -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package. The
product path never imports it and shares no code with it. The arithmetic lives in ``oracle.c``
(plain C, built with gcc); this module only builds it and marshals numpy arrays.

Every function here is a thin wrapper; see ``oracle.c`` for which passage of the pages each step
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
GROUP = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP over rows, no intrinsics)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-o", tmp, SRC, "-lm"],
                       check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB selects another build of oracle.c (e.g. one with sanitizers); it is used as it is
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = LIB
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
        L = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_pdep64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.oracle_pdep64.restype = ctypes.c_uint64
        L.oracle_count_nonzero.argtypes = [p, i64]
        L.oracle_count_nonzero.restype = i64
        L.oracle_bitcos_pack.argtypes = [p, i64, i64, p, i64, p, i64, p]
        L.oracle_bitcos_pack.restype = i64
        L.oracle_bitcos_unpack.argtypes = [p, p, i64, i64, p]
        L.oracle_bitcos_unpack.restype = i64
        L.oracle_t5_bytes.argtypes = [i64, i64]
        L.oracle_t5_bytes.restype = i64
        for name in ("oracle_t5_pack", "oracle_b2_pack"):
            getattr(L, name).argtypes = [p, i64, i64, p]
            getattr(L, name).restype = ctypes.c_int
        for name in ("oracle_t5_unpack", "oracle_b2_unpack"):
            getattr(L, name).argtypes = [p, i64, i64, p]
            getattr(L, name).restype = ctypes.c_int
        L.oracle_gemv_acc.argtypes = [p, i64, i64, p, i64, p]
        L.oracle_gemv_acc.restype = None
        L.oracle_combine.argtypes = [p, p, i64, i64, i64, p]
        L.oracle_combine.restype = None
        L.oracle_quantize_x.argtypes = [p, i64, i64, p, p]
        L.oracle_quantize_x.restype = None
        L.oracle_combine_xs.argtypes = [p, p, p, i64, i64, i64, p]
        L.oracle_combine_xs.restype = None
        L.oracle_t5b_blocks.argtypes = [i64]
        L.oracle_t5b_blocks.restype = i64
        L.oracle_t5b_pack.argtypes = [p, i64, i64, p]
        L.oracle_t5b_pack.restype = ctypes.c_int
        L.oracle_t5b_unpack.argtypes = [p, i64, i64, p]
        L.oracle_t5b_unpack.restype = ctypes.c_int
        L.oracle_gemv_acc_blocks.argtypes = [p, i64, i64, p, i64, p]
        L.oracle_gemv_acc_blocks.restype = None
        L.oracle_combine_tensor.argtypes = [p, ctypes.c_float, i64, i64, i64, p]
        L.oracle_combine_tensor.restype = None
        L.oracle_gemv_f16.argtypes = [p, p, p, i64, i64, i64, p]
        L.oracle_gemv_f16.restype = None
        L.oracle_gemv_packed.argtypes = [ctypes.c_int, p, p, p, p, i64, i64, p, i64, p]
        L.oracle_gemv_packed.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h) & 0xFFFF)


def pdep64(src: int, mask: int) -> int:
    return int(lib().oracle_pdep64(src & (2**64 - 1), mask & (2**64 - 1)))


class Bitcos:
    """The BITCOS sections the oracle writes: bitmap bits, sign bits, per-row sign offsets."""

    def __init__(self, bitmap: np.ndarray, signs: np.ndarray, rowoff: np.ndarray, nnz: int, n: int, k: int):
        self.bitmap, self.signs, self.rowoff, self.nnz, self.n, self.k = bitmap, signs, rowoff, nnz, n, k

    def symbol_bits(self) -> int:
        return self.n * self.k + self.nnz


def bitcos_pack(w: np.ndarray) -> Bitcos:
    w = _c(w, np.int8)
    n, k = w.shape
    nnz = lib().oracle_count_nonzero(_ptr(w), n * k)
    if nnz < 0:
        raise ValueError("non-ternary weight")
    bitmap = np.zeros((n * k + 7) // 8, np.uint8)
    signs = np.zeros(max(1, (nnz + 7) // 8), np.uint8)
    rowoff = np.zeros(n + 1, np.uint32)
    got = lib().oracle_bitcos_pack(_ptr(w), n, k, _ptr(bitmap), bitmap.size, _ptr(signs), signs.size, _ptr(rowoff))
    assert got == nnz
    return Bitcos(bitmap, signs[: (nnz + 7) // 8], rowoff, int(nnz), n, k)


def bitcos_unpack(bitmap: np.ndarray, signs: np.ndarray, n: int, k: int) -> tuple[np.ndarray, int]:
    bitmap = _c(bitmap, np.uint8)
    signs = _c(signs, np.uint8)
    if signs.size == 0:
        signs = np.zeros(1, np.uint8)
    w = np.empty((n, k), np.int8)
    used = lib().oracle_bitcos_unpack(_ptr(bitmap), _ptr(signs), n, k, _ptr(w))
    return w, int(used)


def t5_pack(w: np.ndarray) -> np.ndarray:
    w = _c(w, np.int8)
    n, k = w.shape
    out = np.zeros(lib().oracle_t5_bytes(n, k), np.uint8)
    if lib().oracle_t5_pack(_ptr(w), n, k, _ptr(out)):
        raise ValueError("five-trit pack rejected the input")
    return out


def t5_unpack(codes: np.ndarray, n: int, k: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    w = np.empty((n, k), np.int8)
    if lib().oracle_t5_unpack(_ptr(codes), n, k, _ptr(w)):
        raise ValueError("invalid five-trit code")
    return w


def t5b_blocks(k: int) -> int:
    return int(lib().oracle_t5b_blocks(k))


def t5b_pack(w: np.ndarray) -> np.ndarray:
    """uint8 [n, blocks, 32]: five-trit bytes in blocks of 160 weights (padding digits weight 0)."""
    w = _c(w, np.int8)
    n, k = w.shape
    out = np.zeros((n, t5b_blocks(k), 32), np.uint8)
    if lib().oracle_t5b_pack(_ptr(w), n, k, _ptr(out)):
        raise ValueError("t5b pack rejected the input")
    return out


def t5b_unpack(codes: np.ndarray, n: int, k: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    assert codes.size == n * t5b_blocks(k) * 32
    w = np.empty((n, k), np.int8)
    if lib().oracle_t5b_unpack(_ptr(codes), n, k, _ptr(w)):
        raise ValueError("invalid t5b code")
    return w


def gemv_acc_blocks(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """int32 [m, n, blocks]: exact sums of W*x over each 160-weight block of each row."""
    w = _c(w, np.int8)
    x = _c(np.atleast_2d(x), np.int8)
    n, k = w.shape
    m = x.shape[0]
    acc = np.empty((m, n, t5b_blocks(k)), np.int32)
    lib().oracle_gemv_acc_blocks(_ptr(w), n, k, _ptr(x), m, _ptr(acc))
    return acc


def combine_tensor(acc: np.ndarray, scale: float) -> np.ndarray:
    """float32 [m, n]: the per-tensor scale times the exact row sum, rounded once."""
    acc = _c(acc, np.int32)
    m, n, nb = acc.shape
    y = np.empty((m, n), np.float32)
    lib().oracle_combine_tensor(_ptr(acc), float(np.float32(scale)), n, nb, m, _ptr(y))
    return y


def b2_pack(w: np.ndarray) -> np.ndarray:
    w = _c(w, np.int8)
    n, k = w.shape
    out = np.zeros(n * k // 4, np.uint8)
    if lib().oracle_b2_pack(_ptr(w), n, k, _ptr(out)):
        raise ValueError("2-bit pack rejected the input")
    return out


def b2_unpack(codes: np.ndarray, n: int, k: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    w = np.empty((n, k), np.int8)
    if lib().oracle_b2_unpack(_ptr(codes), n, k, _ptr(w)):
        raise ValueError("invalid 2-bit code")
    return w


def gemv_acc(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """int32 [m, n, k/128] per-group accumulators of the dense definition."""
    w = _c(w, np.int8)
    x = _c(np.atleast_2d(x), np.int8)
    n, k = w.shape
    m = x.shape[0]
    assert x.shape[1] == k and k % GROUP == 0
    acc = np.empty((m, n, k // GROUP), np.int32)
    lib().oracle_gemv_acc(_ptr(w), n, k, _ptr(x), m, _ptr(acc))
    return acc


def combine(acc: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float32 [m, n]: the fp64 sum over groups of scale * acc, rounded once."""
    acc = _c(acc, np.int32)
    sc = _c(scales, np.float16).view(np.uint16)
    m, n, ng = acc.shape
    assert sc.shape == (n, ng)
    y = np.empty((m, n), np.float32)
    lib().oracle_combine(_ptr(acc), _ptr(sc), n, ng, m, _ptr(y))
    return y


def gemv(w: np.ndarray, scales: np.ndarray, x: np.ndarray) -> np.ndarray:
    return combine(gemv_acc(w, x), scales)


def gemv_f16(w: np.ndarray, scales: np.ndarray, x: np.ndarray) -> np.ndarray:
    """float32 [m, n]: the GEMV against fp16 activations [m, k], exact up to the final rounding."""
    w = _c(w, np.int8)
    sc = _c(scales, np.float16).view(np.uint16)
    x16 = _c(np.atleast_2d(x), np.float16).view(np.uint16)
    n, k = w.shape
    m = x16.shape[0]
    assert sc.shape == (n, k // GROUP) and x16.shape[1] == k
    y = np.empty((m, n), np.float32)
    lib().oracle_gemv_f16(_ptr(w), _ptr(sc), _ptr(x16), n, k, m, _ptr(y))
    return y


def quantize_x(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-group int8 quantisation of float32 activations [m, k]: (int8 codes [m, k], float32 group
    scales [m, k/128])."""
    x = _c(np.atleast_2d(x), np.float32)
    m, k = x.shape
    assert k % GROUP == 0
    xq = np.empty((m, k), np.int8)
    xs = np.empty((m, k // GROUP), np.float32)
    lib().oracle_quantize_x(_ptr(x), m, k, _ptr(xq), _ptr(xs))
    return xq, xs


def combine_xs(acc: np.ndarray, scales: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """float32 [m, n]: the fp64 sum over groups of (scale * acc) * xs, rounded once."""
    acc = _c(acc, np.int32)
    sc = _c(scales, np.float16).view(np.uint16)
    m, n, ng = acc.shape
    xs = _c(xs, np.float32)
    assert sc.shape == (n, ng) and xs.shape == (m, ng)
    y = np.empty((m, n), np.float32)
    lib().oracle_combine_xs(_ptr(acc), _ptr(sc), _ptr(xs), n, ng, m, _ptr(y))
    return y


def gemv_xs(w: np.ndarray, scales: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The GEMV of float32 activations quantised per group: quantise, contract, combine."""
    xq, xs = quantize_x(x)
    return combine_xs(gemv_acc(w, xq), scales, xs)


FMT_BITCOS, FMT_5TRIT, FMT_2BIT = 1, 2, 3


def gemv_packed(fmt: int, a: np.ndarray, b: np.ndarray | None, rowoff: np.ndarray | None, scales: np.ndarray,
                n: int, k: int, x: np.ndarray) -> np.ndarray:
    """Row-parallel GEMV decoding each row from packed bytes (the CPU baseline)."""
    a = _c(a, np.uint8)
    b = _c(b if b is not None and np.size(b) else np.zeros(1, np.uint8), np.uint8)
    ro = _c(rowoff if rowoff is not None else np.zeros(n + 1, np.uint32), np.uint32)
    sc = _c(scales, np.float16).view(np.uint16)
    x = _c(np.atleast_2d(x), np.int8)
    m = x.shape[0]
    y = np.empty((m, n), np.float32)
    if lib().oracle_gemv_packed(fmt, _ptr(a), _ptr(b), _ptr(ro), _ptr(sc), n, k, _ptr(x), m, _ptr(y)):
        raise ValueError("oracle_gemv_packed rejected the input")
    return y


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of later oracle calls (timing only: results do not depend on it)."""
    lib().oracle_set_threads(int(n))
