"""Seeded synthetic inputs for the ternary GEMV (weights, fp16 group scales, int8 activations).

This module holds no part of the method's arithmetic: it only draws numbers. Both the HIP path's
tests/bench and the CPU oracle's tests take their inputs from here, so the two sides see the same
tensors without sharing any packing, decoding or contraction code.

Generator: a counter-based SplitMix64. Element i of stream (seed, tensor_id) is
``mix(key(seed, tensor_id) + (i + 1) * GAMMA)`` where ``mix`` is SplitMix64's finaliser
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) and
``GAMMA = 0x9E3779B97F4A7C15``. Because element i depends only on (seed, tensor_id, i), any slice
can be drawn independently and in any order.

Distributions (the workloads of the pages: iid ternary weights at a measured zero density z, with
the non-zeros split evenly between +1 and -1; group-128 fp16 scales; int8 activations):
  * ternary: 0 with probability z, +1 and -1 with probability (1 - z) / 2 each;
  * scales: float16(round-to-nearest-even(uniform[0.01, 0.1]));
  * activations: int8 uniform on [-127, 127].
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 24

# Stream ids: each tensor role gets its own stream so that changing one never perturbs another.
STREAM_W = 1
STREAM_SCALE = 2
STREAM_X = 3
STREAM_DEAD = 4
STREAM_XF = 5


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> np.uint64:
    """Key of one stream: the finaliser applied to a combination of the seed and the tensor id."""
    with np.errstate(over="ignore"):
        a = np.array([(seed * 0xD1B54A32D192ED03 + tensor_id * 0x8CB92BA72F3D8DD7 + 1) & (2**64 - 1)],
                     dtype=np.uint64)
        return _mix(a)[0]


def raw_u64(key: np.uint64, start: int, count: int) -> np.ndarray:
    """count consecutive 64-bit draws of the stream with the given key, from counter index start."""
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            hi = min(count, lo + _CHUNK)
            idx = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
            out[lo:hi] = _mix(key + idx * GAMMA)
    return out


def _u53(key: np.uint64, start: int, count: int) -> np.ndarray:
    return raw_u64(key, start, count) >> np.uint64(11)


def tensor_id(layer: int, role: int, kind: int) -> int:
    """Stream id for (layer, matrix role, tensor kind); kinds are the STREAM_* constants."""
    return (layer * 64 + role) * 8 + kind


def ternary(n: int, k: int, z: float, seed: int = 0, tid: int = STREAM_W) -> np.ndarray:
    """int8 [n, k] with P(0) = z and P(+1) = P(-1) = (1 - z) / 2, decided on 53-bit integers."""
    if not (0.0 <= z <= 1.0):
        raise ValueError("zero density must lie in [0, 1]")
    key = stream_key(seed, tid)
    t0 = np.uint64(min(int(z * 2.0**53), 2**53))
    t1 = np.uint64(min(int((z + (1.0 - z) / 2.0) * 2.0**53), 2**53))
    out = np.empty(n * k, dtype=np.int8)
    for lo in range(0, n * k, _CHUNK):
        hi = min(n * k, lo + _CHUNK)
        u = _u53(key, lo, hi - lo)
        v = np.where(u < t0, 0, np.where(u < t1, 1, -1)).astype(np.int8)
        out[lo:hi] = v
    return out.reshape(n, k)


def exact_density_ternary(n: int, k: int, zeros: int, seed: int = 0, tid: int = STREAM_W) -> np.ndarray:
    """int8 [n, k] with exactly `zeros` zeros at seeded random positions and seeded random signs."""
    total = n * k
    if not (0 <= zeros <= total):
        raise ValueError("zero count out of range")
    key = stream_key(seed, tid)
    order = np.argsort(raw_u64(key, 0, total), kind="stable")
    signs = np.where((raw_u64(key, total, total) >> np.uint64(63)) == 0, 1, -1).astype(np.int8)
    out = signs.copy()
    out[order[:zeros]] = 0
    return out.reshape(n, k)


def scales(n: int, ng: int, seed: int = 0, tid: int = STREAM_SCALE, lo: float = 0.01, hi: float = 0.1) -> np.ndarray:
    """float16 [n, ng]: uniform[lo, hi] in float64, rounded to nearest-even float16."""
    u = _u53(stream_key(seed, tid), 0, n * ng).astype(np.float64) * 2.0**-53
    return (lo + (hi - lo) * u).astype(np.float16).reshape(n, ng)


def activations(m: int, k: int, seed: int = 0, tid: int = STREAM_X) -> np.ndarray:
    """int8 [m, k] uniform on [-127, 127]."""
    u = _u53(stream_key(seed, tid), 0, m * k)
    v = (u * np.uint64(255)) >> np.uint64(53)
    return (v.astype(np.int16) - 127).astype(np.int8).reshape(m, k)


def float_activations(m: int, k: int, seed: int = 0, tid: int = STREAM_XF) -> np.ndarray:
    """float32 [m, k]: uniform[-1, 1] times a per-128-block magnitude 10^e, e uniform[-1, 1], so that
    blocks differ in range (as activation channels do); every value is finite and normal."""
    key = stream_key(seed, tid)
    u = _u53(key, 0, m * k).astype(np.float64) * 2.0**-53
    e = _u53(key, m * k, m * (k // 128)).astype(np.float64) * 2.0**-53
    mag = np.repeat(10.0 ** (2.0 * e - 1.0), 128)
    return ((2.0 * u - 1.0) * mag).astype(np.float32).reshape(m, k)


def dead_rows(n: int, count: int, seed: int = 0, tid: int = STREAM_DEAD) -> np.ndarray:
    """Sorted indices of `count` rows chosen by a seeded permutation of range(n)."""
    order = np.argsort(raw_u64(stream_key(seed, tid), 0, n), kind="stable")
    return np.sort(order[:count])
