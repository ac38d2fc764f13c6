"""Comparison bounds of the parity checks -- test infrastructure, like the rest of ``oracle/``.

Every GPU check of an fp32 output against the oracle goes through one of these functions, so that
each path has exactly one bound, stated and derived here.

int8 activations (fp32 y; also the quantised-activation path with activation group scales):
    The oracle rounds the exact sum y = sum_g t_g, t_g = s_g * acc_g (* xs_g), once to fp32
    ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C: int32 group sums, the scale applied
    once per group). The required agreement is 1e-5 relative. Measured against |y_ref| alone that
    fails where cancellation makes y_ref tiny, so the scale of the comparison is the larger of |y_ref|
    and the typical size of the terms:
        |y - y_ref| <= 1e-5 * max(|y_ref|, sum_g |t_g| / sqrt(ng))
    The kernels add exact fp64 products (fp16 times an int32 of at most 15 bits), so in practice y is
    bit-identical; the checks also count the elements that differ at all.

t5b (one fp32 scale per tensor, per-block sums):
    the same form with t_b = scale * acc_b over the ceil(k/160) blocks.

fp16 activations:
    The exact value is y = sum_g s_g * sum_{k in g} W[k] x16[k]. The kernels form each group sum in
    fp32: every product W x16 is exact (x16 is binary16, W in {-1, 0, 1}), and at most 127 additions
    of partial sums each no larger than S_g = sum_{k in g} |W x16| in magnitude are rounded, so the
    group error is at most gamma_127 * S_g with gamma_n = n u / (1 - n u), u = 2^-24, and gamma_127 =
    (127/128)(1 + 7.6e-6) 2^-17. The product with s_g is exact in fp64 (a 24-bit significand times an
    11-bit one); the fp64 sum over at most 2^16 groups adds at most 2^-37 of sum_g |s_g| S_g; the
    final store rounds once more, by at most u |v| for the fp64 value v. Altogether
        |y - y_exact| <= 2^-24 |y_exact| + 2^-17 * sum_g |s_g| S_g
    (the factor 127/128 in gamma_127 absorbs the second-order terms), which the checks widen to
        |y - y_ref| <= 2^-22 |y_ref| + 2^-17 * sum_g |s_g| S_g,
    the slack in the first term covering the gap between y_exact and the oracle's correctly rounded
    y_ref (at most 2^-24 |y_exact|).
"""
from __future__ import annotations

import numpy as np

REL = 1e-5  # the required relative agreement of fp32 outputs


def int8_y_ok(y, y_ref, acc, scales, xs=None):
    """(within the bound, number of elements that differ) for fp32 y of the int8 path.

    acc: int32 [m][n][ng]; scales: fp16 or float [n][ng]; xs: optional float [m][ng]."""
    t = scales.astype(np.float64)[None, :, :] * acc.astype(np.float64)
    if xs is not None:
        t = t * xs.astype(np.float64)[:, None, :]
    size = np.abs(t).sum(-1) / np.sqrt(acc.shape[-1])
    bound = REL * np.maximum(np.abs(y_ref.astype(np.float64)), size)
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    return bool(np.all(err <= bound)), int((y != y_ref).sum())


def tensor_y_ok(y, y_ref, acc, scale):
    """The same check for t5b: acc int32 [m][n][blocks], one fp32 tensor scale."""
    t = np.abs(float(scale) * acc.astype(np.float64)).sum(-1) / np.sqrt(acc.shape[-1])
    bound = REL * np.maximum(np.abs(y_ref.astype(np.float64)), t)
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    return bool(np.all(err <= bound)), int((y != y_ref).sum())


def f16_bound(w, scales, x16, y_ref):
    """The fp16-activation bound, element by element: 2^-22 |y_ref| + 2^-17 sum_g |s_g| S_g.

    w: int8 [n][k]; scales: [n][ng]; x16: binary16 [m][k]; y_ref: [m][n]."""
    m, k = x16.shape
    n = w.shape[0]
    ng = k // 128
    prod = np.abs(x16.astype(np.float64))[:, None, :] * np.abs(w.astype(np.float64))[None]
    sg = prod.reshape(m, n, ng, 128).sum(-1)
    t = (np.abs(scales.astype(np.float64))[None] * sg).sum(-1)
    return 2.0 ** -22 * np.abs(y_ref.astype(np.float64)) + 2.0 ** -17 * t


def f16_y_ok(y, y_ref, w, scales, x16):
    """(within the fp16 bound, worst error as a multiple of the bound)."""
    bound = f16_bound(w, scales, x16, y_ref)
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    return bool(np.all(err <= bound)), worst
