"""MI355X (gfx950) ternary GEMV: BITCOS / five-trit / 2-bit packed weights, int8 activations.

The compute path is libternary_gemv.so (C ABI in include/ternary_gemv.h; HIP kernels for gfx950);
this package is its Python binding plus the seeded synthetic-input generator.
"""
from .binding import (DECODE_ARITH, DECODE_BYTE, DECODE_NIBBLE, FMT_2BIT, FMT_5TRIT, FMT_BITCOS, FMT_NAMES, FMT_T5B, groups_per_row, pack_t5b, TG_GROUP, TG_MAX_M, DeviceWeights, Packed,
                      Plan, TgError, describe, pack, pack_2bit, pack_5trit, pack_bitcos, quantize_x, ternary_gemv,
                      ternary_gemv_acc, ternary_gemv_f16, ternary_gemv_xs, unpack, validate)

__all__ = ["FMT_BITCOS", "FMT_5TRIT", "FMT_2BIT", "FMT_T5B", "FMT_NAMES", "groups_per_row", "pack_t5b", "TG_GROUP", "TG_MAX_M", "DeviceWeights", "Packed",
           "Plan", "TgError", "describe", "pack", "pack_bitcos", "pack_5trit", "pack_2bit", "ternary_gemv",
           "ternary_gemv_acc", "ternary_gemv_xs", "ternary_gemv_f16", "quantize_x", "DECODE_BYTE", "DECODE_NIBBLE", "DECODE_ARITH", "unpack", "validate"]
