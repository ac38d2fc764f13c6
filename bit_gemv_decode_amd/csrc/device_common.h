// Device helpers shared by the GEMV kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// DPP control codes (GFX9 encoding).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]

// Inclusive prefix sum over the 64 lanes of a wave (every lane must be active).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr1, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr2, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr4, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr8, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false);
    return v;
}

// Sum over each aligned group of 4 lanes; every lane of the quad receives the sum.
__device__ __forceinline__ int quad_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap2, 0xF, 0xF, false);
    return v;
}

// Sum of a double over all 64 lanes (every lane receives it).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// IEEE binary16 bit pattern -> float (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

}  // namespace tg
