// Device helpers shared by the GEMV kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_internal.h"

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

constexpr int kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141;

// v moved across lanes by one DPP pattern. Lanes in rows the mask leaves out receive an undefined
// value: only use results from lanes whose source is defined.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum of v over each aligned group of `width` lanes (width 1, 2, 4, 8 or 16, wave-uniform); every lane
// of the group receives it. width 32: lanes 31 and 63 receive their half's sum. width 64: lane 63
// receives the total. In every case the last lane of each group holds the group's sum. All lanes
// must be active.
__device__ __forceinline__ double seg_sum_f64(double v, int width) {
    if (width >= 2) v += dpp_f64<kDppQuadSwap1>(v);
    if (width >= 4) v += dpp_f64<kDppQuadSwap2>(v);
    if (width >= 8) v += dpp_f64<kDppRowHalfMirror>(v);
    if (width >= 16) v += dpp_f64<kDppRowMirror>(v);
    if (width >= 32) v += dpp_f64<kDppRowBcast15, 0xA>(v);
    if (width >= 64) v += dpp_f64<kDppRowBcast31, 0xC>(v);
    return v;
}

// Total of v over the wave, returned as a wave-uniform value.
__device__ __forceinline__ double wave_total_f64(double v) {
    v = seg_sum_f64(v, 64);
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// IEEE binary16 bit pattern -> float (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw (untyped) buffer resource over `bytes` bytes at p. Loads through it that fall outside the
// range return zero instead of faulting. Loads through buffer intrinsics are also never merged
// across loop iterations by the compiler, which keeps software-pipelined loads where they are
// written. Ranges are limited to 4 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ u32x3 buf_u32x3(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Wave-uniform copies of values the compiler cannot prove uniform (e.g. loaded from a table in
// global memory with a vector load): buffer resources built from them then live in scalar
// registers instead of being rebuilt per lane in a loop around every load.
__device__ __forceinline__ int32_t uniform_i32(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return (T *)(uintptr_t)(lo | (hi << 32));
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// GEMV description i of a launch: entry i of its table, or the one passed by value. Table entries are
// read through the constant address space, so that the wave fetches them with scalar loads straight
// into scalar registers (a generic pointer would take vector loads that the wave must wait for and
// move to scalar registers before going on, e.g. before the table fill it should overlap).
__device__ __forceinline__ Problem launch_problem(const GroupArgs &ga, int i) {
    static_assert(sizeof(Problem) % 4 == 0, "whole words");
    constexpr int kWords = (int)(sizeof(Problem) / 4);
    if (!ga.table) return ga.one;
    typedef const __attribute__((address_space(4))) uint32_t *ConstWords;
    const ConstWords src = (ConstWords)ga.table + (size_t)i * kWords;
    uint32_t w[kWords];
#pragma unroll
    for (int j = 0; j < kWords; ++j) w[j] = src[j];
    return __builtin_bit_cast(Problem, w);
}

// Entry r of a BITCOS GEMV's row index (the stream position of row r's first sign), read with a scalar
// load through the constant address space: the wave waits for it only where the value is used.
__device__ __forceinline__ uint32_t row_index_entry(const Problem &p, int r) {
    typedef const __attribute__((address_space(4))) uint32_t *ConstWords;
    return ((ConstWords)p.rowoff)[r];
}

// A GEMV description (read from a table, or passed by value) as wave-uniform values.
__device__ __forceinline__ Problem uniform_problem(const Problem &q) {
    Problem p;
    p.codes = uniform_ptr(q.codes);
    p.signs = uniform_ptr(q.signs);
    p.rowoff = uniform_ptr(q.rowoff);
    p.scales = uniform_ptr(q.scales);
    p.x = uniform_ptr(q.x);
    p.y = uniform_ptr(q.y);
    p.acc = uniform_ptr(q.acc);
    p.xs = uniform_ptr(q.xs);
    p.codes_bytes = uniform_u32(q.codes_bytes);
    p.sign_bytes = uniform_u32(q.sign_bytes);
    p.n = uniform_i32(q.n);
    p.k = uniform_i32(q.k);
    p.unit_begin = uniform_i32(q.unit_begin);
    p.nunits = uniform_i32(q.nunits);
    p.ng = uniform_i32(q.ng);
    p.nch = uniform_i32(q.nch);
    p.G = uniform_i32(q.G);
    p.R = uniform_i32(q.R);
    p.glast = uniform_i32(q.glast);
    p.nbu = uniform_i32(q.nbu);
    p.rpu = uniform_i32(q.rpu);
    p.gmagic = uniform_u32(q.gmagic);
    p.rmagic = uniform_u32(q.rmagic);
    p.tscale = __builtin_bit_cast(float, uniform_u32(__builtin_bit_cast(uint32_t, q.tscale)));
    p.empty_rows = uniform_i32(q.empty_rows);
    return p;
}

}  // namespace tg
