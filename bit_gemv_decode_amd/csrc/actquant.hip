// Per-group int8 quantisation of fp32 activations (gfx950).
//
// "Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C (the int8 path after Fig. 5): the
// activations are quantised to int8 per group of 128 before the integer dot products, and each
// group's scale is applied once per group, beside the weight scale. The quantiser itself is not
// spelled out there; this is the symmetric absmax form: per group of 128 consecutive activations of
// one row, sigma = max |x| / 127 and code = x / sigma rounded to nearest-even, clamped to
// [-127, 127]; an all-zero group has sigma = 0 and codes 0. Both divisions are IEEE single-precision
// operations, so every code is decided in fp32.
//
// One wave per group: lane l holds activations 2l and 2l + 1 (one 8-byte load), the group maximum
// comes from a butterfly over the wave, and each lane writes its two codes with one 2-byte store.
#include "device_common.h"

namespace tg {
namespace {

constexpr int kQuantWaves = 4;  // waves (groups) per block

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ int quant_code(float v, float sigma) {
    // __fdiv_rn: IEEE division rounded to nearest-even; rintf: nearest-even
    const float r = rintf(__fdiv_rn(v, sigma));
    return r > 127.0f ? 127 : r < -127.0f ? -127 : (int)r;
}

__global__ __launch_bounds__(64 * kQuantWaves) void quantize_x_kernel(const float *__restrict__ x, int64_t groups,
                                                                      int8_t *__restrict__ xq, float *__restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
    if (g >= groups) return;  // uniform across the wave
    const float2 v = *reinterpret_cast<const float2 *>(x + g * 128 + 2 * lane);
    const float a = wave_max_f32(fmaxf(fabsf(v.x), fabsf(v.y)));
    const float sigma = __fdiv_rn(a, 127.0f);
    int c0 = 0, c1 = 0;
    if (a > 0.0f) {
        c0 = quant_code(v.x, sigma);
        c1 = quant_code(v.y, sigma);
    }
    *reinterpret_cast<uint16_t *>(xq + g * 128 + 2 * lane) = (uint16_t)((c0 & 0xFF) | ((c1 & 0xFF) << 8));
    if (lane == 0) xs[g] = sigma;
}

}  // namespace

hipError_t launch_quantize_x(const float *x, int64_t groups, int8_t *xq, float *xs, hipStream_t s) {
    const int64_t blocks = (groups + kQuantWaves - 1) / kQuantWaves;
    if (groups < 1 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_x_kernel, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0, s, x, groups, xq, xs);
    return hipGetLastError();
}

}  // namespace tg
