// Streaming-read reference kernel: the achievable HBM read bandwidth on this GPU, against which the
// GEMV kernels' effective bandwidth is compared (the pages compare each GEMV with the platform's
// measured stream-read rate, "Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. III-B2 and
// III-C). Each lane keeps UNROLL 16-byte loads in flight, waves stride over the buffer, and the
// XOR of everything read is folded into one word per wave so that no load can be dropped.
#include <algorithm>

#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t *buf, uint32_t bytes, uint32_t *sink) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint32_t nwaves = gridDim.x * 4;
    constexpr uint32_t kStep = 64 * 16 * UNROLL;  // bytes one wave reads per iteration
    uint32_t acc = 0;
    for (uint32_t off = wave * kStep; off < bytes; off += nwaves * kStep) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = buf_u32x4(r, off + (uint32_t)u * 1024u + lane * 16u);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one store per wave keeps the loads alive
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0) sink[wave] = acc;
}

// One wave samples the shader-clock counter (s_memtime, which counts at the shader clock) and the
// constant 100 MHz counter (s_memrealtime) at its start, spins until `spin` ticks of the constant
// counter have passed, and samples both again: slot i of out gets the four values. Launched between
// other launches on a stream, consecutive probes bracket them (their duration, from the constant
// counter) and each probe gives the shader clock of its moment ((memtime delta) / (realtime delta) x
// 100 MHz).
__global__ void clock_probe_kernel(uint64_t *out, uint32_t slot, uint32_t spin) {
    if (threadIdx.x == 0) {
        const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
        const uint64_t c0 = __builtin_amdgcn_s_memtime();
        uint64_t r1 = r0, c1 = c0;
        while (r1 - r0 < spin) {
            r1 = __builtin_amdgcn_s_memrealtime();
            c1 = __builtin_amdgcn_s_memtime();
        }
        out[4 * (uint64_t)slot] = r0;
        out[4 * (uint64_t)slot + 1] = c0;
        out[4 * (uint64_t)slot + 2] = r1;
        out[4 * (uint64_t)slot + 3] = c1;
    }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, uint32_t slot, uint32_t spin, hipStream_t s) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, out, slot, spin);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *buf, uint32_t bytes, uint32_t *sink, int blocks, int unroll, hipStream_t s) {
    const uint8_t *b = (const uint8_t *)buf;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, b, bytes, sink); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, s, b, bytes, sink); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, b, bytes, sink); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, b, bytes, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tg
