// Five-trit GEMV for gfx950: five ternary weights per byte as base-3 digits (digit = weight + 1,
// first weight least significant), 26 bytes per 128-weight group ("Breaking the 1.58-bit Barrier
// for Ternary LLMs", Sec. I; "Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic
// Decoding", abstract).
//
// Mapping: a lane owns one 128-weight group of a row, across the rows of a wave's tile, so its
// activation bytes are aligned once into the 26 five-byte windows the code bytes cover and reused
// for every row. A code byte selects its five int8 weights (plus three zero bytes) from a 243-entry
// table in LDS; two v_dot4_i32_i8 contract them. The group's int32 sum is exact; the fp16 scale is
// applied in fp64 and one wave reduction per row gives y.
#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTileRows = 4;

template <int M, bool ACC>
__global__ __launch_bounds__(kBlock) void t5_gemv_valu(GroupArgs ga) {
    __shared__ uint2 s_lut[256];
    if (threadIdx.x < 256) {
        uint32_t v = threadIdx.x < 243 ? threadIdx.x : 121;  // 121 = five weight-0 digits
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint32_t w = (uint32_t)((int)(v % 3) - 1) & 0xFFu;
            v /= 3;
            if (i < 4) lo |= w << (8 * i);
            else hi = w;
        }
        s_lut[threadIdx.x] = make_uint2(lo, hi);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    // wave-uniform index, so that the tile loop is not compiled as divergent
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // table mode: all waves work through the GEMVs one after the other
    const int count = ga.table ? ga.count : 1;
    for (int pi = 0; pi < count; ++pi) {
        const Problem a = uniform_problem(ga.table ? ga.table[pi] : ga.one);
        const int n = a.n, k = a.k, ng = k >> 7;
        const int ntiles = (n + kTileRows - 1) / kTileRows;
        const int nwaves = gridDim.x * kWaves;

        for (int tile = blockIdx.x * kWaves + wave; tile < ntiles; tile += nwaves) {
            const int row0 = tile * kTileRows;
            double yp[kTileRows][M];
    #pragma unroll
            for (int r = 0; r < kTileRows; ++r)
    #pragma unroll
                for (int mi = 0; mi < M; ++mi) yp[r][mi] = 0.0;

            for (int g0 = 0; g0 < ng; g0 += 64) {
                const int g = g0 + lane;
                const bool active = g < ng;
                // Activation windows: xl[b] = x bytes 5b..5b+3, xh[b] = x byte 5b+4 in the low byte
                // (bytes past weight 127 meet zero table bytes, so their values do not matter).
                uint32_t xl[M][26], xh[M][26];
    #pragma unroll
                for (int mi = 0; mi < M; ++mi) {
                    uint32_t X[33];
                    const uint4 *xp = reinterpret_cast<const uint4 *>(a.x + (size_t)mi * k + 128 * (active ? g : 0));
    #pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint4 v = xp[j];
                        X[4 * j] = v.x; X[4 * j + 1] = v.y; X[4 * j + 2] = v.z; X[4 * j + 3] = v.w;
                    }
                    X[32] = 0;
    #pragma unroll
                    for (int b = 0; b < 26; ++b) {
                        const int s0 = 5 * b, s1 = 5 * b + 4;
                        xl[mi][b] = __builtin_amdgcn_alignbyte(X[s0 / 4 + 1], X[s0 / 4], s0 % 4);
                        xh[mi][b] = __builtin_amdgcn_alignbyte(X[s1 / 4 + 1 <= 32 ? s1 / 4 + 1 : 32], X[s1 / 4], s1 % 4);
                    }
                }
    #pragma unroll
                for (int r = 0; r < kTileRows; ++r) {
                    const int row = row0 + r;
                    if (row >= n) break;
                    // 26 code bytes start at byte 26*(row*ng + g), which is 2-byte aligned: read 8 dwords
                    // from the enclosing dword and shift by 0 or 2 bytes.
                    const size_t gidx = (size_t)row * ng + (active ? g : 0);
                    const size_t byte0 = gidx * 26;
                    const uint32_t *cp = reinterpret_cast<const uint32_t *>(a.codes + (byte0 & ~(size_t)3));
                    const uint32_t sh = (uint32_t)(byte0 & 3);
                    uint32_t C[8];
    #pragma unroll
                    for (int j = 0; j < 8; ++j) C[j] = cp[j];
                    uint32_t Y[7];
    #pragma unroll
                    for (int j = 0; j < 7; ++j) Y[j] = __builtin_amdgcn_alignbyte(C[j + 1], C[j], sh);
    #pragma unroll
                    for (int mi = 0; mi < M; ++mi) {
                        int v = 0;
    #pragma unroll
                        for (int b = 0; b < 26; ++b) {
                            const uint32_t code = (Y[b / 4] >> (8 * (b % 4))) & 0xFFu;
                            const uint2 e = s_lut[code];
                            v = dot4(e.x, xl[mi][b], v);
                            v = dot4(e.y, xh[mi][b], v);
                        }
                        if (active) {
                            if (ACC) a.acc[((size_t)mi * n + row) * ng + g] = v;
                            else yp[r][mi] += (double)half_bits_to_float(a.scales[(size_t)row * ng + g]) * (double)v;
                        }
                    }
                }
            }
            if (!ACC) {
    #pragma unroll
                for (int r = 0; r < kTileRows; ++r)
    #pragma unroll
                    for (int mi = 0; mi < M; ++mi) {
                        const double t = wave_sum_f64(yp[r][mi]);
                        if (lane == 0 && row0 + r < n) a.y[(size_t)mi * n + row0 + r] = (float)t;
                    }
            }
        }

    }
}

template <int M>
hipError_t launch_m(const GroupArgs &g, bool acc_out, hipStream_t s) {
    int blocks;
    if (g.table) {
        blocks = device_cus() * 4;
    } else {
        const int ntiles = (g.one.n + kTileRows - 1) / kTileRows;
        blocks = std::max(1, std::min((ntiles + kWaves - 1) / kWaves, 4096));
    }
    if (acc_out)
        hipLaunchKernelGGL((t5_gemv_valu<M, true>), dim3(blocks), dim3(kBlock), 0, s, g);
    else
        hipLaunchKernelGGL((t5_gemv_valu<M, false>), dim3(blocks), dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_t5(const GroupArgs &g, bool acc_out, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_m<1>(g, acc_out, s);
        case 2: return launch_m<2>(g, acc_out, s);
        case 3: return launch_m<3>(g, acc_out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
