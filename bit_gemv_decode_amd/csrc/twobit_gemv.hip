// 2-bit GEMV for gfx950: code = weight + 1 in two bits, four codes per byte, first weight in the
// low bits (Table I's 2-bit packing in "Breaking the 1.58-bit Barrier for Ternary LLMs"; the
// expansion is a shift, a mask and a subtraction).
//
// Mapping: as for BITCOS, a lane owns 32 consecutive weights (8 code bytes) of each row of a wave's
// tile. For a code dword (16 weights) the four masks (d >> 2i) & 0x03030303 each hold one code per
// byte -- weights i, i+4, i+8, i+12 -- so the lane's activation bytes are transposed 4x4 once per
// k chunk (v_perm) and reused for all rows. v_dot4 accumulates sum(code * x); subtracting the
// group's sum(x), computed once per chunk and shared by every row, gives sum(w * x) exactly.
#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTileRows = 4;

// (A,B,C,D) -> four dwords; dword i holds byte i of A, B, C, D.
__device__ __forceinline__ void transpose4x4(uint32_t A, uint32_t B, uint32_t C, uint32_t D, uint32_t *o) {
    const uint32_t ab_lo = __builtin_amdgcn_perm(B, A, 0x05010400u);
    const uint32_t ab_hi = __builtin_amdgcn_perm(B, A, 0x07030602u);
    const uint32_t cd_lo = __builtin_amdgcn_perm(D, C, 0x05010400u);
    const uint32_t cd_hi = __builtin_amdgcn_perm(D, C, 0x07030602u);
    o[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

template <int M, bool ACC>
__global__ __launch_bounds__(kBlock) void b2_gemv_valu(GroupArgs ga) {
    const int lane = threadIdx.x & 63;
    // wave-uniform index, so that the tile loop is not compiled as divergent
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // table mode: all waves work through the GEMVs one after the other
    const int count = ga.table ? ga.count : 1;
    for (int pi = 0; pi < count; ++pi) {
        const Problem a = uniform_problem(ga.table ? ga.table[pi] : ga.one);
        const int n = a.n, k = a.k, ng = k >> 7, kw = k >> 5;
        const int ntiles = (n + kTileRows - 1) / kTileRows;
        const int nwaves = gridDim.x * kWaves;
        const uint2 *codes = reinterpret_cast<const uint2 *>(a.codes);

        for (int tile = blockIdx.x * kWaves + wave; tile < ntiles; tile += nwaves) {
            const int row0 = tile * kTileRows;
            double yp[kTileRows][M];
    #pragma unroll
            for (int r = 0; r < kTileRows; ++r)
    #pragma unroll
                for (int mi = 0; mi < M; ++mi) yp[r][mi] = 0.0;

            for (int c0 = 0; c0 < kw; c0 += 64) {
                const int wi = c0 + lane;
                const bool active = wi < kw;
                const int g = wi >> 2;
                uint32_t xt[M][8];
                int sx[M];
    #pragma unroll
                for (int mi = 0; mi < M; ++mi) {
                    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
                    if (active) {
                        const uint4 *xp = reinterpret_cast<const uint4 *>(a.x + (size_t)mi * k + 32 * wi);
                        lo = xp[0];
                        hi = xp[1];
                    }
                    transpose4x4(lo.x, lo.y, lo.z, lo.w, &xt[mi][0]);
                    transpose4x4(hi.x, hi.y, hi.z, hi.w, &xt[mi][4]);
                    int s = 0;
                    s = dot4(lo.x, 0x01010101u, s); s = dot4(lo.y, 0x01010101u, s);
                    s = dot4(lo.z, 0x01010101u, s); s = dot4(lo.w, 0x01010101u, s);
                    s = dot4(hi.x, 0x01010101u, s); s = dot4(hi.y, 0x01010101u, s);
                    s = dot4(hi.z, 0x01010101u, s); s = dot4(hi.w, 0x01010101u, s);
                    sx[mi] = quad_sum(s);
                }
    #pragma unroll
                for (int r = 0; r < kTileRows; ++r) {
                    const int row = row0 + r;
                    if (row >= n) break;
                    const uint2 cw = active ? codes[(size_t)row * kw + wi] : make_uint2(0x55555555u, 0x55555555u);
    #pragma unroll
                    for (int mi = 0; mi < M; ++mi) {
                        int v = 0;
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v = dot4((cw.x >> (2 * i)) & 0x03030303u, xt[mi][i], v);
                            v = dot4((cw.y >> (2 * i)) & 0x03030303u, xt[mi][4 + i], v);
                        }
                        v = quad_sum(v) - sx[mi];
                        if (active && (lane & 3) == 0) {
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
        hipLaunchKernelGGL((b2_gemv_valu<M, true>), dim3(blocks), dim3(kBlock), 0, s, g);
    else
        hipLaunchKernelGGL((b2_gemv_valu<M, false>), dim3(blocks), dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_b2(const GroupArgs &g, bool acc_out, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_m<1>(g, acc_out, s);
        case 2: return launch_m<2>(g, acc_out, s);
        case 3: return launch_m<3>(g, acc_out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
