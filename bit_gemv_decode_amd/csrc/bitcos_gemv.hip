// BITCOS unpack-fused GEMV for gfx950 (int8 activations, ternary weights, fp16 group scales).
//
// Format ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-A, Fig. 2): a presence bitmap
// with one bit per weight and a compacted sign stream with one bit per non-zero weight; the j-th sign
// bit belongs to the j-th set bit of the bitmap. Decoding places the compact signs back onto the
// present positions (the deposit of Fig. 4); the int8 path of Sec. II-C turns each (present,
// negative) pair into w = p - 2n (Eq. 2), contracts against int8 activations in int32 and applies
// the group scale once per 128-element group.
//
// Mapping on CDNA4 (wave64):
//   * a wave owns a tile of rows; each lane owns one 32-bit bitmap word (32 consecutive k) of the
//     current 2048-wide k chunk, so bitmap loads are 256-byte coalesced rows;
//   * a lane finds where its word's signs start with a wave-wide exclusive prefix sum of the word
//     popcounts (DPP row shifts and row broadcasts), offset by the row's entry in the sign index;
//   * the lane reads the two sign dwords that hold its (at most 32) signs and aligns them with one
//     funnel shift (the 2-word span bound: start bit <= 31 plus <= 32 signs ends inside the second
//     dword);
//   * the Fig. 4 deposit is replaced by a table in LDS: for each byte of presence bits pb and the
//     popcount(pb) compact signs that follow, the table holds the 8 ternary int8 weights. It is
//     indexed compactly, base[pb] + signs, 3^8 = 6561 entries of 8 bytes;
//   * v_dot4_i32_i8 contracts 4 weights per instruction against the lane's activation bytes, which
//     stay in registers for all rows of the tile;
//   * the 4 lanes of a 128-group sum their partials with two DPP quad swaps; the first lane applies
//     the fp16 scale in fp64, and one wave reduction per row gives y (rounded once to fp32).
#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kByteLutEntries = 6561;  // sum over the 256 presence bytes of 2^popcount = 3^8

struct alignas(16) ByteLut {
    uint64_t ent[kByteLutEntries + 1];  // padded to an even count for 16-byte copies
    uint16_t base[256];
};

constexpr ByteLut make_byte_lut() {
    ByteLut t{};
    uint32_t e = 0;
    for (uint32_t pb = 0; pb < 256; ++pb) {
        t.base[pb] = (uint16_t)e;
        uint32_t c = 0;
        for (uint32_t i = 0; i < 8; ++i) c += (pb >> i) & 1;
        for (uint32_t sc = 0; sc < (1u << c); ++sc) {
            uint64_t v = 0;
            uint32_t rank = 0;
            for (uint32_t i = 0; i < 8; ++i) {
                if ((pb >> i) & 1) {
                    uint64_t byte = ((sc >> rank) & 1) ? 0xFFull : 0x01ull;  // -1 or +1 as int8
                    v |= byte << (8 * i);
                    ++rank;
                }
            }
            t.ent[e++] = v;
        }
    }
    return t;
}

__device__ const ByteLut kByteLut = make_byte_lut();

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTileRows = 4;

template <int M, bool ACC>
__global__ __launch_bounds__(kBlock) void bitcos_gemv_valu(GemvArgs a) {
    __shared__ uint4 s_ent4[(kByteLutEntries + 1) / 2];
    __shared__ uint16_t s_base[256];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(kByteLut.ent);
        for (int i = threadIdx.x; i < (kByteLutEntries + 1) / 2; i += kBlock) s_ent4[i] = src[i];
        s_base[threadIdx.x] = kByteLut.base[threadIdx.x];
    }
    __syncthreads();
    const uint2 *s_ent = reinterpret_cast<const uint2 *>(s_ent4);

    const int lane = threadIdx.x & 63;
    const int n = a.n, k = a.k;
    const int kw = k >> 5;  // 32-bit bitmap words per row
    const int ng = k >> 7;
    const uint32_t *bm = reinterpret_cast<const uint32_t *>(a.codes);
    const uint32_t last_sign = a.sign_dwords - 1;
    const int ntiles = (n + kTileRows - 1) / kTileRows;
    const int nwaves = gridDim.x * kWaves;

    for (int tile = blockIdx.x * kWaves + (threadIdx.x >> 6); tile < ntiles; tile += nwaves) {
        const int row0 = tile * kTileRows;
        uint32_t rowpos[kTileRows];
        double yp[kTileRows][M];
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) {
            rowpos[r] = row0 + r < n ? a.rowoff[row0 + r] : 0u;
#pragma unroll
            for (int mi = 0; mi < M; ++mi) yp[r][mi] = 0.0;
        }
        for (int c0 = 0; c0 < kw; c0 += 64) {
            const int wi = c0 + lane;
            const bool active = wi < kw;
            const int g = wi >> 2;
            uint32_t xd[M][8];
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
                if (active) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(a.x + (size_t)mi * k + 32 * wi);
                    lo = xp[0];
                    hi = xp[1];
                }
                xd[mi][0] = lo.x; xd[mi][1] = lo.y; xd[mi][2] = lo.z; xd[mi][3] = lo.w;
                xd[mi][4] = hi.x; xd[mi][5] = hi.y; xd[mi][6] = hi.z; xd[mi][7] = hi.w;
            }
#pragma unroll
            for (int r = 0; r < kTileRows; ++r) {
                const int row = row0 + r;
                if (row >= n) break;
                const uint32_t p = active ? bm[(size_t)row * kw + wi] : 0u;
                const uint32_t pc = __builtin_popcount(p);
                const uint32_t incl = wave_incl_scan(pc);
                const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                const uint32_t o = rowpos[r] + incl - pc;
                rowpos[r] += total;
                const uint32_t q = o >> 5;
                const uint32_t d0 = a.signs[min(q, last_sign)];
                const uint32_t d1 = a.signs[min(q + 1, last_sign)];
                const uint32_t s = __builtin_amdgcn_alignbit(d1, d0, o & 31);
                uint32_t wd[8];
                uint32_t cur = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t pb = (p >> (8 * t)) & 0xFFu;
                    const uint32_t c = __builtin_popcount(pb);
                    const uint32_t sc = __builtin_amdgcn_ubfe(s, cur, c);
                    cur += c;
                    const uint2 e = s_ent[s_base[pb] + sc];
                    wd[2 * t] = e.x;
                    wd[2 * t + 1] = e.y;
                }
#pragma unroll
                for (int mi = 0; mi < M; ++mi) {
                    int v = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) v = dot4(wd[i], xd[mi][i], v);
                    v = quad_sum(v);
                    if (active && (lane & 3) == 0) {
                        if (ACC) {
                            a.acc[((size_t)mi * n + row) * ng + g] = v;
                        } else {
                            yp[r][mi] += (double)half_bits_to_float(a.scales[(size_t)row * ng + g]) * (double)v;
                        }
                    }
                }
            }
        }
        if (!ACC) {
#pragma unroll
            for (int r = 0; r < kTileRows; ++r) {
#pragma unroll
                for (int mi = 0; mi < M; ++mi) {
                    const double t = wave_sum_f64(yp[r][mi]);
                    if (lane == 0 && row0 + r < n) a.y[(size_t)mi * n + row0 + r] = (float)t;
                }
            }
        }
    }
}

int max_blocks() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        cached = cus * 3;  // the 53 KB decode table limits residency to 3 blocks per CU
    }
    return cached;
}

template <int M>
hipError_t launch_m(const GemvArgs &a, bool acc_out, hipStream_t s) {
    const int ntiles = (a.n + kTileRows - 1) / kTileRows;
    const int blocks = std::max(1, std::min((ntiles + kWaves - 1) / kWaves, max_blocks()));
    if (acc_out)
        hipLaunchKernelGGL((bitcos_gemv_valu<M, true>), dim3(blocks), dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((bitcos_gemv_valu<M, false>), dim3(blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bitcos(const GemvArgs &args, bool acc_out, hipStream_t s) {
    // Activation rows are processed four at a time; each launch re-reads the weights.
    for (int m0 = 0; m0 < args.m; m0 += 4) {
        GemvArgs a = args;
        const int mt = std::min(4, args.m - m0);
        a.m = mt;
        a.x = args.x + (size_t)m0 * args.k;
        if (acc_out) a.acc = args.acc + (size_t)m0 * args.n * (args.k / TG_GROUP);
        else a.y = args.y + (size_t)m0 * args.n;
        hipError_t e;
        switch (mt) {
            case 1: e = launch_m<1>(a, acc_out, s); break;
            case 2: e = launch_m<2>(a, acc_out, s); break;
            case 3: e = launch_m<3>(a, acc_out, s); break;
            default: e = launch_m<4>(a, acc_out, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tg
