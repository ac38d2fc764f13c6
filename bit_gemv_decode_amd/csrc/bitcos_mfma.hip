// Thin-batch BITCOS GEMV on matrix cores (gfx950): m = 4 .. 16 activation rows read the packed
// weights once.
//
// Once activations form a small matrix, decoding turns the ternary weights into int8 operands of a
// matrix product ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. III: batched decoding is a
// matrix product; the int8 path of Sec. II-C: w = p - 2n by Eq. 2, int32 per-group sums times the
// group scale). Here the product is v_mfma_i32_16x16x64_i8 with
//   A = X[m][k]  (16 activation rows, rows at and beyond m read as zero),
//   B = W^T      (16 weight rows of one tile, decoded in registers),
// so C[m][row] comes out per 128-weight group in int32 and takes that group's fp16 scale in fp64.
//
// Lane roles follow the operand layout: lane l serves weight row (l % 16) of a tile and quarter
// q = l / 16 of each group, i.e. bitmap dword q (weights 32q .. 32q + 31); the first product covers
// the first 16 of them, the second the other 16, and lane l's activation operand is row l % 16 of X
// at the same k positions (the k order inside an operand is the same for A and B, so the products
// sum over exactly the group's 128 k). The result lane l holds is C[4q + i][l % 16], i = 0..3.
//
// A wave takes units of T consecutive 16-row tiles and walks their groups in order, so each row's
// sign cursor runs on from group to group (starting at the row index entry). Inside a group the four
// lanes of a row find their first sign with an exclusive prefix sum of their dwords' popcounts over
// lanes l, l + 16, l + 32, l + 48 (two permlane swaps, no LDS). The decode per bitmap byte is the
// lookup of the BITCOS tables (two LDS reads), whose entries are already the 8 int8 weights of the
// B operand. The activation operand is loaded once per group and shared by the T tiles.
//
// Loads are software-pipelined like the vector kernels: the bitmap of step h, the signs,
// activations and scales of step h - 2 and the decode of step h - 4 share one half-step, in a loop
// body of four half-steps with fixed register homes, every load issued unconditionally (dead steps
// use out-of-range offsets, which return zero without a memory request).
#include <algorithm>

#include "bitcos_tables.h"
#include "gemv_pipeline.h"

namespace tg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kMfmaWavesPerCu;  // waves per block (one block per CU)
constexpr int kBlock = 64 * kWaves;
constexpr int kT = kMfmaTiles;           // 16-row tiles per unit
constexpr int kLagS = 2;                 // half-steps between a bitmap load and its sign stage

__device__ __forceinline__ u32x3 ld3(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
}

#ifndef TG_MFMA_PHASE_FENCE
#define TG_MFMA_PHASE_FENCE() TG_SCHED_FENCE()
#endif

// The weights of every tile's bitmap dword for one step, as two B operands (16 int8 each) per tile.
// sg/sh: the sign-stream dwords and funnel shift giving the stream from 3 bits before the dword's
// first sign. The per-byte (mask, base) reads of all tiles go out first, then all entry reads: two
// LDS round trips per step.
template <int T>
__device__ __forceinline__ void decode_step(const uint32_t (&bmw)[T], const u32x3 (&sg)[T], const uint32_t (&sh)[T],
                                            const char *lds, uint32_t laneoff, i32x4 (&b0)[T], i32x4 (&b1)[T]) {
    uint2 info[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ia = __builtin_amdgcn_perm(bmw[t], laneoff, 0x0C0C0000u | ((4u + i) << 8));
            info[t][i] = *reinterpret_cast<const uint2 *>(lds + ia);
        }
    TG_MFMA_PHASE_FENCE();
    uint2 e[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint32_t lo = __builtin_amdgcn_alignbit(sg[t].y, sg[t].x, sh[t]);
        const uint32_t hi = __builtin_amdgcn_alignbit(sg[t].z, sg[t].y, sh[t]);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = i == 0 ? lo : __builtin_amdgcn_alignbit(hi, lo, c);
            e[t][i] = *reinterpret_cast<const uint2 *>(lds + ((w & info[t][i].x) | info[t][i].y));
            if (i < 3) c = __builtin_popcount(info[t][i].x) + c;
        }
    }
    TG_MFMA_PHASE_FENCE();
#pragma unroll
    for (int t = 0; t < T; ++t) {
        b0[t] = i32x4{(int)e[t][0].x, (int)e[t][0].y, (int)e[t][1].x, (int)e[t][1].y};
        b1[t] = i32x4{(int)e[t][2].x, (int)e[t][2].y, (int)e[t][3].x, (int)e[t][3].y};
    }
}

template <bool ACC>
__device__ __forceinline__ void run_mfma(const Problem &p, int u0, int u1, int mrows, const char *lds) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;  // weight row within a tile; activation row of the A operand
    const int q = lane >> 4;   // quarter of the group
    const int ng = p.ng;
    const uint32_t kb = (uint32_t)(p.k >> 3);  // bitmap bytes per row
    const __amdgpu_buffer_rsrc_t rbm = make_rsrc(p.codes, p.codes_bytes);
    // the sign resource starts 4 bytes early so that a window starting below bit 3 is in range
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc(reinterpret_cast<const uint8_t *>(p.signs) - 4, p.sign_bytes + 4u);
    const __amdgpu_buffer_rsrc_t rro = make_rsrc(p.rowoff, (uint32_t)(p.n + 1) * 4u);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(p.scales, ACC ? 0u : (uint32_t)p.n * (uint32_t)ng * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)mrows * (uint32_t)p.k);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y, ACC ? 0u : (uint32_t)mrows * (uint32_t)p.n * 4u);
    const __amdgpu_buffer_rsrc_t racc =
        make_rsrc(p.acc, ACC ? (uint32_t)mrows * (uint32_t)p.n * (uint32_t)ng * 4u : 0u);
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    const uint32_t m_odd = (q & 1) ? ~0u : 0u, m_hi = (q >> 1) ? ~0u : 0u;
    const uint32_t voff_x = lr < mrows ? (uint32_t)lr * (uint32_t)p.k + 32u * (uint32_t)q : kOffOff;

    const int S = (u1 - u0) * ng;  // steps: (unit, group) in order
    const int row_first = (u0 - p.unit_begin) * 16 * kT;

    uint32_t bm[4][kT] = {}, ro[4][kT] = {}, sh[4][kT] = {}, sc[4][kT] = {}, cur[kT];
    u32x3 sg[4][kT] = {};
    u32x4 xa[4] = {}, xb[4] = {};
    double facc[kT][4];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        cur[t] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) facc[t][i] = 0.0;
    }
    // stage positions: first row of the unit and group of the step each stage handles
    int rB = row_first, gB = 0, rS = row_first, gS = 0, rD = row_first, gD = 0;

    for (int it = 0; 4 * it - 4 < S; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * it + j;
            // ---- decode step h - 4 (slot j) ----
            {
                const int s = h - 4;
                const bool live = s >= 0 && s < S;
                i32x4 b0[kT], b1[kT], cc[kT];
                decode_step<kT>(bm[j], sg[j], sh[j], lds, laneoff, b0, b1);
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    cc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)xa[j], b0[t], i32x4{0, 0, 0, 0}, 0, 0, 0);
                    cc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)xb[j], b1[t], cc[t], 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    const i32x4 c = cc[t];
                    const int row = rD + 16 * t + lr;
                    if constexpr (ACC) {
                        // acc[m][row][g]: the unit's first row and the group go in the scalar offset
                        const uint32_t soff = live_or_dead(live, ((uint32_t)rD * (uint32_t)ng + (uint32_t)gD) * 4u);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int m = 4 * q + i;
                            st1((uint32_t)c[i], racc,
                                m < mrows && row < p.n
                                    ? ((uint32_t)(m * p.n) + (uint32_t)(16 * t + lr)) * (uint32_t)ng * 4u
                                    : kOffOff,
                                soff);
                        }
                    } else {
                        const double sd = (double)half_bits_to_float((uint16_t)sc[j][t]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) facc[t][i] = __builtin_fma((double)c[i], sd, facc[t][i]);
                    }
                }
                if constexpr (!ACC) {
                    if (live && gD == ng - 1) {  // the unit's rows are complete
#pragma unroll
                        for (int t = 0; t < kT; ++t) {
                            const int row = rD + 16 * t + lr;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int m = 4 * q + i;
                                st1(__builtin_bit_cast(uint32_t, (float)facc[t][i]), ry,
                                    m < mrows && row < p.n ? (uint32_t)(m * p.n + row) * 4u : kOffOff, 0u);
                                facc[t][i] = 0.0;
                            }
                        }
                    }
                }
                const bool wrap = gD == ng - 1;
                rD = live && wrap ? rD + 16 * kT : rD;
                gD = live ? (wrap ? 0 : gD + 1) : gD;
            }
            TG_SCHED_FENCE();
            // ---- bitmap of step h (slot j) and, at a unit's first group, its rows' index entries ----
            {
                const bool live = h < S;
                const uint32_t soff = live_or_dead(live, (uint32_t)rB * kb + (uint32_t)gB * 16u);
                const uint32_t soff_ro = live_or_dead(live && gB == 0, (uint32_t)rB * 4u);
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    bm[j][t] = ld1(rbm, (uint32_t)(16 * t + lr) * kb + 4u * (uint32_t)q, soff);
                    ro[j][t] = ld1(rro, (uint32_t)(16 * t + lr) * 4u, soff_ro);
                }
                const bool wrap = gB == ng - 1;
                rB = live && wrap ? rB + 16 * kT : rB;
                gB = live ? (wrap ? 0 : gB + 1) : gB;
            }
            TG_SCHED_FENCE();
            // ---- signs, activations and scales of step h - kLagS (slot (j - kLagS) & 3) ----
            {
                const int s = h - kLagS;
                const int k3 = (j + 4 - kLagS) & 3;
                const bool live = s >= 0 && s < S;
                const uint32_t sd = live_or_dead(live, 0u);
                const bool first = gS == 0;
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    const uint32_t c = __builtin_popcount(bm[k3][t]);
                    // lanes of one row: quarters 0..3 at l, l + 16, l + 32, l + 48
                    const auto ev = __builtin_amdgcn_permlane16_swap(c, c, false, false);  // quarters (0,0,2,2), (1,1,3,3)
                    const uint32_t pair = ev[0] + ev[1];                                     // c0 + c1 or c2 + c3
                    const auto hv = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);  // c0 + c1, c2 + c3
                    const uint32_t base = first ? ro[k3][t] : cur[t];
                    const uint32_t pos = base + (ev[0] & m_odd) + (hv[0] & m_hi);
                    cur[t] = base + hv[0] + hv[1];
                    // window from 3 bits before the first sign, biased by +32 (resource starts 4 bytes early)
                    const uint32_t b = pos + 29u;
                    sg[k3][t] = ld3(rsg, (b >> 5) << 2, sd);
                    sh[k3][t] = b;
                }
                const uint32_t soff_x = live_or_dead(live, (uint32_t)gS * 128u);
                xa[k3] = ld4(rx, voff_x, soff_x);
                xb[k3] = ld4(rx, voff_x + 16u, soff_x);
                if constexpr (!ACC) {
                    const uint32_t soff_sc = live_or_dead(live, ((uint32_t)rS * (uint32_t)ng + (uint32_t)gS) * 2u);
#pragma unroll
                    for (int t = 0; t < kT; ++t)
                        sc[k3][t] = ldh(rsc, (uint32_t)(16 * t + lr) * (uint32_t)ng * 2u, soff_sc);
                }
                const bool wrap = gS == ng - 1;
                rS = live && wrap ? rS + 16 * kT : rS;
                gS = live ? (wrap ? 0 : gS + 1) : gS;
            }
            TG_SCHED_FENCE();
        }
    }
}

template <bool ACC>
__global__ __launch_bounds__(kBlock) void bitcos_mfma_kernel(GroupArgs ga) {
    __shared__ uint4 s_tab[kTabBytes / 16];
    load_bitcos_tables<kBlock>(s_tab);
    __syncthreads();
    const char *lds = reinterpret_cast<const char *>(s_tab);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int u, u_end, pi;
    wave_range<kWaves>(ga, wave, u, u_end, pi);
    while (u < u_end) {
        if (ga.table && pi >= ga.count) break;  // ranges inconsistent with the table: stop
        const Problem p = uniform_problem(ga.table ? ga.table[pi] : ga.one);
        const int u1 = min(u_end, p.unit_begin + p.nunits);
        if (u < u1) run_mfma<ACC>(p, u, u1, ga.m, lds);
        u = max(u, u1);
        ++pi;
    }
}

}  // namespace

void mfma_geometry(Problem &p) {
    p.ng = p.k / 128;
    p.nch = 1;
    p.G = p.ng;
    p.R = 1;
    p.glast = p.ng;
    p.nbu = kT;
    p.rpu = 16 * kT;
    p.gmagic = 0;
    p.rmagic = 0;
    p.nunits = (p.n + p.rpu - 1) / p.rpu;
}

hipError_t launch_bitcos_mfma(const GroupArgs &g, bool acc_out, hipStream_t s) {
    if (g.m < kMfmaMinM || g.m > TG_MAX_M) return hipErrorInvalidValue;
    const int blocks = grid_blocks<kWaves>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    if (acc_out)
        hipLaunchKernelGGL((bitcos_mfma_kernel<true>), dim3(blocks), dim3(kBlock), 0, s, g);
    else
        hipLaunchKernelGGL((bitcos_mfma_kernel<false>), dim3(blocks), dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

}  // namespace tg
