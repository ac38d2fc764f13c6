// Device pieces shared by the persistent GEMV kernels (BITCOS, five-trit, 2-bit): launch geometry
// per activation-row count, branch-free buffer access with dead offsets, per-GEMV context, the
// activation slice of a lane, and the unit-end row reduction through an LDS tile.
//
// Work geometry (all formats): a lane owns one 128-weight group of one row per step. A row of k
// weights takes ng = k/128 lanes; when ng <= 64 a step holds R = 64/ng consecutive rows (at most 16),
// otherwise the row is split into chunks of 64 groups. A unit is NB steps (single chunk) or NB rows
// taken chunk pass by chunk pass. Each group's int32 sum times its fp16 scale (exact in fp64) goes to
// a per-wave LDS tile, whose rows are summed once per unit (fp64, DPP) and stored as fp32.
#pragma once

#include <algorithm>

#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

template <int M, int FMT>
struct Cfg {
    // row bundles (steps per chunk pass) per unit: 2 for BITCOS at m = 3 (its 118 KB of tables leave
    // no room for a larger tile), else 4. The fixed-code formats' 4-row units at m = 3 were measured
    // against 2-row ones (96 copies, identical outputs): chunked 4096x14336 +64-67 % (the activation
    // slices are reloaded once per pass for twice the rows), five-trit single-chunk shapes +9-11 %,
    // 2-bit single-chunk shapes within 1 %.
    static constexpr int NB = FMT == TG_FMT_BITCOS && M == 3 ? 2 : 4;
    static constexpr int WAVES = gemv_waves(FMT, M);  // waves per block (= per CU)
    static constexpr int BLOCK = 64 * WAVES;
};

// Scheduling fence: the compiler may not move instructions across it. Keeps the loads of the
// pipeline stages in program order, so that each wait covers exactly the loads it needs.
#define TG_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Wait until this wave's copies from global memory into LDS (global_load_lds) have landed: they count
// as vector memory loads. The block barrier that follows makes every wave's copies visible.
__device__ __forceinline__ void lds_copies_landed() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Buffer offsets. A lane with nothing to read gets kOffOff as its own (vector) offset; a pipeline
// stage with nothing to do gets kDeadS as its wave-uniform (scalar) offset. Either way the sum lies
// beyond every resource (bitmaps, scales and outputs are limited to less than 1 GiB, sign windows to
// less than 512 MiB) without wrapping, so the access returns zero and makes no memory request.
constexpr uint32_t kOffOff = 0x80000000u;
constexpr uint32_t kDeadS = 0x7FFFFFF0u;

// live ? v : kDeadS without a branch (the compiler turns a select over a product into a branch).
__device__ __forceinline__ uint32_t live_or_dead(bool live, uint32_t v) {
    const uint32_t m = 0u - (uint32_t)live;
    return (v & m) | (kDeadS & ~m);
}

__device__ __forceinline__ u32x4 ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t ldh(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
// Streamed loads with the non-temporal cache policy, for data each byte of which is read once by one
// instruction: the BITCOS vector kernel's bitmaps and weight scales, which then leave the caches to
// the data that is reused (activation slices, sign windows, row index). Measured on MI355X, layer set,
// alternating builds with identical outputs: +1.7 % with the bitmaps marked, +1.8-2.7 % with the
// bitmaps and scales. Marking the sign windows too (neighbouring lanes and steps re-read them) was
// slower, and so were the five-trit code loads (-2.7 %; their 26-byte groups straddle lines that the
// neighbouring lane's load also reads) and the thin-batch kernel's bitmap loads (-5 to -17 %); 2-bit
// codes were unchanged. Those keep the default policy.
constexpr int kStreamPolicy = 2;  // cache-policy operand of the buffer-load builtins: nt
__device__ __forceinline__ u32x4 ld4s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy);
}
__device__ __forceinline__ uint16_t ldhs(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStreamPolicy);
}
__device__ __forceinline__ void st1(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}

// Wave-uniform per-GEMV values.
struct Ctx {
    __amdgpu_buffer_rsrc_t rbm, rsg, rsc, rro, rx, ry, racc, rxs;
    int n, k, ng, nch, G, R, glast;
};

// Activation slice of the lane's group for every activation row: XW dwords per row, 32 for int8
// activations (128 bytes), 64 for fp16 ones (256 bytes); lanes without a group read nothing.
template <int M, int XW = 32>
__device__ __forceinline__ void load_x(const Ctx &x, uint32_t voff, uint32_t (&xr)[M][XW]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
#pragma unroll
        for (int j = 0; j < XW / 4; ++j) {
            const u32x4 v = ld4(x.rx, voff + 16u * j, (uint32_t)(mi * x.k * (XW / 32)));
            xr[mi][4 * j] = v.x;
            xr[mi][4 * j + 1] = v.y;
            xr[mi][4 * j + 2] = v.z;
            xr[mi][4 * j + 3] = v.w;
        }
}

// x must have arrived before a loop starts: a loop entered with x as the newest loads would get
// the waits compiled for that entry on every iteration.
template <int M, int XW = 32>
__device__ __forceinline__ void wait_x(const uint32_t (&xr)[M][XW]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
#pragma unroll
        for (int j = 0; j < XW; j += 4) asm volatile("" ::"v"(xr[mi][j]));
}

// Activation group scale of the lane's group (the group whose x bytes load_x reads at voff, i.e. group
// voff / 128 of each activation row) for every activation row, when the GEMV has them (XS); lanes
// without a group (voff = kOffOff, which stays out of range after the shift) read zero. Without
// activation scales every factor is 1.
template <int M, bool XS>
__device__ __forceinline__ void load_xs(const Ctx &x, uint32_t voff, float (&xsv)[M]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
        xsv[mi] = XS ? __builtin_bit_cast(float, ld1(x.rxs, voff >> 5, (uint32_t)(mi * x.ng) * 4u)) : 1.0f;
}

template <int M, bool XS>
__device__ __forceinline__ void wait_xs(const float (&xsv)[M]) {
    if constexpr (XS) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) asm volatile("" ::"v"(xsv[mi]));
    }
}

// Lane roles in the unit-end reduction: the tile's rows are summed by lpr lanes each.
struct Red {
    int lpr;   // lanes per row (power of two)
    int epl;   // tile terms per lane
    int base;  // tile index of the lane's first term
    int cnt;   // terms the lane sums (0 .. epl)
    int rho;   // tile row of the lane
    bool own;  // the lane ends up holding row rho's sum (last lane of its group, rho < rows)
};

__device__ __forceinline__ Red make_red(int rows, int R, int geff, uint32_t rmagic) {
    const int lane = threadIdx.x & 63;
    Red r;
    int lg = 0;
    while ((2 << lg) * rows <= 64) ++lg;  // largest power of two with lpr * rows <= 64
    r.lpr = 1 << lg;
    r.epl = (geff + r.lpr - 1) >> lg;
    r.rho = lane >> lg;
    const int pi = lane & (r.lpr - 1);
    const int sb = (int)(((uint32_t)r.rho * rmagic) >> 16);  // step of the row
    const int qb = r.rho - sb * R;
    r.base = sb * 64 + qb * geff + pi * r.epl;
    r.cnt = min(max(geff - pi * r.epl, 0), r.epl);
    if (r.rho >= rows) r.cnt = 0;
    r.own = r.rho < rows && pi == r.lpr - 1;
    return r;
}

// Row sums of a finished tile, stored as fp32: tile row rho is output row row0 + rho (stored when
// below row_end and `live`).
template <int M, int NB>
__device__ __forceinline__ void reduce_store(const Ctx &x, const Red &r, const double *tile, int row0, int row_end,
                                             bool live) {
    double yv[M];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
        double t = 0.0;
        for (int e = 0; e < r.epl; ++e)
            if (e < r.cnt) t += tile[mi * NB * 64 + r.base + e];
        yv[mi] = seg_sum_f64(t, r.lpr);
    }
    __builtin_amdgcn_wave_barrier();
    const int row = row0 + r.rho;
    const bool own = live && r.own && row < row_end;
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
        st1(__builtin_bit_cast(uint32_t, (float)yv[mi]), x.ry, own ? (uint32_t)row * 4u : kOffOff,
            (uint32_t)(mi * x.n) * 4u);
}

// Decode stage epilogue: the group terms (int32 sum times the group's weight scale s, times the
// activation group scale when XS; fp64, every product exact) go to tile slot `slot` (added to what earlier chunks left there
// when `add`); accumulator outputs are stored directly.
template <int M, bool ACC, int NB, bool XS, typename A>
__device__ __forceinline__ void emit(const Ctx &x, const A (&acc)[M], double s, const float (&xsv)[M],
                                     double *tile, int slot, bool add, uint32_t voff_acc, uint32_t soff_acc) {
    const int lane = threadIdx.x & 63;
    if constexpr (ACC) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
            st1((uint32_t)acc[mi], x.racc, voff_acc, soff_acc + (uint32_t)(mi * x.n * x.ng) * 4u);
    } else {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            double *t = tile + mi * NB * 64 + slot * 64 + lane;
            double term = (double)acc[mi] * s;
            if constexpr (XS) term *= (double)xsv[mi];
            *t = add ? *t + term : term;
        }
    }
}

// The wave's unit range [u, u_end) and its first GEMV. With a per-wave range table (grouped launch)
// the host fixed it; for one GEMV the units are dealt in equal shares across blocks first, so that a
// small GEMV still spreads over the CUs. Blocks are dealt to the XCDs round-robin; virtual block
// numbers put consecutive ranges on one XCD (its L2 then sees neighbouring rows).
template <int WAVES>
__device__ __forceinline__ void wave_range(const GroupArgs &ga, int wave, int &u, int &u_end, int &pi) {
    const int nblk = gridDim.x;
    const int vblk = (nblk % 8 == 0) ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
    if (ga.ranges) {
        // through the constant address space: scalar loads, which do not wait for vector memory
        // operations in flight (e.g. the table fill)
        typedef const __attribute__((address_space(4))) int32_t *ConstWords;
        const int vw = vblk * WAVES + wave;
        static_assert(sizeof(WaveRange) == 16, "four words per range");
        const ConstWords r = (ConstWords)ga.ranges + 4 * vw;
        u = uniform_i32(r[0]);
        u_end = uniform_i32(r[1]);
        pi = uniform_i32(r[2]);
    } else {
        const int nw = nblk * WAVES;
        const int vw = wave * nblk + vblk;
        const int share = (ga.units + nw - 1) / nw;
        u = min(vw * share, ga.units);
        u_end = min(u + share, ga.units);
        pi = 0;
    }
}

// Blocks of a launch: the range table fixes them; otherwise at most one per CU (the decode tables
// take most of the LDS), a multiple of 8 so that every XCD gets the same number. 0: invalid.
template <int WAVES>
inline int grid_blocks(const GroupArgs &g) {
    if (g.ranges) return g.waves % WAVES ? 0 : g.waves / WAVES;
    int blocks = std::min(g.units, device_cus());
    if (blocks > 8) blocks = blocks / 8 * 8;
    return std::max(1, blocks);
}

}  // namespace
}  // namespace tg
