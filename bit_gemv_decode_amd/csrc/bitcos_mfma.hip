// Thin-batch BITCOS GEMV on matrix cores (gfx950): m = 4 .. 16 activation rows read the packed
// weights once.
//
// Once activations form a small matrix the GEMV is a matrix product, and the ternary weights are
// expanded into int8 operands of a matrix engine (the untitled page on a NUMA-aware decode engine for
// ternary models, Sec. 6.5 and its appendix "Ternary GEMM on AMX", where 2-bit rows are expanded into
// int8 tiles). The values follow the int8 path of "Breaking the 1.58-bit Barrier for Ternary LLMs",
// Sec. II-C: w = p - 2n by Eq. 2, int32 per-group sums times the group scale. Here the product is
// v_mfma_i32_16x16x64_i8 with
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
// Memory side. A wave owns units of T tiles (16T consecutive rows) over whole rows and walks them in
// chunks of 8 groups (1024 weights). Per chunk and row, the four lanes of the row load the row's
// bitmap bytes of the chunk (128 contiguous bytes), its 8 scales and the chunk's stretch of the sign
// stream (36 dwords from the chunk's first sign) with a few wide loads, instead of small pieces of
// 16 rows per group: the address unit sees a handful of instructions per cache line. Across lanes
// the data is then rearranged without memory traffic: a 4 x 4 transpose over the four lane rows
// (permlane16/permlane32 swaps) hands each lane its bitmap dword of every group, the scales are
// gathered the same way, and the sign stretch goes to a per-wave LDS buffer from which each lane
// reads its own three-dword window per group (its first sign follows from the row cursor plus an
// exclusive prefix of the popcounts of lanes l, l + 16, l + 32, l + 48, again by permlane swaps).
// The decode per bitmap byte is the lookup of the BITCOS tables (two LDS reads); its entries are
// already the 8 int8 weights of the B operand.
//
// fp16 activations ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-B and II-D: weights
// rebuilt as +-1 or 0 in fp16; the Xe2 kernel feeds fp16 weights and activations to its matrix
// engine): the entries come from the fp16 table (binary16 high bytes of +-1), a byte-permute widens
// each entry's 8 bytes into 8 fp16 weights, and v_mfma_f32_16x16x32_f16 takes one presence byte's
// weights (k = 32q + 8j .. + 7 for entry j) per product, four products per group, in fp32; the
// activation operand is the fp16 x at the same k.
//
// Pipeline, in half-steps h (one group step of all T tiles each): decode + products of step h - 4,
// sign windows of step h - 3, activation operand of step h - 2; chunk c's data is rearranged at the
// half-step where its first sign window is read, its bitmaps and scales were loaded six half-steps
// earlier and its sign stretch at the previous chunk's rearrangement. The loop body is one chunk
// (eight half-steps), fully unrolled, so every stage buffer has a fixed register home. Loads are
// issued unconditionally; dead ones use out-of-range offsets, which return zero without a memory
// request.
#include <algorithm>

#include "bitcos_tables.h"
#include "gemv_pipeline.h"

namespace tg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

// T: 16-row tiles per unit (kMfmaTiles, or kMfmaTilesWide from kMfmaWideM rows), mfma_waves(T) waves
// per block (one block per CU).
constexpr int kCG = 8;                   // groups per chunk
constexpr int kSW = 36;                  // staged sign-stream dwords per row and chunk
constexpr int kSWL = kSW / 4;            // ... loaded by each lane of the row
constexpr uint32_t stage_dwords(int T) { return (uint32_t)T * 16u * kSW; }  // per wave
constexpr uint32_t kXsDwords = kCG * 16;          // per wave: a chunk's activation scales, [group][m]

// (a, b) -> (a', b'): lane rows 1 and 3 of a take rows 0 and 2 of b, and rows 0 and 2 of b take rows 1
// and 3 of a (lane row = 16 consecutive lanes).
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// Lane rows 2 and 3 of a take rows 0 and 1 of b, and rows 0 and 1 of b take rows 2 and 3 of a.
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// 4 x 4 transpose between lane rows and registers: afterwards r[d] in lane row q holds what r[q] held
// in lane row d.
__device__ __forceinline__ void transpose4(uint32_t &r0, uint32_t &r1, uint32_t &r2, uint32_t &r3) {
    swap16(r0, r1);
    swap16(r2, r3);
    swap32(r0, r2);
    swap32(r1, r3);
}

// v of lane rows 0..3 (same lane within the row), returned to every lane: out[a] = v of lane row a.
__device__ __forceinline__ void gather4(uint32_t v, uint32_t (&out)[4]) {
    uint32_t e = v, o = v;
    swap16(e, o);  // e: rows (0, 0, 2, 2); o: rows (1, 1, 3, 3)
    uint32_t e2 = e, o2 = o;
    swap32(e, e2);  // e: row 0, e2: row 2
    swap32(o, o2);  // o: row 1, o2: row 3
    out[0] = e;
    out[1] = o;
    out[2] = e2;
    out[3] = o2;
}

// The weights of every tile's bitmap dword for one step, as two B operands (16 int8 each) per tile.
// sw: the sign-stream dwords and sh the funnel shift giving the stream from 3 bits before the dword's
// first sign. The per-byte (mask, base) reads of all tiles go out first, then all entry reads: two LDS
// round trips per step.
template <int T>
__device__ __forceinline__ void decode_step(const uint32_t (&bmw)[T], const uint32_t (&sw)[T][3],
                                            const uint32_t (&sh)[T], const char *lds, uint32_t laneoff,
                                            uint2 (&e)[T][4]) {
    uint2 info[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ia = __builtin_amdgcn_perm(bmw[t], laneoff, 0x0C0C0000u | ((4u + i) << 8));
            info[t][i] = *reinterpret_cast<const uint2 *>(lds + ia);
        }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint32_t lo = __builtin_amdgcn_alignbit(sw[t][1], sw[t][0], sh[t]);
        const uint32_t hi = __builtin_amdgcn_alignbit(sw[t][2], sw[t][1], sh[t]);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = i == 0 ? lo : __builtin_amdgcn_alignbit(hi, lo, c);
            e[t][i] = *reinterpret_cast<const uint2 *>(lds + ((w & info[t][i].x) | info[t][i].y));
            if (i < 3) c = __builtin_popcount(info[t][i].x) + c;
        }
    }
}

// One tile's products for one group: C[m][row] = sum over the group's 128 k of X[m][k] W[row][k]
// (int32 exact; fp32 with F16). xo: the activation operand parts of the step (two of 16 int8, or four
// of 8 fp16 per lane); e: the lane's four entries (presence bytes 0..3 of its bitmap dword).
template <bool F16>
__device__ __forceinline__ auto tile_products(const u32x4 (&xo)[F16 ? 4 : 2], const uint2 (&e)[4]) {
    if constexpr (F16) {
        f32x4 c = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // entry bytes to the high bytes of 8 binary16 weights (low bytes zero)
            const u32x4 w{__builtin_amdgcn_perm(e[j].x, e[j].x, 0x050C040Cu),
                          __builtin_amdgcn_perm(e[j].x, e[j].x, 0x070C060Cu),
                          __builtin_amdgcn_perm(e[j].y, e[j].y, 0x050C040Cu),
                          __builtin_amdgcn_perm(e[j].y, e[j].y, 0x070C060Cu)};
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, xo[j]), __builtin_bit_cast(h8v, w), c,
                                                       0, 0, 0);
        }
        return c;
    } else {
        const i32x4 b0{(int)e[0].x, (int)e[0].y, (int)e[1].x, (int)e[1].y};
        const i32x4 b1{(int)e[2].x, (int)e[2].y, (int)e[3].x, (int)e[3].y};
        i32x4 c = __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)xo[0], b0, i32x4{0, 0, 0, 0}, 0, 0, 0);
        return __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)xo[1], b1, c, 0, 0, 0);
    }
}

// Position of a chunk in the wave's stream: first row of its unit and chunk index within the rows.
struct CPos {
    int row, cu;
};

template <int T>
__device__ __forceinline__ CPos next_chunk(CPos c, int nck) {
    const bool wrap = c.cu == nck - 1;
    return CPos{wrap ? c.row + 16 * T : c.row, wrap ? 0 : c.cu + 1};
}

// With XS each group's term is also multiplied by its activation group scales xs[m][g]: lane (lr, q)
// loads xs[lr][g] of two groups of the next chunk with its other chunk loads, the values go to a per-wave
// LDS buffer [group][m] when the chunk's data is rearranged, and each step's sign-window stage reads
// the four scales of its rows m = 4q .. 4q + 3 with one 16-byte LDS read.
template <int kT, bool ACC, bool XS, bool F16>
__device__ __forceinline__ void run_mfma(const Problem &p, int u0, int u1, int mrows, const char *lds,
                                         uint32_t *stg) {
    constexpr uint32_t kStageDwords = stage_dwords(kT);
    static_assert(!(F16 && (ACC || XS)), "fp16 activations: fp32 outputs only");
    constexpr uint32_t EB = F16 ? 2u : 1u;  // activation element bytes
    constexpr int NP = F16 ? 4 : 2;         // activation operand parts (16 bytes each) per group
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;  // weight row within a tile; activation row of the A operand
    const int q = lane >> 4;   // quarter of the group
    const int ng = p.ng;
    const int nck = (ng + kCG - 1) / kCG;
    const uint32_t kb = (uint32_t)(p.k >> 3);  // bitmap bytes per row
    const __amdgpu_buffer_rsrc_t rbm = make_rsrc(p.codes, p.codes_bytes);
    // Sign stretches: the resource starts 4 bytes early (a window may start up to 3 bits before the
    // stream) and runs to the end of the row index, which follows the sign section in the packed
    // buffer, so a stretch that starts inside the stream is read whole.
    const uint32_t sg_bytes = (uint32_t)(reinterpret_cast<const uint8_t *>(p.rowoff) -
                                         reinterpret_cast<const uint8_t *>(p.signs)) +
                              (uint32_t)(p.n + 1) * 4u + 4u;
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc(reinterpret_cast<const uint8_t *>(p.signs) - 4, sg_bytes);
    const __amdgpu_buffer_rsrc_t rro = make_rsrc(p.rowoff, (uint32_t)(p.n + 1) * 4u);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(p.scales, ACC ? 0u : (uint32_t)p.n * (uint32_t)ng * 2u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)mrows * (uint32_t)p.k * EB);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y, ACC ? 0u : (uint32_t)mrows * (uint32_t)p.n * 4u);
    const __amdgpu_buffer_rsrc_t racc =
        make_rsrc(p.acc, ACC ? (uint32_t)mrows * (uint32_t)p.n * (uint32_t)ng * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.xs, XS ? (uint32_t)mrows * (uint32_t)ng * 4u : 0u);
    uint32_t *const sxs = stg + kStageDwords;  // XS: the chunk's activation scales, [group][m]
    if constexpr (XS) {
        // The pipeline-fill steps read this buffer before the first chunk is written to it; their
        // products are zero, but a stale Inf or NaN bit pattern left in LDS by an earlier kernel would
        // still turn 0 * xs into NaN in the row sums. Zero it first (in-order within the wave).
#pragma unroll
        for (int i = 0; i < (int)kXsDwords / 64; ++i) sxs[64 * i + lane] = 0u;
    }
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    const uint32_t m_odd = (q & 1) ? ~0u : 0u, m_hi = (q >> 1) ? ~0u : 0u;
    const uint32_t voff_x = lr < mrows ? ((uint32_t)lr * (uint32_t)p.k + 32u * (uint32_t)q) * EB : kOffOff;
    // this lane's row slot in the staging buffer, per tile
    uint32_t *stg_row[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) stg_row[t] = stg + (t * 16 + lr) * kSW;

    const int NC = (u1 - u0) * nck;  // chunks of the range
    const CPos c0{(u0 - p.unit_begin) * 16 * kT, 0};

    // chunk stage buffers
    uint32_t rawb[kT][8] = {};      // bitmap bytes of the next chunk as loaded: groups 2q, 2q + 1
    uint32_t raws[kT][2] = {};      // scales of the next chunk as loaded: groups 2q, 2q + 1
    uint32_t rawsg[kT][kSWL] = {};  // sign stretch of the next chunk, quarter q
    uint32_t ro_cur[kT] = {}, ro_nxt[kT] = {};  // row index entries of chunks ci + 1 and ci + 2
    uint32_t bmc[kT][kCG] = {};     // current chunk: the lane's bitmap dword of each group
    uint32_t scc[kT][4] = {};       // current chunk: scales of groups 2a, 2a + 1 (low, high half)
    uint32_t d0c[kT] = {}, d0n[kT] = {};  // first staged dword (resource dword index) of chunks ci, ci + 1
    uint32_t cbn[kT] = {};          // sign cursor at the start of chunk ci + 1 (row-uniform)
    uint32_t cur[kT] = {};          // running sign cursor of the sign-window stage
    // step stage buffers
    uint32_t bms[2][kT] = {}, sws[2][kT][3] = {}, shs[2][kT] = {}, scs[2][kT] = {};
    uint32_t rawx[2] = {};          // XS: xs[lr][g] of groups 2q, 2q + 1 of the next chunk as loaded
    u32x4 xss[2] = {};              // XS: step stage, xs[4q + i][g] of the step's group
    u32x4 xo[4][NP] = {};            // activation operand of the step, by step slot
    double facc[kT][4];
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) facc[t][i] = 0.0;

    // Chunk loads: bitmaps and scales of chunk c into rawb / raws (groups past the row end read zero).
    auto load_chunk = [&](CPos c, bool live) {
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const uint32_t rowb = (uint32_t)(c.row + 16 * t + lr);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int g = c.cu * kCG + 2 * q + e;
                const bool ok = live && g < ng;
                const u32x4 v = ld4(rbm, ok ? rowb * kb + (uint32_t)g * 16u : kOffOff, 0u);
                rawb[t][4 * e] = v.x;
                rawb[t][4 * e + 1] = v.y;
                rawb[t][4 * e + 2] = v.z;
                rawb[t][4 * e + 3] = v.w;
                if constexpr (!ACC)
                    raws[t][e] = ldh(rsc, ok ? (rowb * (uint32_t)ng + (uint32_t)g) * 2u : kOffOff, 0u);
            }
        }
        if constexpr (XS) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int g = c.cu * kCG + 2 * q + e;
                const bool ok = live && g < ng && lr < mrows;
                rawx[e] = ld1(rxs, ok ? ((uint32_t)lr * (uint32_t)ng + (uint32_t)g) * 4u : kOffOff, 0u);
            }
        }
    };
    // Row index entries of chunk c when it starts a unit (else zero) into ro_nxt.
    auto load_ro = [&](CPos c, bool live) {
        const uint32_t soff = live_or_dead(live && c.cu == 0, (uint32_t)c.row * 4u);
#pragma unroll
        for (int t = 0; t < kT; ++t) ro_nxt[t] = ld1(rro, (uint32_t)(16 * t + lr) * 4u, soff);
    };
    // Sign stretches of the chunk whose first sign is cbn: quarter q of the kSW dwords from the dword
    // holding the bit 3 before it.
    auto load_signs = [&](bool live) {
        const uint32_t sd = live_or_dead(live, 0u);
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            d0n[t] = (cbn[t] + 29u) >> 5;  // the resource starts one dword early: +32 - 3
            const uint32_t vo = (d0n[t] + (uint32_t)(kSWL * q)) * 4u;
            const u32x4 a = ld4(rsg, vo, sd);
            const u32x4 b = ld4(rsg, vo + 16u, sd);
            rawsg[t][0] = a.x;
            rawsg[t][1] = a.y;
            rawsg[t][2] = a.z;
            rawsg[t][3] = a.w;
            rawsg[t][4] = b.x;
            rawsg[t][5] = b.y;
            rawsg[t][6] = b.z;
            rawsg[t][7] = b.w;
            rawsg[t][8] = ld1(rsg, vo + 32u, sd);
        }
    };

    // ---- prologue: chunk 0's data, the row index of chunk 1 ----
    {
        const bool live0 = NC > 0;
        load_ro(c0, live0);
#pragma unroll
        for (int t = 0; t < kT; ++t) cbn[t] = ro_nxt[t];  // waits for the row index of chunk 0
        load_signs(live0);
        load_chunk(c0, live0);
        load_ro(next_chunk<kT>(c0, nck), NC > 1);
#pragma unroll
        for (int t = 0; t < kT; ++t) ro_cur[t] = ro_nxt[t];
    }

    CPos prev = c0, cp = c0;  // chunks ci - 1 and ci (prev is dead at ci = 0)
    for (int ci = 0; ci <= NC; ++ci) {
        const CPos nx = next_chunk<kT>(cp, nck), nn = next_chunk<kT>(nx, nck);
        const bool live_prev = ci >= 1, live_cur = ci < NC;
#pragma unroll
        for (int j = 0; j < kCG; ++j) {
            // ---- decode and products of step h - 4: chunk (j < 4 ? prev : cur), position (j - 4) & 7 ----
            {
                const int pos = (j - 4) & 7;
                const CPos c = j < 4 ? prev : cp;
                const bool live = j < 4 ? live_prev : live_cur;
                const int sl = j & 1;  // slot of step h - 4
                uint2 e[kT][4];
                decode_step<kT>(bms[sl], sws[sl], shs[sl], lds, laneoff, e);
                decltype(tile_products<F16>(xo[0], e[0])) cc[kT];
#pragma unroll
                for (int t = 0; t < kT; ++t) cc[t] = tile_products<F16>(xo[j & 3], e[t]);
                const int g = c.cu * kCG + pos;
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    const auto cv = cc[t];
                    const int row = c.row + 16 * t + lr;
                    if constexpr (ACC) {
                        // acc[m][row][g]: the unit's first row and the group go in the scalar offset
                        const uint32_t soff =
                            live_or_dead(live && g < ng, ((uint32_t)c.row * (uint32_t)ng + (uint32_t)g) * 4u);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int m = 4 * q + i;
                            st1((uint32_t)cv[i], racc,
                                m < mrows && row < p.n
                                    ? ((uint32_t)(m * p.n) + (uint32_t)(16 * t + lr)) * (uint32_t)ng * 4u
                                    : kOffOff,
                                soff);
                        }
                    } else {
                        const double sd = (double)half_bits_to_float((uint16_t)scs[sl][t]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // scale times activation scale is exact in fp64 (11 + 24 significant bits),
                            // and so is its product with the int32 sum inside the fma
                            // (the element goes through a scalar first: a bit cast of a vector element
                            // expression reinterprets the vector's first element)
                            const uint32_t xv = xss[sl][i];
                            const double f = XS ? sd * (double)__builtin_bit_cast(float, xv) : sd;
                            facc[t][i] = __builtin_fma((double)cv[i], f, facc[t][i]);
                        }
                    }
                }
                if constexpr (!ACC) {
                    if (pos == kCG - 1) {               // static: the chunk's last step
                        if (live && c.cu == nck - 1) {  // the unit's rows are complete
#pragma unroll
                            for (int t = 0; t < kT; ++t) {
                                const int row = c.row + 16 * t + lr;
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
                }
            }
            TG_SCHED_FENCE();
            // ---- activation operand of step h - 2: chunk (j < 2 ? prev : cur), position (j - 2) & 7 ----
            {
                const int pos = (j - 2) & 7;
                const CPos c = j < 2 ? prev : cp;
                const bool live = j < 2 ? live_prev : live_cur;
                const uint32_t soff = live_or_dead(live, (uint32_t)(c.cu * kCG + pos) * 128u * EB);
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) xo[(j + 2) & 3][pp] = ld4(rx, voff_x + 16u * pp, soff);
            }
            TG_SCHED_FENCE();
            if (j == 3) {
                // ---- chunk ci's data to its stage homes; chunk ci + 1's sign stretches ----
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    // bitmap: lane row a loaded groups 2a, 2a + 1; lane row q wants dword q of each group
                    transpose4(rawb[t][0], rawb[t][1], rawb[t][2], rawb[t][3]);
                    transpose4(rawb[t][4], rawb[t][5], rawb[t][6], rawb[t][7]);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        bmc[t][2 * a] = rawb[t][a];
                        bmc[t][2 * a + 1] = rawb[t][4 + a];
                    }
                    if constexpr (!ACC) gather4(raws[t][0] | (raws[t][1] << 16), scc[t]);
                    // the sign stretch to this wave's LDS rows
#pragma unroll
                    for (int i = 0; i < kSWL; ++i) stg_row[t][kSWL * q + i] = rawsg[t][i];
                    d0c[t] = d0n[t];
                    cur[t] = cbn[t];
                    // row total of the chunk's signs, and the next chunk's first sign
                    uint32_t cnt = 0;
#pragma unroll
                    for (int g = 0; g < kCG; ++g) cnt = __builtin_popcount(bmc[t][g]) + cnt;
                    uint32_t ce = cnt, co = cnt;
                    swap16(ce, co);
                    uint32_t pr = ce + co, pr2 = pr;
                    swap32(pr, pr2);
                    cbn[t] = nx.cu == 0 ? ro_cur[t] : cbn[t] + pr + pr2;
                }
                if constexpr (XS) {
                    // chunk ci's activation scales to the wave's LDS buffer: group 2q + e, row lr
#pragma unroll
                    for (int e = 0; e < 2; ++e) sxs[(2 * q + e) * 16 + lr] = rawx[e];
                }
                load_ro(nn, ci + 2 < NC);
                load_signs(ci + 1 < NC);
            }
            TG_SCHED_FENCE();
            if (j == 5) load_chunk(nx, ci + 1 < NC);
            TG_SCHED_FENCE();
            // ---- sign windows of step h - 3: chunk (j < 3 ? prev : cur), position (j - 3) & 7 ----
            {
                const int pos = (j - 3) & 7;
                const int sl = (j + 1) & 1;  // slot of step h - 3
#pragma unroll
                for (int t = 0; t < kT; ++t) {
                    const uint32_t bw = bmc[t][pos];
                    const uint32_t c = __builtin_popcount(bw);
                    uint32_t ev = c, od = c;
                    swap16(ev, od);  // quarters (0, 0, 2, 2) and (1, 1, 3, 3)
                    uint32_t pr = ev + od, pr2 = pr;
                    swap32(pr, pr2);  // c0 + c1 and c2 + c3
                    const uint32_t pq = cur[t] + (ev & m_odd) + (pr & m_hi);
                    cur[t] += pr + pr2;
                    const uint32_t b = pq + 29u;  // window from 3 bits before the first sign, +32 bias
                    const uint32_t *src = stg_row[t] + ((b >> 5) - d0c[t]);
                    sws[sl][t][0] = src[0];
                    sws[sl][t][1] = src[1];
                    sws[sl][t][2] = src[2];
                    shs[sl][t] = b;
                    bms[sl][t] = bw;
                    scs[sl][t] = (scc[t][pos >> 1] >> (16 * (pos & 1))) & 0xFFFFu;
                }
                if constexpr (XS) {
                    // read as the uint32_t words they were written as (one 16-byte LDS read)
                    const uint32_t *src = sxs + pos * 16 + 4 * q;
                    xss[sl] = u32x4{src[0], src[1], src[2], src[3]};
                }
            }
            TG_SCHED_FENCE();
        }
        if (ci + 1 <= NC) {
#pragma unroll
            for (int t = 0; t < kT; ++t) ro_cur[t] = ro_nxt[t];
        }
        prev = cp;
        cp = nx;
    }
}

template <int T, bool ACC, bool XS, bool F16 = false>
__global__ __launch_bounds__(64 * mfma_waves(T)) void bitcos_mfma_kernel(GroupArgs ga) {
    constexpr int kWaves = mfma_waves(T), kBlock = 64 * kWaves;
    constexpr uint32_t kWaveDwords = stage_dwords(T) + (XS ? kXsDwords : 0u);
    __shared__ uint4 s_tab[kTabBytes / 16];
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[kWaves * kWaveDwords];
    // The table fill goes out first (straight into LDS); the wave's unit range and its first GEMV
    // descriptor (two dependent scalar round trips) are read while it is in flight.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    load_bitcos_tables<kBlock, F16>(s_tab);
    TG_SCHED_FENCE();
    int u, u_end, pi;
    wave_range<kWaves>(ga, wave, u, u_end, pi);
    const bool bad0 = ga.table && pi >= ga.count;
    const Problem p0 = uniform_problem(launch_problem(ga, bad0 ? 0 : pi));
    lds_copies_landed();
    __syncthreads();
    const char *lds = reinterpret_cast<const char *>(s_tab);
    uint32_t *stg = s_stage + wave * kWaveDwords;
    bool first = true;
    while (u < u_end) {
        if (ga.table && pi >= ga.count) break;  // ranges inconsistent with the table: stop
        const Problem p = first ? p0 : uniform_problem(launch_problem(ga, pi));
        first = false;
        const int u1 = min(u_end, p.unit_begin + p.nunits);
        if (u < u1) run_mfma<T, ACC, XS, F16>(p, u, u1, ga.m, lds, stg);
        u = max(u, u1);
        ++pi;
    }
}

}  // namespace

void mfma_geometry(Problem &p, int tiles) {
    p.ng = p.k / 128;
    p.nch = 1;
    p.G = p.ng;
    p.R = 1;
    p.glast = p.ng;
    p.nbu = tiles;
    p.rpu = 16 * tiles;
    p.gmagic = 0;
    p.rmagic = 0;
    p.nunits = (p.n + p.rpu - 1) / p.rpu;
}

namespace {
template <int T>
hipError_t launch_mfma_t(const GroupArgs &g, int out, hipStream_t s) {
    constexpr int W = mfma_waves(T);
    const int blocks = grid_blocks<W>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    if (out == kOutAcc)
        hipLaunchKernelGGL((bitcos_mfma_kernel<T, true, false>), dim3(blocks), dim3(64 * W), 0, s, g);
    else if (out == kOutYxs)
        hipLaunchKernelGGL((bitcos_mfma_kernel<T, false, true>), dim3(blocks), dim3(64 * W), 0, s, g);
    else
        hipLaunchKernelGGL((bitcos_mfma_kernel<T, false, false>), dim3(blocks), dim3(64 * W), 0, s, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_bitcos_mfma(const GroupArgs &g, int out, hipStream_t s) {
    if (g.m < kMfmaMinM || g.m > TG_MAX_M) return hipErrorInvalidValue;
    return mfma_tiles(g.m, false) == kMfmaTilesWide ? launch_mfma_t<kMfmaTilesWide>(g, out, s)
                                                     : launch_mfma_t<kMfmaTiles>(g, out, s);
}

hipError_t launch_bitcos_mfma_f16(const GroupArgs &g, hipStream_t s) {
    if (g.m < 1 || g.m > TG_MAX_M) return hipErrorInvalidValue;
    constexpr int W = mfma_waves(kMfmaTiles);
    const int blocks = grid_blocks<W>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bitcos_mfma_kernel<kMfmaTiles, false, false, true>), dim3(blocks), dim3(64 * W), 0, s, g);
    return hipGetLastError();
}

}  // namespace tg
