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
//   * one persistent grid serves one GEMV or a whole table of them; the work unit is a block of NB
//     consecutive rows of one matrix, taken by one wave. Units are dealt so that consecutive units
//     run on the same XCD (its L2 then sees whole sign-stream lines and shares x).
//   * within a unit the wave walks k chunk by chunk. A full chunk is 4096 weights, one row per step,
//     lane l owning bitmap dwords 2l, 2l+1 of the chunk (64 weights, half a 128-group). When k is
//     not a multiple of 4096, the remainder of several rows is packed into one step.
//   * the activation bytes a lane needs for its 64 weights stay in registers for every row of the
//     unit, so x is read once per unit rather than once per row;
//   * a lane's first sign sits at the row's running cursor plus the exclusive prefix sum of the
//     popcounts of the lanes before it (DPP row shifts and broadcasts; the sign stream is one
//     contiguous bit string over all rows, so rows of one step simply continue each other);
//   * the lane fetches the <= 64 signs of its two dwords with one 3-dword load and funnel-shifts
//     them into place (start <= bit 31 of the first dword, <= 64 bits: inside three dwords);
//   * the Fig. 4 deposit is replaced by a table in LDS: for each presence byte pb and the
//     popcount(pb) compact signs that follow, the table holds the 8 ternary int8 weights; it is
//     indexed compactly, base[pb] + signs, 3^8 = 6561 entries of 8 bytes, loaded once per block;
//   * v_dot4_i32_i8 contracts 4 weights per instruction; the two lanes of a 128-group add their
//     int32 partials with one DPP swap and the even lane applies the fp16 scale in fp64. The group
//     terms of all NB rows go through LDS and are summed by 64/NB lanes per row, so the fp64
//     cross-lane reduction runs once per batch, not once per row;
//   * a unit is one fully unrolled batch per chunk: all NB bitmap loads are issued first, then each
//     row's scan and sign-window load, then the decodes, so NB rows of loads are in flight per wave
//     and the compiler waits for exactly the load each step needs. All loads go through buffer
//     resources: out-of-range reads return zero (a corrupt sign index cannot fault).
#include <algorithm>

#include "device_common.h"
#include "tg_internal.h"

namespace tg {
namespace {

constexpr int kByteLutEntries = 6561;  // sum over the 256 presence bytes of 2^popcount = 3^8

struct alignas(16) ByteLut {
    uint64_t ent[kByteLutEntries + 1];  // padded to an even count for 16-byte copies
    uint32_t base8[256];                // byte offset (8 * entry index) of presence byte pb's first entry
};

constexpr ByteLut make_byte_lut() {
    ByteLut t{};
    uint32_t e = 0;
    for (uint32_t pb = 0; pb < 256; ++pb) {
        t.base8[pb] = 8 * e;
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

constexpr int kWaves = kBitcosWavesPerBlock;
constexpr int kBlock = 64 * kWaves;
constexpr int kChunkDwords = 128;  // bitmap dwords of one full chunk (64 lanes x 2)

// Scheduling fence: the compiler may not move instructions across it. Keeps the phases of a batch
// (loads, scans, decodes) and of a decode (base reads, entry reads, dot products) apart, so that
// the loads and LDS reads of one phase are all in flight together.
#define TG_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

struct LutView {
    const char *ent;    // LDS byte address of the entry table
    const char *base8;  // LDS byte address of the base table (u32 per presence byte)
};

// Buffer resources over the sections one GEMV reads.
struct Rsrc {
    __amdgpu_buffer_rsrc_t bm, sg, sc, x;
};

// Out-of-range buffer offset: a load there returns zero and makes no memory request.
constexpr uint32_t kNoLoad = 0xFFFFFFF0u;

// One lane's share of a step after its bitmap dwords arrived: sign window and scale loads issued.
struct Staged {
    uint2 bm;
    u32x3 sg;        // sign dwords q, q+1, q+2 of the stream
    uint32_t r0;     // bit of sg.x where the lane's first sign sits
    uint16_t scale;  // fp16 scale bits of the lane's group (value path)
};

// Sign window for a lane whose first sign is at stream position o0 (the window covers o0 .. o0+95,
// enough for the <= 64 signs of two bitmap dwords), and the scale of its group.
template <bool ACC>
__device__ __forceinline__ Staged issue_signs(const Rsrc &r, uint2 bm, bool act, uint32_t o0, uint32_t scale_idx) {
    Staged st;
    st.bm = bm;
    st.r0 = o0 & 31;
    st.sg = buf_u32x3(r.sg, act ? (o0 >> 5) * 4 : kNoLoad);
    // unconditional for every lane (a branch around a load makes the compiler wait for every load in
    // flight); inactive lanes read nothing
    st.scale = ACC ? (uint16_t)0 : buf_u16(r.sc, act ? scale_idx * 2 : kNoLoad);
    return st;
}

// Decode a staged lane share: the int32 sum of the lane's 64 weights times x, per m.
// Phase 1 needs only the bitmap: presence bytes (pre-scaled by 4 to address the base table),
// popcounts, in-window sign cursors and the eight base-table reads. Phase 2 aligns the sign windows
// and reads the eight table entries. Phase 3 contracts them with the activations.
template <int M>
__device__ __forceinline__ void decode_staged(const Staged &st, const LutView &lut, const uint32_t (&xr)[M][16],
                                              int (&acc)[M]) {
    uint32_t c[8], cur[8], base[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t p = i < 4 ? st.bm.x : st.bm.y;
        const uint32_t pb4 = ((p >> (8 * (i & 3))) & 0xFFu) << 2;
        c[i] = __builtin_popcount(pb4);
        cur[i] = (i & 3) == 0 ? 0u : cur[i - 1] + c[i - 1];
        base[i] = *reinterpret_cast<const uint32_t *>(lut.base8 + pb4);
    }
    TG_SCHED_FENCE();
    const uint32_t pc0 = cur[3] + c[3];  // signs of the first dword
    const uint32_t w0 = __builtin_amdgcn_alignbit(st.sg.y, st.sg.x, st.r0);
    const uint32_t r1 = st.r0 + pc0;  // 0 .. 63
    const bool hi = r1 & 32;
    const uint32_t w1 = __builtin_amdgcn_alignbit(hi ? st.sg.z : st.sg.y, hi ? st.sg.y : st.sg.x, r1 & 31);
    uint2 e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t sc = __builtin_amdgcn_ubfe(i < 4 ? w0 : w1, cur[i], c[i]);
        e[i] = *reinterpret_cast<const uint2 *>(lut.ent + base[i] + 8 * sc);
    }
    TG_SCHED_FENCE();
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
        int v = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v = dot4(e[i].x, xr[mi][2 * i], v);
            v = dot4(e[i].y, xr[mi][2 * i + 1], v);
        }
        acc[mi] = v;
    }
}

// Geometry of one chunk of k (wave-uniform). A full chunk is 4096 weights: one row per step, 64
// lanes of 2 bitmap dwords. The tail chunk (k % 4096) gives each row L = tail/2 lanes and, when L
// is a power of two, packs 64/L rows into a step; otherwise one row per step. Lane l sits in step
// row l >> lg, at segment position l & (2^lg - 1); for a non-power-of-two tail lg = 6 (one
// segment) and lanes at or past L are idle. All derived by shifts, without branches.
struct Geo {
    int dw_base;  // first bitmap dword of the chunk within a row
    int L;        // lanes per row
    int lg;       // log2 of the segment width
    int rps;      // rows per step (1 << (6 - lg))
    int G;        // 128-groups per row in the chunk (L / 2)
    bool full;    // L == 64
};

__device__ __forceinline__ int nchunks_of(const Problem &p) {
    const int kd = p.k >> 5;
    return kd / kChunkDwords + ((kd % kChunkDwords) ? 1 : 0);
}

__device__ __forceinline__ Geo geo_of(const Problem &p, int c) {
    const int kd = p.k >> 5;
    const int nfull = kd / kChunkDwords;
    Geo g;
    g.full = c < nfull;
    g.dw_base = (g.full ? c : nfull) * kChunkDwords;
    g.L = g.full ? 64 : (kd - g.dw_base) >> 1;
    const bool pow2 = (g.L & (g.L - 1)) == 0;
    g.lg = pow2 ? 31 - __builtin_clz((unsigned)g.L) : 6;
    g.rps = 1 << (6 - g.lg);
    g.G = g.L >> 1;
    return g;
}

// Steps of a batch of nrows unit rows: ceil(nrows / rps).
__device__ __forceinline__ int nsteps_of(const Geo &g, int nrows) {
    return (nrows + g.rps - 1) >> (6 - g.lg);
}

// Per-lane view of a chunk geometry.
struct LaneGeo {
    int ri;   // row of the lane within a step
    int seg;  // lane index within its row segment
    bool ok;  // lane belongs to a row segment
    int dw0;  // lane's first bitmap dword within the row
};

__device__ __forceinline__ LaneGeo lane_geo(const Geo &g, int lane) {
    LaneGeo l;
    l.ri = lane >> g.lg;
    l.seg = lane & ((1 << g.lg) - 1);
    l.ok = l.seg < g.L;
    l.dw0 = g.dw_base + 2 * l.seg;
    return l;
}

// Everything a batch needs before its scans: bitmap dwords of each step, the activation bytes of
// the lane's 64 weights, and (for a unit's first chunk) the unit rows' sign cursors.
template <int M, int NB>
struct Batch {
    uint32_t xr[M][16];
    uint2 b[NB];
    uint32_t rowoff;
};

// `live` false: issue the same instructions with out-of-range offsets (no memory traffic), so that
// the caller needs no branch around the loads.
template <int M, int NB>
__device__ __forceinline__ void issue_batch(const Problem &p, int u, int c, bool live, Batch<M, NB> &bt) {
    const int lane = threadIdx.x & 63;
    const int kd = p.k >> 5;
    const int row0 = (u - p.unit_begin) * NB;
    const int nrows = min(NB, p.n - row0);
    const Geo g = geo_of(p, c);
    const LaneGeo l = lane_geo(g, lane);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)M * (uint32_t)p.k);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.codes, p.codes_bytes);
    // x first: a later wait for x then never has to wait for the (HBM) bitmap loads
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = buf_u32x4(rx, (live && l.ok) ? (uint32_t)(mi * p.k + 32 * l.dw0 + 16 * j) : kNoLoad);
            bt.xr[mi][4 * j] = v.x;
            bt.xr[mi][4 * j + 1] = v.y;
            bt.xr[mi][4 * j + 2] = v.z;
            bt.xr[mi][4 * j + 3] = v.w;
        }
#pragma unroll
    for (int st = 0; st < NB; ++st) {
        const int ur = st * g.rps + l.ri;
        const bool act = live && l.ok && ur < nrows;
        const u32x2 v = buf_u32x2(rb, act ? (uint32_t)((row0 + ur) * kd + l.dw0) * 4 : kNoLoad);
        bt.b[st] = make_uint2(v.x, v.y);
    }
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(p.rowoff, (uint32_t)(p.n + 1) * 4u);
    bt.rowoff = buf_u32(ri, (live && c == 0 && lane < nrows) ? (uint32_t)(row0 + lane) * 4 : kNoLoad);
}

// Scan each step's lane popcounts, advance the unit rows' cursors (lane u tracks unit row u) and
// issue the sign-window and scale loads.
template <int M, bool ACC, int NB>
__device__ __forceinline__ void stage_batch(const Problem &p, int u, int c, const Batch<M, NB> &bt, uint32_t &cur_v,
                                            Staged (&S)[NB]) {
    const int lane = threadIdx.x & 63;
    const int ng = p.k >> 7;
    const int row0 = (u - p.unit_begin) * NB;
    const int nrows = min(NB, p.n - row0);
    const Geo g = geo_of(p, c);
    const LaneGeo l = lane_geo(g, lane);
    const int gcol = l.dw0 >> 2;
    Rsrc r;
    r.sg = make_rsrc(p.signs, p.sign_bytes);
    r.sc = make_rsrc(p.scales, ACC ? 0u : (uint32_t)p.n * (uint32_t)ng * 2u);
    if (c == 0) cur_v = bt.rowoff;
    const int nsteps = nsteps_of(g, nrows);
#pragma unroll
    for (int st = 0; st < NB; ++st) {
        if (st >= nsteps) break;  // wave-uniform: no row of the unit left for this step
        const uint2 b = bt.b[st];
        const uint32_t pc = __builtin_popcount(b.x) + __builtin_popcount(b.y);
        const uint32_t incl = wave_incl_scan(pc);
        const int ur = st * g.rps + l.ri;
        const bool act = l.ok && ur < nrows;
        uint32_t o0;
        if (g.full) {
            const uint32_t rowcur = (uint32_t)__builtin_amdgcn_readlane((int)cur_v, st);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            cur_v += lane == st ? total : 0u;
            o0 = rowcur + incl - pc;
        } else {
            // inclusive sums just before this lane's row segment and at its end (the shuffles run
            // on every lane: a lane-permute reading from a lane that is switched off returns zero)
            const int seg_first = l.ri << g.lg;
            const uint32_t prev = (uint32_t)__shfl((int)incl, max(seg_first - 1, 0), 64);
            const uint32_t before = seg_first > 0 ? prev : 0u;
            const uint32_t end = (uint32_t)__shfl((int)incl, min(seg_first + g.L - 1, 63), 64);
            const uint32_t rowcur = (uint32_t)__shfl((int)cur_v, min(ur, 63), 64);
            // unit row v = st*rps + i takes the total of step row i (held by lane i*L)
            const int i = lane - st * g.rps;
            const bool mine = i >= 0 && i < g.rps;
            const uint32_t t = (uint32_t)__shfl((int)(end - before), mine ? i * g.L : 0, 64);
            cur_v += mine ? t : 0u;
            o0 = rowcur + incl - pc - before;
        }
        S[st] = issue_signs<ACC>(r, b, act, o0, (uint32_t)((row0 + ur) * ng + gcol));
    }
}

// Decode every step of a batch. Accumulator path: store each group's int32 sum. Value path: the
// group sums and scale bits go to the wave's LDS scratch; the batch's rows are then summed by 64/NB
// lanes each (scale * acc in fp64) and added to the row sums held by lane u for unit row u.
template <int M, bool ACC, int NB>
__device__ __forceinline__ void finish_batch(const Problem &p, int u, int c, const Staged (&S)[NB],
                                             const uint32_t (&xr)[M][16], const LutView &lut, int32_t *red_acc,
                                             uint16_t *red_sc, double (&yv)[M]) {
    const int lane = threadIdx.x & 63;
    const int ng = p.k >> 7;
    const int row0 = (u - p.unit_begin) * NB;
    const int nrows = min(NB, p.n - row0);
    const Geo g = geo_of(p, c);
    const LaneGeo l = lane_geo(g, lane);
    const int gi = l.seg >> 1;  // lane's group within the chunk
    const int nsteps = nsteps_of(g, nrows);
#pragma unroll
    for (int st = 0; st < NB; ++st) {
        if (st >= nsteps) break;  // wave-uniform
        const int ur = st * g.rps + l.ri;
        const bool act = l.ok && ur < nrows;
        int acc[M];
        decode_staged<M>(S[st], lut, xr, acc);
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            const int v = acc[mi] + __builtin_amdgcn_update_dpp(0, acc[mi], kDppQuadSwap1, 0xF, 0xF, false);
            if (act && !(lane & 1)) {
                if (ACC) {
                    p.acc[((size_t)mi * p.n + row0 + ur) * ng + (l.dw0 >> 2)] = v;
                } else {
                    red_acc[(mi * NB + ur) * 32 + gi] = v;
                    if (mi == 0) red_sc[ur * 32 + gi] = S[st].scale;
                }
            }
        }
    }
    if (!ACC) {
        // Row rj's G group terms are summed by the LPR lanes of segment rj.
        constexpr int LPR = 64 / NB;                     // lanes per row
        constexpr int EPL = LPR >= 32 ? 1 : 32 / LPR;    // term slots per lane
        const int rj = lane / LPR;
        const int e0 = (lane % LPR) * EPL;               // (one row: lanes 32..63 have no slot)
        double sc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) sc[e] = (double)half_bits_to_float(red_sc[rj * 32 + min(e0 + e, 31)]);
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            double t = 0.0;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (e0 + e < g.G) t += sc[e] * (double)red_acc[(mi * NB + rj) * 32 + min(e0 + e, 31)];
            t = seg_sum_f64(t, LPR);
            const double rowsum = __shfl(t, (min(lane, NB - 1) + 1) * LPR - 1, 64);
            yv[mi] += lane < nrows ? rowsum : 0.0;
        }
    }
}

template <int M, bool ACC, int NB>
__global__ __launch_bounds__(kBlock) void bitcos_gemv_kernel(GroupArgs ga) {
    __shared__ uint4 s_ent4[(kByteLutEntries + 1) / 2];
    __shared__ uint32_t s_base8[256];
    __shared__ int32_t s_red_acc[kWaves][ACC ? 1 : M * NB * 32];
    __shared__ uint16_t s_red_sc[kWaves][ACC ? 2 : NB * 32];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(kByteLut.ent);
        for (int i = threadIdx.x; i < (kByteLutEntries + 1) / 2; i += kBlock) s_ent4[i] = src[i];
        if (threadIdx.x < 256) s_base8[threadIdx.x] = kByteLut.base8[threadIdx.x];
    }
    __syncthreads();
    const LutView lut{reinterpret_cast<const char *>(s_ent4), reinterpret_cast<const char *>(s_base8)};

    // The wave index is uniform across the wave: say so, so that all unit bookkeeping lives in
    // scalar registers and the loops are not compiled as divergent.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    int32_t *red_acc = s_red_acc[wave];
    uint16_t *red_sc = s_red_sc[wave];
    // Blocks are dealt to the XCDs round-robin; renumber them so that consecutive virtual blocks
    // sit on one XCD. Each wave takes a contiguous range of units (adjacent rows share sign-stream
    // lines and x stays hot in its XCD's L2).
    const int nblk = gridDim.x;
    const int vblk = (nblk % 8 == 0) ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
    const int vw = vblk * kWaves + wave;
    int u, u_end, pi;
    if (ga.ranges) {
        u = uniform_i32(ga.ranges[vw].begin);
        u_end = uniform_i32(ga.ranges[vw].end);
        pi = uniform_i32(ga.ranges[vw].problem);
    } else {
        const int nw = nblk * kWaves;
        const int share = (ga.units + nw - 1) / nw;
        u = min(vw * share, ga.units);
        u_end = min(u + share, ga.units);
        pi = 0;
    }
    if (u >= u_end) return;

    Problem p = uniform_problem(ga.table ? ga.table[pi] : ga.one);
    const bool more = ga.table && pi + 1 < ga.count;
    Problem pn = more ? uniform_problem(ga.table[pi + 1]) : p;  // next GEMV, fetched ahead
    int c = 0;
    uint32_t cur_v = 0;
    double yv[M];
#pragma unroll
    for (int mi = 0; mi < M; ++mi) yv[mi] = 0.0;

    Batch<M, NB> cur;
    issue_batch<M, NB>(p, u, c, true, cur);
    while (true) {
        // position of the next batch: the unit's next chunk, or the next unit's first chunk
        const bool last_chunk = c + 1 >= nchunks_of(p);
        int u2 = u, c2 = c + 1;
        bool switch_p = false;
        if (last_chunk) {
            u2 = u + 1;
            c2 = 0;
            switch_p = ga.table && pi + 1 < ga.count && u2 >= pn.unit_begin;
        }
        const bool has_next = u2 < u_end;
        const Problem &p2 = switch_p ? pn : p;

        Staged S[NB];
        stage_batch<M, ACC, NB>(p, u, c, cur, cur_v, S);
        TG_SCHED_FENCE();
        Batch<M, NB> nxt;
        issue_batch<M, NB>(has_next ? p2 : p, has_next ? u2 : u, has_next ? c2 : c, has_next, nxt);
        TG_SCHED_FENCE();
        finish_batch<M, ACC, NB>(p, u, c, S, cur.xr, lut, red_acc, red_sc, yv);

        if (last_chunk) {
            const int row0 = (u - p.unit_begin) * NB;
            if (!ACC && lane < min(NB, p.n - row0)) {
#pragma unroll
                for (int mi = 0; mi < M; ++mi) p.y[(size_t)mi * p.n + row0 + lane] = (float)yv[mi];
            }
#pragma unroll
            for (int mi = 0; mi < M; ++mi) yv[mi] = 0.0;
        }
        if (!has_next) break;
        if (switch_p) {
            ++pi;
            p = pn;
            if (pi + 1 < ga.count) pn = uniform_problem(ga.table[pi + 1]);
        }
        u = u2;
        c = c2;
        cur = nxt;
    }
}

template <int M, int NB>
hipError_t launch_nb(const GroupArgs &g, bool acc_out, hipStream_t s) {
    int blocks;
    if (g.ranges) {
        blocks = g.waves / kWaves;  // the table's per-wave ranges fix the grid
    } else {
        // one wave per unit up to two 512-thread blocks per CU (the 53 KB decode table allows no
        // more), a multiple of 8 so that every XCD gets the same number
        blocks = std::min((g.units + kWaves - 1) / kWaves, device_cus() * kBitcosBlocksPerCu);
        if (blocks > 8) blocks = blocks / 8 * 8;
        blocks = std::max(1, blocks);
    }
    if (acc_out)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, true, NB>), dim3(blocks), dim3(kBlock), 0, s, g);
    else
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, NB>), dim3(blocks), dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

// Largest batch (rows per unit) that keeps a wave within 128 registers, so that two 512-thread
// blocks fit a CU: 4 rows for one activation row, 2 for two, 1 for three.
template <int M>
constexpr int kMaxRowsPerUnit = M == 1 ? 4 : M == 2 ? 2 : 1;

template <int M>
hipError_t launch_m(const GroupArgs &g, bool acc_out, hipStream_t s) {
    if (g.rows_per_unit > kMaxRowsPerUnit<M>) return hipErrorInvalidValue;
    switch (g.rows_per_unit) {
        case 1: return launch_nb<M, 1>(g, acc_out, s);
        case 2:
            if constexpr (kMaxRowsPerUnit<M> >= 2) return launch_nb<M, 2>(g, acc_out, s);
            return hipErrorInvalidValue;
        case 4:
            if constexpr (kMaxRowsPerUnit<M> >= 4) return launch_nb<M, 4>(g, acc_out, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Rows per unit for BITCOS: a power of two (the batch size). Enough units to give every wave slot
// one, but at least the rows one tail step covers (so tail lanes are not left idle), and at most
// what keeps a wave within 128 registers. `table`: a grouped launch, where work is plentiful and
// the largest batch is used.
int bitcos_rows_per_unit(int64_t n, int64_t k, int m, bool table) {
    const int64_t cap = m == 1 ? kMaxRowsPerUnit<1> : m == 2 ? kMaxRowsPerUnit<2> : kMaxRowsPerUnit<3>;
    if (table) return (int)cap;
    const int64_t slots = (int64_t)device_cus() * kBitcosBlocksPerCu * kWaves;
    const int64_t kd = k >> 5;
    const int64_t tail = kd % kChunkDwords;
    const int64_t L = tail >> 1;
    const int64_t rps = (tail && (L & (L - 1)) == 0) ? 64 / L : 1;
    int64_t rpu = (n + slots - 1) / slots;
    rpu = std::max(rpu, std::min(rps, cap));
    int nb = 1;
    while (nb < rpu && nb < cap) nb <<= 1;
    return nb;
}

hipError_t launch_bitcos(const GroupArgs &g, bool acc_out, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_m<1>(g, acc_out, s);
        case 2: return launch_m<2>(g, acc_out, s);
        case 3: return launch_m<3>(g, acc_out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
