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

constexpr int kWaves = 8;
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

// One lane's share of a step after its bitmap dwords arrived: sign window and scale loads issued.
struct Staged {
    uint2 bm;
    u32x3 sg;        // sign dwords q, q+1, q+2 of the stream
    uint32_t r0;     // bit of sg.x where the lane's first sign sits
    uint16_t scale;  // fp16 scale of the lane's group (value path)
};

// `o0` is the stream position of the lane's first sign. The window load covers o0 .. o0 + 95
// (a lane's <= 64 signs start at most 31 bits into the first dword); reads past the section
// return zero.
template <bool ACC>
__device__ __forceinline__ Staged issue_signs(const Rsrc &r, uint2 bm, uint32_t o0, uint32_t scale_idx) {
    Staged st;
    st.bm = bm;
    st.r0 = o0 & 31;
    st.sg = buf_u32x3(r.sg, (o0 >> 5) * 4);
    // unconditional for every lane: a branch around a load makes the compiler wait for every load
    // in flight (the accumulator path has no scales)
    st.scale = ACC ? (uint16_t)0 : buf_u16(r.sc, scale_idx * 2);
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

// Load the 64 activation bytes of each of the M rows of x that a lane needs, starting at byte k0
// (zeros for an inactive lane).
template <int M>
__device__ __forceinline__ void load_x(const Rsrc &r, int k, int k0, bool active, uint32_t (&xr)[M][16]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = buf_u32x4(r.x, (uint32_t)(mi * k + k0 + 16 * j));
            xr[mi][4 * j] = active ? v.x : 0u;
            xr[mi][4 * j + 1] = active ? v.y : 0u;
            xr[mi][4 * j + 2] = active ? v.z : 0u;
            xr[mi][4 * j + 3] = active ? v.w : 0u;
        }
    }
}

// Process one unit: rows [row0, row0 + nrows) of problem p (1 <= nrows <= NB), all k.
// Each chunk of k is one fully unrolled batch of NB steps. Steps past the unit re-read its last
// row, change no cursor and write nothing. `red` is the wave's LDS scratch of M * NB * 32 doubles.
template <int M, bool ACC, int NB>
__device__ void run_unit(const Problem &p, const Rsrc &r, int row0, int nrows, const LutView &lut, double *red) {
    const int lane = threadIdx.x & 63;
    const int n = p.n, k = p.k;
    const int kd = k >> 5;  // bitmap dwords per row
    const int ng = k >> 7;
    const int nfull = kd / kChunkDwords;
    const int tail = kd - nfull * kChunkDwords;  // multiple of 4
    const int last = nrows - 1;

    // lane u < nrows tracks row row0 + u: its running sign cursor and its output sums
    uint32_t cur_v = p.rowoff[row0 + min(lane, last)];
    double yv[M];
#pragma unroll
    for (int mi = 0; mi < M; ++mi) yv[mi] = 0.0;

    uint32_t xr[M][16];

    // ---------------- full chunks: one row per step, 64 lanes x 2 dwords ----------------
    for (int c = 0; c < nfull; ++c) {
        const int dw0 = c * kChunkDwords + 2 * lane;  // lane's first bitmap dword in the row
        const int g = dw0 >> 2;                       // lane's group
        load_x<M>(r, k, 32 * dw0, true, xr);
        uint2 b[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const u32x2 v = buf_u32x2(r.bm, (uint32_t)((row0 + min(j, last)) * kd + dw0) * 4);
            b[j] = make_uint2(v.x, v.y);
        }
        TG_SCHED_FENCE();
        Staged S[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int jc = min(j, last);
            const uint32_t pc = __builtin_popcount(b[j].x) + __builtin_popcount(b[j].y);
            const uint32_t incl = wave_incl_scan(pc);
            const uint32_t rowcur = (uint32_t)__builtin_amdgcn_readlane((int)cur_v, jc);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            cur_v += (lane == j && j < nrows) ? total : 0u;
            S[j] = issue_signs<ACC>(r, b[j], rowcur + incl - pc, ACC ? 0u : (uint32_t)((row0 + jc) * ng + g));
        }
        TG_SCHED_FENCE();
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int acc[M];
            decode_staged<M>(S[j], lut, xr, acc);
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                const int v = acc[mi] + __builtin_amdgcn_update_dpp(0, acc[mi], kDppQuadSwap1, 0xF, 0xF, false);
                if (ACC) {
                    if (!(lane & 1) && j < nrows) p.acc[((size_t)mi * n + row0 + j) * ng + g] = v;
                } else if (!(lane & 1)) {
                    red[(mi * NB + j) * 32 + (lane >> 1)] = (double)half_bits_to_float(S[j].scale) * (double)v;
                }
            }
        }
        if (!ACC) {
            // Row j's 32 group terms are summed by the 64/NB lanes of segment j.
            constexpr int LPR = 64 / NB;                  // lanes per row
            constexpr int EPL = NB >= 2 ? NB / 2 : 1;     // terms per lane
            const int rj = lane / LPR;
            const int e0 = (lane % LPR) * EPL;
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                double t = 0.0;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    if (NB >= 2 || lane < 32) t += red[(mi * NB + rj) * 32 + e0 + e];
                t = seg_sum_f64(t, LPR);
                const double rowsum = __shfl(t, (min(lane, NB - 1) + 1) * LPR - 1, 64);
                yv[mi] += lane < NB ? rowsum : 0.0;
            }
        }
    }

    // ---------------- tail: the last `tail` dwords of several rows per step ----------------
    if (tail) {
        const int L = tail >> 1;                  // lanes per row (even, < 64)
        const bool pow2 = (L & (L - 1)) == 0;
        // rows per step: power-of-two segments are reduced inside the segment; other widths take
        // one row per step and reduce over the whole wave
        const int rps = pow2 ? 64 / L : 1;
        const int ri = lane / L;                  // row of this lane within a step
        const int seg = lane - ri * L;
        const bool lane_ok = ri < rps;
        const int dw0 = nfull * kChunkDwords + 2 * seg;
        const int g = dw0 >> 2;
        const int seg_first = ri * L;
        const int seg_last = min(seg_first + L - 1, 63);
        load_x<M>(r, k, 32 * dw0, lane_ok, xr);
        const int nsteps = (nrows + rps - 1) / rps;  // <= NB
        uint2 b[NB];
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const int u = st * rps + ri;
            const u32x2 v = buf_u32x2(r.bm, (uint32_t)((row0 + min(u, last)) * kd + (lane_ok ? dw0 : 0)) * 4);
            b[st] = (lane_ok && u < nrows) ? make_uint2(v.x, v.y) : make_uint2(0, 0);
        }
        TG_SCHED_FENCE();
        Staged S[NB];
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const int u = st * rps + ri;
            const bool act = lane_ok && u < nrows;
            const uint32_t pc = __builtin_popcount(b[st].x) + __builtin_popcount(b[st].y);
            const uint32_t incl = wave_incl_scan(pc);
            // inclusive sums just before this lane's row segment and at its end (the shuffles run
            // on every lane: a lane-permute reading from a lane that is switched off returns zero)
            const uint32_t prev = (uint32_t)__shfl((int)incl, max(seg_first - 1, 0), 64);
            const uint32_t before = seg_first > 0 ? prev : 0u;
            const uint32_t end = (uint32_t)__shfl((int)incl, seg_last, 64);
            const uint32_t rowcur = (uint32_t)__shfl((int)cur_v, min(u, 63), 64);
            // unit row v = st*rps + i takes the total of step row i (held by lane i*L)
            const int i = lane - st * rps;
            const bool mine = i >= 0 && i < rps && lane < nrows;
            const uint32_t t = (uint32_t)__shfl((int)(end - before), mine ? i * L : 0, 64);
            cur_v += mine ? t : 0u;
            S[st] = issue_signs<ACC>(r, b[st], act ? rowcur + incl - pc - before : 0u,
                                     (act && !ACC) ? (uint32_t)((row0 + u) * ng + g) : 0u);
        }
        TG_SCHED_FENCE();
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            if (st >= nsteps) break;  // wave-uniform
            int acc[M];
            decode_staged<M>(S[st], lut, xr, acc);
            const int u = st * rps + ri;
            const bool act = lane_ok && u < nrows;
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                const int v = acc[mi] + __builtin_amdgcn_update_dpp(0, acc[mi], kDppQuadSwap1, 0xF, 0xF, false);
                if (ACC) {
                    if (act && !(lane & 1)) p.acc[((size_t)mi * n + row0 + u) * ng + g] = v;
                } else {
                    double part = (act && !(lane & 1)) ? (double)half_bits_to_float(S[st].scale) * (double)v : 0.0;
                    part = seg_sum_f64(part, pow2 ? L : 64);
                    // the last lane of a power-of-two segment holds its sum; otherwise lane 63
                    // holds the (single) row's sum
                    const int i = lane - st * rps;
                    const bool mine = i >= 0 && i < rps;
                    const double t = __shfl(part, !mine ? 0 : pow2 ? i * L + L - 1 : 63, 64);
                    yv[mi] += mine ? t : 0.0;
                }
            }
        }
    }

    if (!ACC && lane < nrows) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) p.y[(size_t)mi * n + row0 + lane] = (float)yv[mi];
    }
}

template <int M, bool ACC, int NB>
__global__ __launch_bounds__(kBlock) void bitcos_gemv_kernel(GroupArgs ga) {
    __shared__ uint4 s_ent4[(kByteLutEntries + 1) / 2];
    __shared__ uint32_t s_base8[256];
    __shared__ double s_red[kWaves][ACC ? 1 : M * NB * 32];
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
    double *red = s_red[wave];
    // Blocks are dealt to the XCDs round-robin; renumber them so that consecutive virtual blocks
    // sit on one XCD, and give consecutive units to consecutive virtual waves.
    const int nblk = gridDim.x;
    const int vblk = (nblk % 8 == 0) ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
    const int nwaves = nblk * kWaves;
    const int rpu = ga.rows_per_unit;

    int pi = 0;  // current problem (table mode); units are visited in increasing order
    Problem p = ga.table ? ga.table[0] : ga.one;
    for (int u = vblk * kWaves + wave; u < ga.units; u += nwaves) {
        if (ga.table) {
            bool moved = false;
            while (pi + 1 < ga.count && ga.table[pi + 1].unit_begin <= u) {
                ++pi;
                moved = true;
            }
            if (moved) p = ga.table[pi];
        }
        Rsrc r;
        r.bm = make_rsrc(p.codes, p.codes_bytes);
        r.sg = make_rsrc(p.signs, p.sign_bytes);
        r.sc = make_rsrc(p.scales, ACC ? 0u : (uint32_t)p.n * (uint32_t)(p.k >> 7) * 2u);
        r.x = make_rsrc(p.x, (uint32_t)ga.m * (uint32_t)p.k);
        const int row0 = (u - p.unit_begin) * rpu;
        run_unit<M, ACC, NB>(p, r, row0, min(rpu, p.n - row0), lut, red);
    }
}

template <int M, int NB>
hipError_t launch_nb(const GroupArgs &g, bool acc_out, hipStream_t s) {
    // Two 512-thread blocks per CU (the 53 KB decode table allows no more); a persistent grid of at
    // most that many blocks, a multiple of 8 so that every XCD gets the same number.
    const int cap = device_cus() * 2;
    int blocks = std::min((g.units + kWaves - 1) / kWaves, cap);
    if (blocks > 8) blocks = blocks / 8 * 8;
    blocks = std::max(1, blocks);
    if (acc_out)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, true, NB>), dim3(blocks), dim3(kBlock), 0, s, g);
    else
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, NB>), dim3(blocks), dim3(kBlock), 0, s, g);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const GroupArgs &g, bool acc_out, hipStream_t s) {
    switch (g.rows_per_unit) {
        case 1: return launch_nb<M, 1>(g, acc_out, s);
        case 2: return launch_nb<M, 2>(g, acc_out, s);
        case 4: return launch_nb<M, 4>(g, acc_out, s);
        case 8:
            if constexpr (M == 1) return launch_nb<M, 8>(g, acc_out, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Rows per unit for BITCOS: a power of two (the batch size). Enough units to give every wave slot
// one, but at least the rows one tail step covers (so tail lanes are not left idle); at most 8 for
// one activation row and 4 for more (the LDS scratch grows with both).
int bitcos_rows_per_unit(int64_t n, int64_t k, int m) {
    const int64_t slots = (int64_t)device_cus() * 2 * kWaves;
    const int64_t kd = k >> 5;
    const int64_t tail = kd % kChunkDwords;
    const int64_t L = tail >> 1;
    const int64_t rps = (tail && (L & (L - 1)) == 0) ? 64 / L : 1;
    const int64_t cap = m == 1 ? 8 : 4;
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
