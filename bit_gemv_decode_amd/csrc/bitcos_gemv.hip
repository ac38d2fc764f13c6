// BITCOS unpack-fused GEMV for gfx950 (int8 activations, ternary weights, fp16 group scales).
//
// Format ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-A, Fig. 2): a presence bitmap
// with one bit per weight and a compacted sign stream with one bit per non-zero weight; the j-th sign
// bit belongs to the j-th set bit of the bitmap. Decoding places the compact signs back onto the
// present positions (the deposit of Fig. 4); the int8 path of Sec. II-C turns each (present,
// negative) pair into w = p - 2n (Eq. 2), contracts against int8 activations in int32 and applies
// the group scale once per 128-element group.
//
// Mapping on CDNA4 (wave64, one persistent block per CU: 1024 threads at m = 1, 512 at m = 2, 3; 768 at
// m = 2 for launches without chunked rows, with two-step units):
//   * a lane owns one 128-weight group of one row per step: its four bitmap dwords arrive with one
//     16-byte load, its scale with one 2-byte load. A row of k weights takes ng = k/128 lanes; when
//     ng <= 64 a step holds R = 64/ng consecutive rows (at most 64/NB, so that a unit's NB steps hold
//     no more rows than a wave has lanes: k = 128 and 256 leave lanes idle), otherwise a row is split
//     into chunks of 64 groups, one chunk per step. A lane's activation bytes (its group's 128 x values) stay in
//     registers for every row it sees, so x is read once per GEMV (or once per chunk pass). Rows of
//     40 groups (k = 5120) at m = 1 with fp32 outputs take wide lanes instead: 80 weights per lane, so
//     one row fills the wave (see kW80Groups).
//   * sign positions: rows of a step are consecutive in the sign stream, so a lane's first sign sits
//     at the step's cursor (from the row index, or carried from the row's previous chunk) plus the
//     exclusive prefix sum of the popcounts of the lanes before it (DPP scan). For each pair of bitmap
//     dwords the lane loads the four sign-stream dwords holding bits [pos - 3, pos + 93) and
//     funnel-shifts them (pos is the pair's first sign; the second dword's window follows by a 64-bit
//     shift of the popcount of the first).
//   * the deposit of Fig. 4 is a table lookup in LDS, keyed per presence byte (the nibble-keyed
//     lookup of Sec. II-D, Eq. 4 and Fig. 9, widened to a byte): entry (pb, s) holds the 8 ternary
//     int8 weights for presence byte pb followed by the popcount(pb) compact signs s; 3^8 = 6561
//     entries of 8 bytes. The entries of one pb form a block of 2^popcount(pb) entries aligned to its
//     own size, so the entry address is (window & mask) | base: one instruction, with mask and base
//     fetched per presence byte from a 256-entry table. That small table is kept in 32 copies, one
//     per LDS bank, and lane l reads copy l % 32, so those reads never conflict; the copy address is
//     one byte-permute of the bitmap dword. The per-byte sign cursor is the running popcount of the
//     masks.
//   * v_dot4_i32_i8 contracts 4 weights per instruction. Each group's int32 sum times its fp16 scale
//     (exact in fp64) goes to an LDS tile; once per unit the tile's rows are summed (fp64, DPP) and
//     stored as fp32. Chunked rows at m = 1 keep those terms in registers instead (one fp64 per row
//     of the unit and lane, summed over the chunk passes) and, at the unit's end, pass them through
//     the tile four rows at a time: each lane sums four terms of one row, then 16 lanes by DPP.
//   * alternative decode (NIB, Sec. II-D, Eq. 4): the Xe2 kernel's nibble-keyed lookup, a 256-entry
//     table keyed by a presence nibble and the next four compact signs, each entry the nibble's 4 int8
//     weights; one conflict-free 4-byte LDS read and one v_dot4_i32_i8 per nibble, with the sign
//     cursor advanced by the nibble's popcount. Selected per grouped launch for comparison; it takes
//     one LDS round trip per nibble but about twice the VALU work per weight of the byte-keyed decode.
//   * fp16 activations (Sec. II-B: the weights rebuilt as +-1 or 0 in 16-bit floating point; Sec.
//     II-D: lookup entries holding fp16 weights): the same lookups on a second table whose entry bytes
//     are the binary16 high bytes of +1.0 and -1.0 (low bytes zero), so one byte-permute turns two
//     entry bytes into two fp16 weights and v_dot2_f32_f16 contracts them with two activations into
//     an fp32 group sum. Each lane holds its group's 128 activations (256 bytes) in registers.
//   * loads are software-pipelined: a step's bitmap four half-steps before its decode, its sign
//     windows two, with the loop unrolled so that no register with a load in flight is ever copied.
//     Every load goes through a buffer resource and is issued unconditionally; lanes with nothing to
//     read use an out-of-range offset, which returns zero without a memory request.
#include <algorithm>
#include <type_traits>

#include "bitcos_tables.h"
#include "gemv_pipeline.h"

namespace tg {
namespace {

// Sign stage of one step: for each pair of bitmap dwords, the four sign-stream dwords holding bits
// [pos - 3, pos + 93) (pos = the pair's first sign); the two funnel-shift amounts into them (bytes 0
// and 1 of `sh`); the group scale.
struct SgBuf {
    u32x4 s[2];
    uint32_t sh;
    uint16_t scale;
};

// Scan the step's bitmap popcounts and issue its sign-window and scale loads. `cur` is the stream
// position of the step's first sign; returns the step's sign count.
template <bool ACC>
__device__ __forceinline__ uint32_t stage_signs(const Ctx &x, const u32x4 &bm, uint32_t cur, bool live,
                                                uint32_t voff_sc, uint32_t soff_sc, SgBuf &g) {
    const uint32_t t1 = __builtin_popcount(bm.x);
    const uint32_t t2 = __builtin_popcount(bm.y) + t1;
    const uint32_t t3 = __builtin_popcount(bm.z) + t2;
    const uint32_t pc = __builtin_popcount(bm.w) + t3;
    const uint32_t incl = wave_incl_scan(pc);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    // window start = first sign - 3, biased by +32 (the sign resource starts one dword early)
    const uint32_t b0 = cur + 29u + incl - pc;
    const uint32_t b2 = b0 + t2;
    const uint32_t sd = live_or_dead(live, 0u);
    g.s[0] = ld4(x.rsg, (b0 >> 5) << 2, sd);
    g.s[1] = ld4(x.rsg, (b2 >> 5) << 2, sd);
    g.sh = __builtin_amdgcn_perm(b2, b0, 0x0C0C0400u);  // byte 0: b0, byte 1: b2 (low 5 bits used)
    g.scale = ACC ? (uint16_t)0 : ldhs(x.rsc, voff_sc, live_or_dead(live, soff_sc));
    return total;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// acc + a.lo * b.lo + a.hi * b.hi for two fp16 pairs (products exact in fp32).
__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, a), __builtin_bit_cast(h2v, b), acc, false);
}

// Two bitmap dwords (64 weights) of decode. lo*/hi* hold the sign-stream bits starting 3 bits before
// each dword's first sign. All eight per-byte (mask, base) reads go out first, then all eight entry
// reads, then the dot products: two LDS round trips for the 64 weights.
// With F16, entries come from the fp16 table and xr holds fp16 activations (two per dword). With NIB
// the lookups are nibble-keyed instead (int8 only).
template <int M, bool F16, bool NIB, int XW, typename A>
__device__ __forceinline__ void decode_pair(uint32_t bma, uint32_t bmb, uint32_t loa, uint32_t hia, uint32_t lob,
                                            uint32_t hib, const uint32_t (&xr)[M][XW], int d, const char *lds,
                                            uint32_t laneoff, A (&acc)[M]) {
    if constexpr (NIB) {
        static_assert(!F16, "nibble-keyed decode: int8 activations");
        const uint32_t lane4 = laneoff >> 1;  // copy (lane % 32) of an entry
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t bm = h ? bmb : bma, lo = h ? lob : loa, hi = h ? hib : hia;
            uint32_t c = 3;  // the dword's first sign sits at bit 3 of its window
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t nb = (bm >> (4 * j)) & 15u;
                // c <= 3 + 28: the nibble's signs start inside the 64-bit window's low 35 bits
                const uint32_t sg = __builtin_amdgcn_alignbit(hi, lo, c) & 15u;
                const uint32_t ent = *reinterpret_cast<const uint32_t *>(lds + ((sg << 11) | (nb << 7) | lane4));
                if (j < 7) c = __builtin_popcount(nb) + c;
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(ent, xr[mi][8 * d + 8 * h + j], acc[mi]);
            }
        }
        return;
    }
    uint2 info[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // (pb << 8) | laneoff: copy (lane % 32) of presence byte pb's (mask, base)
        const uint32_t ia = __builtin_amdgcn_perm(i < 4 ? bma : bmb, laneoff, 0x0C0C0000u | ((4u + (i & 3)) << 8));
        info[i] = *reinterpret_cast<const uint2 *>(lds + ia);
    }
    uint2 e[8];
    uint32_t ca = 0, cb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // byte i's signs sit at bits 3 .. 3 + popcount of the window shifted by the bytes before it
        const uint32_t wa = i == 0 ? loa : __builtin_amdgcn_alignbit(hia, loa, ca);
        const uint32_t wb = i == 0 ? lob : __builtin_amdgcn_alignbit(hib, lob, cb);
        e[i] = *reinterpret_cast<const uint2 *>(lds + ((wa & info[i].x) | info[i].y));
        e[4 + i] = *reinterpret_cast<const uint2 *>(lds + ((wb & info[4 + i].x) | info[4 + i].y));
        if (i < 3) {
            ca = __builtin_popcount(info[i].x) + ca;
            cb = __builtin_popcount(info[4 + i].x) + cb;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (F16) {
            // weights 2j, 2j + 1 of the entry as a half2: entry bytes to bits 8..15 and 24..31
            const uint32_t w0 = __builtin_amdgcn_perm(e[i].x, e[i].x, 0x050C040Cu);
            const uint32_t w1 = __builtin_amdgcn_perm(e[i].x, e[i].x, 0x070C060Cu);
            const uint32_t w2 = __builtin_amdgcn_perm(e[i].y, e[i].y, 0x050C040Cu);
            const uint32_t w3 = __builtin_amdgcn_perm(e[i].y, e[i].y, 0x070C060Cu);
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                const int xi = 16 * d + 4 * i;
                acc[mi] = fdot2(w0, xr[mi][xi], acc[mi]);
                acc[mi] = fdot2(w1, xr[mi][xi + 1], acc[mi]);
                acc[mi] = fdot2(w2, xr[mi][xi + 2], acc[mi]);
                acc[mi] = fdot2(w3, xr[mi][xi + 3], acc[mi]);
            }
        } else {
#pragma unroll
            for (int mi = 0; mi < M; ++mi) {
                acc[mi] = dot4(e[i].x, xr[mi][8 * d + 2 * i], acc[mi]);
                acc[mi] = dot4(e[i].y, xr[mi][8 * d + 2 * i + 1], acc[mi]);
            }
        }
    }
}

// Sums of the lane's 128 weights times x, per activation row (int32; fp32 with F16).
template <int M, bool F16, bool NIB, int XW, typename A>
__device__ __forceinline__ void decode(const u32x4 &bm, const SgBuf &g, const uint32_t (&xr)[M][XW],
                                       const char *lds, uint32_t laneoff, A (&acc)[M]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) acc[mi] = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const u32x4 s = g.s[q];
        const uint32_t sh = q == 0 ? g.sh : g.sh >> 8;
        const uint32_t a0 = __builtin_amdgcn_alignbit(s.y, s.x, sh);
        const uint32_t a1 = __builtin_amdgcn_alignbit(s.z, s.y, sh);
        const uint32_t a2 = __builtin_amdgcn_alignbit(s.w, s.z, sh);
        // the pair's second dword starts popcount(first dword) = 0 .. 32 bits later
        const uint32_t pc = __builtin_popcount(q == 0 ? bm.x : bm.z);
        const uint64_t w01 = ((uint64_t)a1 << 32) | a0, w12 = ((uint64_t)a2 << 32) | a1;
        const uint32_t b0 = (uint32_t)(w01 >> pc), b1 = (uint32_t)(w12 >> pc);
        decode_pair<M, F16, NIB>(q == 0 ? bm.x : bm.z, q == 0 ? bm.y : bm.w, a0, a1, b0, b1, xr, 2 * q, lds, laneoff, acc);
    }
}

// Rows of 5120 weights (40 groups) at m = 1 with fp32 outputs. With a lane per 128-weight group,
// a step of such a row keeps 24 of the 64 lanes idle. Instead each lane takes 80 consecutive weights
// (ten presence bytes), so a row fills the wave: lane l holds weights [80 l, 80 l + 80), which lie in
// one group or straddle two, the boundary falling on an even presence byte. The lane keeps its int32
// sum up to the boundary apart and scales the two parts with their own group scales.
constexpr int kW80Groups = (int)(kWideLaneK / TG_GROUP);

// Sign stage of one step of a wide-lane row: one four-dword window of the sign stream holding bits
// [pos - 3, pos + 93) (pos = the lane's first sign; its at most 80 signs end before pos + 80), the
// funnel-shift amount into it, the scales of the lane's first and last group.
struct SgBufW {
    u32x4 s;
    uint32_t sh;
    uint16_t sc1, sc2;
};

// The lane's ten bitmap bytes start `bsh` bits (0 or 16) into its 16-byte load: they are moved to the
// bottom of bm (bm.z keeps bytes 8 and 9 in its low half). Then the row's popcount scan and the sign
// and scale loads, as stage_signs does for group lanes.
__device__ __forceinline__ uint32_t stage_signs_w80(const Ctx &x, u32x4 &bm, uint32_t bsh, uint32_t cur, bool live,
                                                    uint32_t voff_sc1, uint32_t voff_sc2, uint32_t soff_sc,
                                                    SgBufW &g) {
    const uint32_t d0 = __builtin_amdgcn_alignbit(bm.y, bm.x, bsh);
    const uint32_t d1 = __builtin_amdgcn_alignbit(bm.z, bm.y, bsh);
    const uint32_t d2 = __builtin_amdgcn_alignbit(bm.w, bm.z, bsh) & 0xFFFFu;
    bm.x = d0;
    bm.y = d1;
    bm.z = d2;
    const uint32_t pc = __builtin_popcount(d0) + __builtin_popcount(d1) + __builtin_popcount(d2);
    const uint32_t incl = wave_incl_scan(pc);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    // window start = first sign - 3, biased by +32 (the sign resource starts one dword early)
    const uint32_t b0 = cur + 29u + incl - pc;
    g.s = ld4(x.rsg, (b0 >> 5) << 2, live_or_dead(live, 0u));
    g.sh = b0;  // alignbit uses the low 5 bits
    const uint32_t so = live_or_dead(live, soff_sc);
    g.sc1 = ldhs(x.rsc, voff_sc1, so);
    g.sc2 = ldhs(x.rsc, voff_sc2, so);
    return total;
}

// Ten presence bytes of a wide lane: bytes 0..3 in d.x, 4..7 in d.y, 8 and 9 in d.z. The (mask, base)
// and entry reads are those of decode_pair, for the pair plus the two bytes after it, whose window
// starts popcount(d.x) + popcount(d.y) signs in. acc1 is the sum over the bytes before `sb` (the byte
// where the lane's second group starts; 10 when it has one group), acc2 over the rest.
__device__ __forceinline__ void decode_w80(const u32x4 &d, const SgBufW &g, const uint32_t (&xr)[1][20],
                                           const char *lds, uint32_t laneoff, int sb, int &acc1, int &acc2) {
    const uint32_t a0 = __builtin_amdgcn_alignbit(g.s.y, g.s.x, g.sh);
    const uint32_t a1 = __builtin_amdgcn_alignbit(g.s.z, g.s.y, g.sh);
    const uint32_t a2 = __builtin_amdgcn_alignbit(g.s.w, g.s.z, g.sh);
    const uint32_t p0 = __builtin_popcount(d.x);
    const uint32_t pp = __builtin_popcount(d.y) + p0;  // 0 .. 64
    const uint64_t w01 = ((uint64_t)a1 << 32) | a0, w12 = ((uint64_t)a2 << 32) | a1;
    const uint32_t b0 = (uint32_t)(w01 >> p0), b1 = (uint32_t)(w12 >> p0);
    const uint32_t we = pp < 32u ? (uint32_t)(w01 >> pp) : (uint32_t)(w12 >> (pp - 32u));
    uint2 info[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t src = i < 4 ? d.x : i < 8 ? d.y : d.z;
        const uint32_t ia = __builtin_amdgcn_perm(src, laneoff, 0x0C0C0000u | ((4u + (i & 3)) << 8));
        info[i] = *reinterpret_cast<const uint2 *>(lds + ia);
    }
    uint2 e[10];
    uint32_t ca = 0, cb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wa = i == 0 ? a0 : __builtin_amdgcn_alignbit(a1, a0, ca);
        const uint32_t wb = i == 0 ? b0 : __builtin_amdgcn_alignbit(b1, b0, cb);
        e[i] = *reinterpret_cast<const uint2 *>(lds + ((wa & info[i].x) | info[i].y));
        e[4 + i] = *reinterpret_cast<const uint2 *>(lds + ((wb & info[4 + i].x) | info[4 + i].y));
        if (i < 3) {
            ca = __builtin_popcount(info[i].x) + ca;
            cb = __builtin_popcount(info[4 + i].x) + cb;
        }
    }
    e[8] = *reinterpret_cast<const uint2 *>(lds + ((we & info[8].x) | info[8].y));
    const uint32_t w9 = we >> __builtin_popcount(info[8].x);
    e[9] = *reinterpret_cast<const uint2 *>(lds + ((w9 & info[9].x) | info[9].y));
    int acc = 0, snap = 0;
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        acc = dot4(e[i].x, xr[0][2 * i], acc);
        acc = dot4(e[i].y, xr[0][2 * i + 1], acc);
        if (i == 1 || i == 3 || i == 5 || i == 7) snap = sb == i + 1 ? acc : snap;
    }
    acc1 = sb < 10 ? snap : acc;
    acc2 = acc - acc1;
}

// Pipeline over the steps of units [u0, u1) of one GEMV. In half-step h, step h - 4 is decoded, the
// bitmap of step h is loaded, and the signs of step h - LAG (LAG = 2 for units of four or more steps,
// else 1) are located and loaded: a bitmap has LAG half-steps to arrive, a sign window 4 - LAG (the
// bitmap load goes first, so that waiting for it never waits for younger sign loads). The loop body holds four half-steps, so every stage
// buffer has a fixed register home (bitmaps and sign windows rotate over four) and no register with
// a load in flight is ever copied. Each stage runs unconditionally (outside the live range its loads
// use dead offsets), apart from decode work that loads nothing.
//
// Single-chunk GEMVs (ng <= 64): step s covers rows row_begin + s*R .. + R - 1, a unit NB steps; the
// sign cursor runs on from step to step. Chunked GEMVs: a unit is NB rows; its steps go chunk by
// chunk (NB steps per chunk pass), each row's cursor carried from its previous chunk. With NB > 4 the
// body holds NB half-steps and the stage slots are taken modulo NB.
template <int M, bool ACC, int NB, bool CHUNKED, bool XS, bool F16, bool NIB>
__device__ __forceinline__ void run_loop(const Problem &p, int u0, int u1, const char *lds, double *tile) {
    static_assert(!(F16 && (ACC || XS)), "fp16 activations: fp32 outputs only");
    // activation slice of a lane: 32 dwords of int8 or 64 dwords of fp16 (XB bytes)
    constexpr int XW = F16 ? 64 : 32;
    constexpr uint32_t XB = 4u * XW;
    using A = typename std::conditional<F16, float, int>::type;
    // Chunked rows at m = 1: units of 8 rows (the activation slice is reloaded once per pass, so
    // longer passes halve those reloads), each lane summing its group terms of the unit's rows in
    // registers across passes; the rows are reduced over the wave once, at the unit's end.
    constexpr bool RACC = CHUNKED && M == 1;
    constexpr int U = NB > 4 ? NB : 4;  // half-steps per loop body
    static_assert(U % NB == 0 && U % 4 == 0, "static stage positions");
    // Half-steps between a step's bitmap load and its sign stage: two, so that the bitmap and the sign
    // windows each have two half-steps to arrive (measured 2 % faster than one and three on MI355X,
    // and it frees the registers that let 16 waves share a CU at m = 1). The row-index entries loaded
    // with a unit's first bitmap are read by its first sign stage; with units of two steps they sit
    // in two registers that alternate from unit to unit. m = 3 chunked (two-step units) keeps one.
    constexpr int LAG = (NB >= 4 || M == 1) ? 2 : 1;
    const int lane = threadIdx.x & 63;
    Ctx x;
    x.n = p.n;
    x.k = p.k;
    x.ng = p.ng;
    x.nch = p.nch;
    x.G = p.G;
    x.R = p.R;
    x.glast = p.glast;
    x.rbm = make_rsrc(p.codes, p.codes_bytes);
    // the sign resource starts 4 bytes early so that the window of a position below 3 (the stream's
    // first bits) is in range; the 4 bytes before the sign section belong to the packed buffer
    x.rsg = make_rsrc(reinterpret_cast<const uint8_t *>(p.signs) - 4, p.sign_bytes + 4u);
    x.rsc = make_rsrc(p.scales, ACC ? 0u : (uint32_t)p.n * (uint32_t)p.ng * 2u);
    x.rro = make_rsrc(p.rowoff, (uint32_t)(p.n + 1) * 4u);
    x.rx = make_rsrc(p.x, (uint32_t)M * (uint32_t)p.k * (F16 ? 2u : 1u));
    x.ry = make_rsrc(p.y, ACC ? 0u : (uint32_t)M * (uint32_t)p.n * 4u);
    x.racc = make_rsrc(p.acc, ACC ? (uint32_t)M * (uint32_t)p.n * (uint32_t)p.ng * 4u : 0u);
    x.rxs = make_rsrc(p.xs, XS ? (uint32_t)M * (uint32_t)p.ng * 4u : 0u);
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    const int rpu = p.rpu;
    const int row_begin = (u0 - p.unit_begin) * rpu;
    const int row_end = min(p.n, (u1 - p.unit_begin) * rpu);
    const uint32_t kb = (uint32_t)(p.k >> 3);  // bitmap bytes per row

    uint32_t xr[M][XW];
    float xsv[M];               // activation group scales of the lane's group (1 without them)
    uint32_t cur = 0;           // single-chunk: sign cursor of the next step to scan
    uint32_t ccur[NB] = {};     // chunked: sign cursor of each row of the unit being scanned
    double facc[RACC ? NB : 1];  // chunked, m = 1: the lane's running term of each row of the unit
#pragma unroll
    for (int r = 0; r < (RACC ? NB : 1); ++r) facc[r] = 0.0;
    uint32_t ro[2] = {0, 0};    // chunked: row-index entries of the unit (lane r: row r), by unit parity
    int T;                      // steps in the range
    // per-lane constant parts of the offsets
    uint32_t voff_bm, voff_sc, voff_acc, voff_x;
    Red red;
    if constexpr (!CHUNKED) {
        const int ql = (int)(((uint32_t)lane * p.gmagic) >> 16);  // lane / G: row within the step
        const int jl = lane - ql * x.G;                           // group within the row
        const bool act = lane < x.R * x.G;
        voff_bm = act ? (uint32_t)ql * kb + (uint32_t)jl * 16u : kOffOff;
        voff_sc = act ? (uint32_t)lane * 2u : kOffOff;  // (ql * ng + jl) = lane when ng = G
        voff_acc = act ? (uint32_t)lane * 4u : kOffOff;
        voff_x = act ? (uint32_t)jl * XB : kOffOff;
        T = (u1 - u0) * NB;
        red = make_red(NB * x.R, x.R, x.G, p.rmagic);
        cur = row_index_entry(p, row_begin);
    } else {
        voff_bm = (uint32_t)lane * 16u;
        voff_sc = (uint32_t)lane * 2u;
        voff_acc = (uint32_t)lane * 4u;
        voff_x = (uint32_t)lane * XB;
        T = (u1 - u0) * NB * x.nch;
        red = make_red(NB, 1, 64, p.rmagic);
    }
    // The activation slice is waited for only before the first decode: its loads go out with the
    // first bitmaps, and waiting for those (the first sign stage) covers the slice too, since vector
    // loads complete in order. One memory round trip less per range than waiting here.
    // (Units of eight chunked rows decode in the first pass of the loop body already: they wait here.)
    load_x<M, XW>(x, voff_x, xr);
    load_xs<M, XS>(x, voff_x, xsv);
    if constexpr (U != 4) {
        wait_x<M, XW>(xr);
        wait_xs<M, XS>(xsv);
    }

    u32x4 bm[4] = {};
    SgBuf g[4] = {};
    // chunked stage positions: chunk and first row of the unit of the step each stage handles
    int cB = 0, rB = row_begin, cS = 0, rS = row_begin, cD = 0, rD = row_begin;

    // Uniform branches cost each wave an instruction-fetch bubble, so the loop body has none: every
    // stage runs on every half-step, dead steps (pipeline fill and drain) decode whatever their
    // buffers hold into tile slots that a live step overwrites before use, and only their stores and
    // loads are switched off (dead offsets). Scalar state advances with selects. The first pass of the
    // body is a copy (FIRST) without the decodes of its first four half-steps, whose steps do not
    // exist; the activation wait sits before its first decode.
    for (int it = 0; U * it - 4 < T; ++it) {
        // with four half-steps per pass, the first pass holds no decode (its steps would be -4 .. -1)
        const bool first = U == 4 && it == 0;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int h = U * it + j;
            const int jb = j & 3;  // stage buffer slot
            // ---- decode step h - 4 (buffers bm[jb], g[jb]) ----
            if (!first) {
                const int s = h - 4;
                const bool live = s >= 0 && s < T;
                A acc[M];
                decode<M, F16, NIB>(bm[jb], g[jb], xr, lds, laneoff, acc);
                const int slot = (j + U - 4) % NB;  // step h - 4 within its unit (pass)
                if constexpr (!CHUNKED) {
                    const int row0 = row_begin + s * x.R;
                    const bool va = live && (lane < x.R * x.G) &&
                                    row0 + (int)(((uint32_t)lane * p.gmagic) >> 16) < row_end;
                    emit<M, ACC, NB, XS>(x, acc, (double)half_bits_to_float(g[jb].scale), xsv, tile, slot, false,
                                         va ? voff_acc : kOffOff,
                                     live_or_dead(live, (uint32_t)row0 * (uint32_t)x.ng * 4u));
                    if constexpr (!ACC) {
                        if (slot == NB - 1) reduce_store<M, NB>(x, red, tile, row0 - (NB - 1) * x.R, row_end, live);
                    }
                } else {
                    const int row = rD + slot;
                    const int gc = cD == x.nch - 1 ? x.glast : 64;
                    const bool va = live && lane < gc && row < row_end;
                    if constexpr (RACC && !ACC) {
                        // the first pass starts the row's term afresh (dead steps of the pipeline fill
                        // leave garbage in it); acc * s is exact in fp64, so one fused multiply-add
                        // rounds as the separate product and sum would
                        const double s = (double)half_bits_to_float(g[jb].scale);
                        const double b = cD != 0 ? facc[slot] : 0.0;
                        if constexpr (XS)
                            facc[slot] = b + (double)acc[0] * s * (double)xsv[0];
                        else
                            facc[slot] = __builtin_fma((double)acc[0], s, b);
                    } else {
                        emit<M, ACC, NB, XS>(x, acc, (double)half_bits_to_float(g[jb].scale), xsv, tile, slot,
                                             cD != 0, va ? voff_acc : kOffOff,
                                         live_or_dead(live, ((uint32_t)row * (uint32_t)x.ng + (uint32_t)cD * 64u) * 4u));
                    }
                    if (slot == NB - 1) {  // static: last step of a chunk pass
                        if constexpr (RACC && !ACC && NB % 4 == 0) {
                            // the unit's rows are complete after the last pass. Four rows at a time go
                            // through the tile (row q of the four at tile[64 q + lane]); lane l sums the
                            // terms 4 (l % 16) .. 4 (l % 16) + 3 of row l / 16, then its 16-lane group
                            // (every lane of the group receives the sum), and the group's first lane
                            // stores the row.
                            if (cD == x.nch - 1) {
#pragma unroll
                                for (int q0 = 0; q0 < NB; q0 += 4) {
                                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                                    for (int q = 0; q < 4; ++q) tile[64 * q + lane] = facc[q0 + q];
                                    __builtin_amdgcn_wave_barrier();
                                    const double *t = tile + 64 * (lane >> 4) + 4 * (lane & 15);
                                    const double v = seg_sum_f64((t[0] + t[1]) + (t[2] + t[3]), 16);
                                    const int row = rD + q0 + (lane >> 4);
                                    const bool own = live && (lane & 15) == 0 && row < row_end;
                                    st1(__builtin_bit_cast(uint32_t, (float)v), x.ry, own ? (uint32_t)row * 4u : kOffOff,
                                        0u);
                                }
                                __builtin_amdgcn_wave_barrier();
                            }
                        } else if constexpr (RACC && !ACC) {
                            // units of two rows: lane r gets row r from a reduction over the wave
                            double yl = 0.0;
                            if (cD == x.nch - 1) {
#pragma unroll
                                for (int r = 0; r < NB; ++r) {
                                    const double tot = wave_total_f64(facc[r]);
                                    yl = lane == r ? tot : yl;
                                }
                            }
                            const bool own = live && cD == x.nch - 1 && lane < NB && rD + lane < row_end;
                            st1(__builtin_bit_cast(uint32_t, (float)yl), x.ry, own ? (uint32_t)(rD + lane) * 4u : kOffOff,
                                0u);
                        } else if constexpr (!ACC) {
                            reduce_store<M, NB>(x, red, tile, rD, row_end, live && cD == x.nch - 1);
                        }
                        const bool wrap = live && cD == x.nch - 1;
                        rD = wrap ? rD + NB : rD;
                        cD = live ? (wrap ? 0 : cD + 1) : cD;
                        TG_SCHED_FENCE();
                        // the next decode pass's x slice, ahead of this half-step's prefetches
                        const int gcn = cD == x.nch - 1 ? x.glast : 64;
                        const uint32_t vx = lane < gcn ? voff_x + (uint32_t)cD * 64u * XB : kOffOff;
                        load_x<M, XW>(x, vx, xr);
                        load_xs<M, XS>(x, vx, xsv);
                    }
                }
            }
            TG_SCHED_FENCE();
            // ---- bitmap of step h -> bm[jb] ----
            {
                const int s = h;
                const bool live = s < T;
                if constexpr (!CHUNKED) {
                    const int row0 = row_begin + s * x.R;
                    bm[jb] = ld4s(x.rbm, voff_bm, live_or_dead(live, (uint32_t)row0 * kb));
                } else {
                    const int slot = j % NB;
                    const int gc = cB == x.nch - 1 ? x.glast : 64;
                    bm[jb] = ld4s(x.rbm, lane < gc ? voff_bm : kOffOff,
                                 live_or_dead(live, (uint32_t)(rB + slot) * kb + (uint32_t)cB * 1024u));
                    if (slot == 0) {
                        // the unit's row-index entries, for its first chunk pass
                        ro[(j / NB) & 1] = ld1(x.rro, lane < NB ? (uint32_t)lane * 4u : kOffOff,
                                 live_or_dead(live && cB == 0, (uint32_t)rB * 4u));
                    }
                    if (slot == NB - 1) {
                        const bool wrap = live && cB == x.nch - 1;
                        rB = wrap ? rB + NB : rB;
                        cB = live ? (wrap ? 0 : cB + 1) : cB;
                    }
                }
            }
            TG_SCHED_FENCE();
            // ---- signs of step h - LAG (bitmap bm[(j + 4 - LAG) & 3] -> g[(j + 4 - LAG) & 3]) ----
            {
                const int s = h - LAG;
                const bool live = s >= 0 && s < T;
                if constexpr (!CHUNKED) {
                    const int row0 = row_begin + s * x.R;
                    const uint32_t total = stage_signs<ACC>(x, bm[(j + 4 - LAG) & 3], cur, live, voff_sc,
                                                            (uint32_t)row0 * (uint32_t)x.ng * 2u,
                                                            g[(j + 4 - LAG) & 3]);
                    cur += live ? total : 0u;
                } else {
                    const int slot = (j + U - LAG) % NB;  // step h - LAG within its unit (pass)
                    if (slot == 0) {  // static: a chunk pass starts; its first pass takes the row index
                        const bool first = live && cS == 0;
#pragma unroll
                        for (int r = 0; r < NB; ++r) {
                            const uint32_t v =
                                (uint32_t)__builtin_amdgcn_readlane((int)ro[((j + U - LAG) % U / NB) & 1], r);
                            ccur[r] = first ? v : ccur[r];
                        }
                    }
                    const uint32_t total = stage_signs<ACC>(
                        x, bm[(j + 4 - LAG) & 3], ccur[slot], live, voff_sc,
                        ((uint32_t)(rS + slot) * (uint32_t)x.ng + (uint32_t)cS * 64u) * 2u, g[(j + 4 - LAG) & 3]);
                    ccur[slot] += live ? total : 0u;
                    if (slot == NB - 1) {
                        const bool wrap = live && cS == x.nch - 1;
                        rS = wrap ? rS + NB : rS;
                        cS = live ? (wrap ? 0 : cS + 1) : cS;
                    }
                }
            }
            TG_SCHED_FENCE();
        }
        if (first) {
            wait_x<M, XW>(xr);
            wait_xs<M, XS>(xsv);
        }
    }
}

// Row sums of a finished tile of four one-row steps whose output rows are r0..r3 (wave-uniform; a
// negative row stores nothing): the lane holding tile row i's sum picks ri with selects on scalar
// operands and stores it.
__device__ __forceinline__ void reduce_store_rows(const Ctx &x, const Red &r, const double *tile, int r0, int r1,
                                                  int r2, int r3) {
    __builtin_amdgcn_wave_barrier();
    double t = 0.0;
    for (int e = 0; e < r.epl; ++e)
        if (e < r.cnt) t += tile[r.base + e];
    const uint32_t yv = __builtin_bit_cast(uint32_t, (float)seg_sum_f64(t, r.lpr));
    __builtin_amdgcn_wave_barrier();
    const int lo = (r.rho & 1) ? r1 : r0, hi = (r.rho & 1) ? r3 : r2;
    const int row = (r.rho & 2) ? hi : lo;
    st1(yv, x.ry, r.own && row >= 0 ? (uint32_t)row * 4u : kOffOff, 0u);
}

// Single-chunk GEMVs with one row per step (32 < k/128 <= 64) at m = 1 with fp32 outputs, when the
// descriptor reports rows without non-zero weights (the dead FFN neurons of "Sub-Two-Bit Ternary
// Weight Storage with Table-Free Arithmetic Decoding", abstract: all-zero rows at the same indices in
// gate and up). A row is empty exactly when its index entries are equal, rowoff[r + 1] == rowoff[r]
// (every non-zero weight has one sign), so the index alone finds them: the steps walk the non-empty
// rows only, and each empty row's output is stored as 0 without reading its bitmap or scales. An
// empty row holds no signs, so the sign cursor of the next row is unchanged.
//
// Rows [row_begin, row_end), at most kLiveSegRows of them. First, 64-row windows of the index are
// read (eight windows' loads in flight at a time); a ballot of rowoff[r + 1] != rowoff[r] gives each
// window's mask of non-empty rows, which lane w keeps for window w (two registers), and the empty
// rows' outputs are stored. The step count is then exact, and each step of the pipeline of run_loop
// (bitmap at step h, signs at h - 2, decode at h - 4) takes its row from the lowest set bit of the
// current window's mask; each step's row rides along in a four-slot ring, and the tile's rows go to
// their output rows by scalar selects.
constexpr int kLiveSegRows = 64 * 64;

//
// W80: rows of kW80Groups groups with wide lanes (above) take the same walk, whether or not they have
// empty rows (without any, every row is taken).
template <bool XS, bool W80>
__device__ __forceinline__ void run_loop_live(const Problem &p, int row_begin, int row_end, const char *lds,
                                              double *tile) {
    constexpr int M = 1, NB = 4, U = 4, LAG = 2, XW = W80 ? 20 : 32;
    constexpr uint32_t XB = 4u * XW;
    // the empty asm keeps the lane constants below inside this walk: hoisted to the kernel's entry they
    // would stay live across every other loop of the kernel and spill there
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    Ctx x;
    x.n = p.n;
    x.k = p.k;
    x.ng = p.ng;
    x.nch = p.nch;
    x.G = p.G;
    x.R = p.R;
    x.glast = p.glast;
    x.rbm = make_rsrc(p.codes, p.codes_bytes);
    x.rsg = make_rsrc(reinterpret_cast<const uint8_t *>(p.signs) - 4, p.sign_bytes + 4u);
    x.rsc = make_rsrc(p.scales, (uint32_t)p.n * (uint32_t)p.ng * 2u);
    x.rro = make_rsrc(p.rowoff, (uint32_t)(p.n + 1) * 4u);
    x.rx = make_rsrc(p.x, (uint32_t)p.k);
    x.ry = make_rsrc(p.y, (uint32_t)p.n * 4u);
    x.racc = make_rsrc(p.acc, 0u);
    x.rxs = make_rsrc(p.xs, XS ? (uint32_t)p.ng * 4u : 0u);
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    const uint32_t kb = (uint32_t)(p.k >> 3);
    // group lanes: lane < G takes group `lane`; wide lanes: every lane takes ten presence bytes, in
    // the 16-byte load at the 4-byte boundary below byte 10 l (groups g1 <= g2 of its first and last
    // weight, second group from byte sb)
    const bool act = W80 || lane < x.G;
    const uint32_t voff_bm = !act ? kOffOff : W80 ? (uint32_t)(10 * lane - 2 * (lane & 1)) : (uint32_t)lane * 16u;
    const uint32_t bsh = (uint32_t)(lane & 1) * 16u;
    const int g1 = (80 * lane) >> 7, g2 = (80 * lane + 79) >> 7;
    const int sb = g2 > g1 ? (128 * g2 - 80 * lane) >> 3 : 10;
    const uint32_t voff_sc = !act ? kOffOff : W80 ? (uint32_t)g1 * 2u : (uint32_t)lane * 2u;
    const uint32_t voff_sc2 = (uint32_t)g2 * 2u;
    const uint32_t voff_x = !act ? kOffOff : W80 ? (uint32_t)lane * 80u : (uint32_t)lane * XB;
    const Red red = make_red(NB, 1, W80 ? 64 : x.G, p.rmagic);

    uint32_t xr[M][XW];
    float xsv[M], xsv2[M];
    load_x<M, XW>(x, voff_x, xr);
    if constexpr (W80) {
        load_xs<M, XS>(x, (uint32_t)g1 * 128u, xsv);
        load_xs<M, XS>(x, (uint32_t)g2 * 128u, xsv2);
    } else {
        load_xs<M, XS>(x, voff_x, xsv);
    }
    uint32_t cur = row_index_entry(p, row_begin);
    // masks of the non-empty rows: lane w holds window w (rows row_begin + 64 w .. + 63)
    const int nw = (row_end - row_begin + 63) >> 6;
    uint32_t mlo = 0, mhi = 0;
    int T = 0;
    for (int w0 = 0; w0 < nw; w0 += 8) {
        u32x2 pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = row_begin + 64 * (w0 + i) + lane;
            pr[i] = __builtin_amdgcn_raw_buffer_load_b64(x.rro, w0 + i < nw ? (uint32_t)r * 4u : kOffOff, 0u, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = row_begin + 64 * (w0 + i) + lane;
            const bool in = w0 + i < nw && r < row_end;
            const bool live = in && pr[i].y != pr[i].x;
            const uint64_t m = __builtin_amdgcn_ballot_w64(live);
            T += __builtin_popcountll(m);
            mlo = lane == w0 + i ? (uint32_t)m : mlo;
            mhi = lane == w0 + i ? (uint32_t)(m >> 32) : mhi;
            st1(0u, x.ry, in && !live ? (uint32_t)r * 4u : kOffOff, 0u);
        }
    }
    wait_x<M, XW>(xr);
    wait_xs<M, XS>(xsv);
    if constexpr (W80) wait_xs<M, XS>(xsv2);
    // windows holding non-empty rows (bit w: window w), so that the next one is found without a loop
    const uint64_t nz = __builtin_amdgcn_ballot_w64(lane < nw && (mlo | mhi) != 0u);

    u32x4 bm[4] = {};
    typename std::conditional<W80, SgBufW, SgBuf>::type g[4] = {};
    int rq[4] = {-1, -1, -1, -1};      // row of the step in each pipeline slot (-1: none)
    int trow[NB] = {-1, -1, -1, -1};   // rows of the tile being filled
    int cw = 0;                        // window of the next row
    uint64_t cm = 0;                   // its non-empty rows not taken yet
    uint64_t ahead = nz;               // windows after cw holding non-empty rows (all of nz at first)

    for (int it = 0; U * it - 4 < T; ++it) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int h = U * it + j;
            const int jb = j & 3;
            // ---- decode step h - 4 ----
            {
                trow[j] = rq[jb];
                if constexpr (W80) {
                    int acc1, acc2;
                    decode_w80(bm[jb], g[jb], xr, lds, laneoff, sb, acc1, acc2);
                    // each part times its group scale (and activation group scale), exact in fp64
                    double t1 = (double)acc1 * (double)half_bits_to_float(g[jb].sc1);
                    double t2 = (double)acc2 * (double)half_bits_to_float(g[jb].sc2);
                    if constexpr (XS) {
                        t1 *= (double)xsv[0];
                        t2 *= (double)xsv2[0];
                    }
                    tile[j * 64 + lane] = t1 + t2;
                } else {
                    int acc[M];
                    decode<M, false, false>(bm[jb], g[jb], xr, lds, laneoff, acc);
                    emit<M, false, NB, XS>(x, acc, (double)half_bits_to_float(g[jb].scale), xsv, tile, j, false, kOffOff,
                                           0u);
                }
                if (j == NB - 1) reduce_store_rows(x, red, tile, trow[0], trow[1], trow[2], trow[3]);
            }
            TG_SCHED_FENCE();
            // ---- row of step h (the next non-empty row), then its bitmap ----
            {
                // when the current window is used up, move to the next window with non-empty rows
                // (selects only: every step runs the same instructions); past the last row, row = -1
                const bool adv = cm == 0 && ahead != 0;
                const int nwin = (int)__builtin_ctzll(ahead | (1ull << 63));
                cw = adv ? nwin : cw;
                ahead = adv ? ahead & (ahead - 1) : ahead;
                const uint64_t fresh = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mhi, cw) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane((int)mlo, cw);
                cm = adv ? fresh : cm;
                const int row = h < T ? row_begin + 64 * cw + (int)__builtin_ctzll(cm | (1ull << 63)) : -1;
                cm &= cm - 1;
                rq[jb] = row;
                bm[jb] = ld4s(x.rbm, voff_bm, row >= 0 ? (uint32_t)row * kb : kDeadS);
            }
            TG_SCHED_FENCE();
            // ---- signs of step h - LAG ----
            {
                const int row = rq[(j + 4 - LAG) & 3];
                const bool live = row >= 0;
                const uint32_t soff = (uint32_t)(live ? row : 0) * (uint32_t)x.ng * 2u;
                uint32_t total;
                if constexpr (W80)
                    total = stage_signs_w80(x, bm[(j + 4 - LAG) & 3], bsh, cur, live, voff_sc, voff_sc2, soff,
                                            g[(j + 4 - LAG) & 3]);
                else
                    total = stage_signs<false>(x, bm[(j + 4 - LAG) & 3], cur, live, voff_sc, soff, g[(j + 4 - LAG) & 3]);
                cur += live ? total : 0u;
            }
            TG_SCHED_FENCE();
        }
    }
}

template <int M, bool ACC, int NB, bool XS, bool F16, bool NIB, bool LIVE>
__device__ __forceinline__ void run_problem(const Problem &p, int u0, int u1, const char *lds, double *tile) {
    if (p.nch == 1) {
        if constexpr (LIVE) {
            static_assert(M == 1 && !ACC && !F16 && !NIB, "the live-row walk: m = 1, fp32 outputs");
            const bool wide = p.ng == kW80Groups;
            if (wide || (p.R == 1 && p.empty_rows > 0)) {
                const int row_begin = (u0 - p.unit_begin) * p.rpu;
                const int row_end = min(p.n, (u1 - p.unit_begin) * p.rpu);
                for (int r = row_begin; r < row_end; r += kLiveSegRows) {
                    if (wide)
                        run_loop_live<XS, true>(p, r, min(row_end, r + kLiveSegRows), lds, tile);
                    else
                        run_loop_live<XS, false>(p, r, min(row_end, r + kLiveSegRows), lds, tile);
                }
                return;
            }
        }
        run_loop<M, ACC, NB, false, XS, F16, NIB>(p, u0, u1, lds, tile);
    } else
        if constexpr (M == 1) {
            if (p.nbu == kChunkRows1Fine)
                run_loop<1, ACC, kChunkRows1Fine, true, XS, F16, NIB>(p, u0, u1, lds, tile);
            else if (p.nbu == kChunkRows1Mid)
                run_loop<1, ACC, kChunkRows1Mid, true, XS, F16, NIB>(p, u0, u1, lds, tile);
            else
                run_loop<1, ACC, kChunkRows1, true, XS, F16, NIB>(p, u0, u1, lds, tile);
        } else {
            run_loop<M, ACC, NB, true, XS, F16, NIB>(p, u0, u1, lds, tile);
        }
}

// F16: fp16 activations, f16_waves(M) waves per CU (the 256-byte activation slices need the registers).
// NIB: the nibble-keyed decode (its 32 KB table replaces the byte-keyed tables in LDS).
// LIVE: single-chunk one-row-per-step GEMVs that report rows without non-zeros walk the other rows
// only (m = 1, fp32 outputs); a separate build, so that the kernel without it keeps its registers.
// SHORT: m = 2 launches without chunked rows: 12 waves per CU with two-step units (the tile of
// four-step units for 12 waves would not fit the LDS beside the tables).
template <int M, bool ACC, bool XS, bool F16 = false, bool NIB = false, bool LIVE = false, bool SHORT = false>
__global__ __launch_bounds__((F16 ? 64 * f16_waves(M)
                              : SHORT ? 64 * kBitcosM2ShortWaves
                                      : Cfg<M, TG_FMT_BITCOS>::BLOCK)) void bitcos_gemv_kernel(GroupArgs ga) {
    using C = Cfg<M, TG_FMT_BITCOS>;
    static_assert(!SHORT || (M == 2 && !F16 && !NIB && !LIVE), "the 12-wave build: m = 2, int8 activations");
    // the fp16 kernel uses four-step units at m = 1, 2 (two-step ones were 3-4 % slower at m = 2)
    constexpr int NB = F16 ? 4 : SHORT ? 2 : C::NB;
    constexpr int WAVES = F16 ? f16_waves(M) : SHORT ? kBitcosM2ShortWaves : C::WAVES, BLOCK = 64 * WAVES;
    __shared__ uint4 s_tab[kTabBytes / 16];
    __shared__ double s_tile[ACC ? 1 : WAVES * M * NB * 64];
    // The table fill goes out first (straight into LDS); the wave's unit range and its first GEMV
    // descriptor (two dependent scalar round trips) are read while it is in flight.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if constexpr (NIB)
        load_nib_table<BLOCK>(s_tab);
    else
        load_bitcos_tables<BLOCK, F16>(s_tab);
    TG_SCHED_FENCE();
    int u, u_end, pi;
    wave_range<WAVES>(ga, wave, u, u_end, pi);
    const bool bad0 = ga.table && pi >= ga.count;
    Problem p0 = uniform_problem(launch_problem(ga, bad0 ? 0 : pi));
    lds_copies_landed();
    __syncthreads();
    const char *lds = reinterpret_cast<const char *>(s_tab);
    double *tile = s_tile + (ACC ? 0 : wave * M * NB * 64);
    bool first = true;
    while (u < u_end) {
        if (ga.table && pi >= ga.count) break;  // ranges inconsistent with the table: stop
        const Problem p = first ? p0 : uniform_problem(launch_problem(ga, pi));
        first = false;
        const int u1 = min(u_end, p.unit_begin + p.nunits);
        if (u < u1) run_problem<M, ACC, NB, XS, F16, NIB, LIVE>(p, u, u1, lds, tile);
        u = max(u, u1);
        ++pi;
    }
}

template <int M>
hipError_t launch_m(const GroupArgs &g, int out, hipStream_t s) {
    using C = Cfg<M, TG_FMT_BITCOS>;
    if constexpr (M == 2) {
        if (g.short_units) {
            constexpr int W = kBitcosM2ShortWaves;
            const int blocks = grid_blocks<W>(g);
            if (blocks < 1) return hipErrorInvalidValue;
            if (out == kOutAcc)
                hipLaunchKernelGGL((bitcos_gemv_kernel<2, true, false, false, false, false, true>), dim3(blocks),
                                   dim3(64 * W), 0, s, g);
            else if (out == kOutYxs)
                hipLaunchKernelGGL((bitcos_gemv_kernel<2, false, true, false, false, false, true>), dim3(blocks),
                                   dim3(64 * W), 0, s, g);
            else
                hipLaunchKernelGGL((bitcos_gemv_kernel<2, false, false, false, false, false, true>), dim3(blocks),
                                   dim3(64 * W), 0, s, g);
            return hipGetLastError();
        }
    }
    const int blocks = grid_blocks<C::WAVES>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    const bool live = M == 1 && g.live;
    if (out == kOutAcc)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, true, false>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    else if (out == kOutYxs && live)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, true, false, false, M == 1>), dim3(blocks), dim3(C::BLOCK), 0,
                           s, g);
    else if (out == kOutYxs)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    else if (live)
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, false, false, false, M == 1>), dim3(blocks), dim3(C::BLOCK),
                           0, s, g);
    else
        hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, false>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    return hipGetLastError();
}

template <int M>
hipError_t launch_f16_m(const GroupArgs &g, hipStream_t s) {
    constexpr int W = f16_waves(M);
    const int blocks = grid_blocks<W>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bitcos_gemv_kernel<M, false, false, true>), dim3(blocks), dim3(64 * W), 0, s, g);
    return hipGetLastError();
}

}  // namespace

void gemv_geometry(Problem &p, int fmt, int m, int chunk, bool f16, bool short_units) {
    const int nb = f16 || fmt != TG_FMT_BITCOS ? 4
                   : short_units ? 2
                   : m == 3 ? Cfg<3, TG_FMT_BITCOS>::NB : m == 2 ? Cfg<2, TG_FMT_BITCOS>::NB : Cfg<1, TG_FMT_BITCOS>::NB;
    p.ng = (int32_t)groups_per_row(fmt, p.k);
    p.nch = (p.ng + 63) / 64;
    if (p.nch == 1) {
        p.G = p.ng;
        // The kernels run units of nb steps and reduce a unit's rows at its end, one lane or more per
        // row, so a unit holds at most 64 rows: rows of one or two groups (k = 128, 256) take at most
        // 64 / nb per step and leave the other lanes idle.
        p.R = std::min(64 / p.ng, 64 / nb);
        p.glast = p.ng;
        p.nbu = std::max(1, std::min(nb, 64 / p.R));
    } else {
        p.G = 64;
        p.R = 1;
        p.glast = p.ng - 64 * (p.nch - 1);
        p.nbu = fmt != TG_FMT_BITCOS || m != 1 ? nb
                : chunk == kChunkFine          ? kChunkRows1Fine
                : chunk == kChunkMid           ? kChunkRows1Mid
                                               : kChunkRows1;
    }
    p.rpu = p.nbu * p.R;
    p.gmagic = (65536u + (uint32_t)p.G - 1) / (uint32_t)p.G;
    p.rmagic = (65536u + (uint32_t)p.R - 1) / (uint32_t)p.R;
    p.nunits = (p.n + p.rpu - 1) / p.rpu;
}

hipError_t launch_bitcos_nibble(const GroupArgs &g, int out, hipStream_t s) {
    using C = Cfg<1, TG_FMT_BITCOS>;
    if (g.m != 1 || (out != kOutY && out != kOutAcc)) return hipErrorInvalidValue;
    const int blocks = grid_blocks<C::WAVES>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    if (out == kOutAcc)
        hipLaunchKernelGGL((bitcos_gemv_kernel<1, true, false, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    else
        hipLaunchKernelGGL((bitcos_gemv_kernel<1, false, false, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_bitcos_f16(const GroupArgs &g, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_f16_m<1>(g, s);
        case 2: return launch_f16_m<2>(g, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bitcos(const GroupArgs &g, int out, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_m<1>(g, out, s);
        case 2: return launch_m<2>(g, out, s);
        case 3: return launch_m<3>(g, out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
