// Ternary GEMV for the fixed-size group codes, on gfx950 (int8 activations, fp16 group scales):
//   five-trit -- five ternary weights per byte as base-3 digits (digit = weight + 1, first weight least
//                significant), 26 bytes per 128-weight group ("Breaking the 1.58-bit Barrier for
//                Ternary LLMs", Sec. I; "Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic
//                Decoding", abstract);
//   2-bit     -- four weights per byte, code = weight + 1 in two bits, first weight lowest (the
//                "2-bit packing" of Table I in the first paper);
//   t5b       -- the five-trit code in aligned 32-byte blocks of 160 weights with one scale per tensor
//                (the second paper's t5b): a lane owns one block, its 160 activation bytes and its
//                block sum; the epilogue applies the tensor scale instead of a group scale.
//
// Same persistent work geometry and unit-end reduction as the BITCOS kernel (gemv_pipeline.h): a lane
// owns one group per step. A group's code bytes sit at a fixed place, so there is no dependent load:
// the codes of step h are loaded while step h - 3 is decoded (four code buffers rotate in a loop body
// of four steps). Decode is one LDS table read per code byte:
//   2-bit:     byte -> its 4 weights as int8 (one v_dot4_i32_i8 against 4 activation bytes);
//   five-trit: byte -> weights 0..3 as int8 plus weight 4 in a second word. The activation bytes are
//              permuted once per slice into matching words: xa[j] = x[5j .. 5j+3] and, for each run
//              of four code bytes, xb[q] = the four activations of their fifth weights, so a run of
//              four bytes (20 weights) takes five dot products.
// The tables are kept in bank-spread copies (lane l reads copy l % 64 or l % 32), so table reads do
// not conflict; a copy's address is one byte-permute of the code word.
#include <algorithm>

#include "gemv_pipeline.h"

namespace tg {
namespace {

// LDS tables: 256 entries, spread so that lane l reads its own copy: 2-bit entries are 4 bytes (64
// copies, 256 bytes per entry value), five-trit entries 8 bytes (32 copies).
constexpr uint32_t kLutBytes = 256 * 256;

// Each entry is stored as the 16 bytes a lane copies into LDS: four copies of a 2-bit entry, two of a
// five-trit one.
struct alignas(16) FixedTables {
    uint32_t b2[256][4];  // 2-bit: code byte -> 4 int8 weights
    uint32_t t5[256][4];  // five-trit: code byte -> weights 0..3 as int8, weight 4 as int8 in word 1
};

constexpr FixedTables make_fixed_tables() {
    FixedTables t{};
    for (uint32_t b = 0; b < 256; ++b) {
        uint32_t v = 0;
        for (uint32_t i = 0; i < 4; ++i) {
            const uint32_t c = (b >> (2 * i)) & 3u;          // code 3 is invalid; read as weight 0
            const uint32_t w = c == 3 ? 0u : (c + 255u) & 0xFFu;  // c - 1 as int8
            v |= w << (8 * i);
        }
        t.b2[b][0] = t.b2[b][1] = t.b2[b][2] = t.b2[b][3] = v;
        uint32_t d = b < 243 ? b : 121;  // invalid bytes read as five zero weights
        uint32_t lo = 0, hi = 0;
        for (uint32_t i = 0; i < 5; ++i) {
            const uint32_t w = (d % 3 + 255u) & 0xFFu;  // digit - 1 as int8
            d /= 3;
            if (i < 4)
                lo |= w << (8 * i);
            else
                hi = w;
        }
        t.t5[b][0] = t.t5[b][2] = lo;
        t.t5[b][1] = t.t5[b][3] = hi;
    }
    return t;
}

__device__ const FixedTables kFixedTables = make_fixed_tables();

template <int FMT>
struct Fmt;
template <>
struct Fmt<TG_FMT_2BIT> {
    static constexpr uint32_t kGroupBytes = 32;
    static constexpr int kXWords = 32;      // activation words per lane and row of x
    static constexpr uint32_t kXBytes = 128;  // activation bytes of one group
};
template <>
struct Fmt<TG_FMT_5TRIT> {
    static constexpr uint32_t kGroupBytes = 26;
    static constexpr int kXWords = 33;  // xa[0..25], xb[0..6]
    static constexpr uint32_t kXBytes = 128;
};
template <>
struct Fmt<TG_FMT_T5B> {
    static constexpr uint32_t kGroupBytes = 32;  // a 160-weight block
    static constexpr int kXWords = 40;           // xa[0..31], xb[0..7]
    static constexpr uint32_t kXBytes = 160;
};

// One step's codes: eight words from the dword-aligned address at or below the group start, the
// bit shift that realigns them (five-trit groups start on 2-byte boundaries), and the scale.
struct CodeBuf {
    u32x4 c[2];
    uint32_t sh;
    uint16_t scale;
};

// The lane's activation words for its group column: plain bytes for 2-bit, the permuted words for
// five-trit (see the file comment). ARITH (2-bit): each 16-byte run transposed as a 4 x 4 byte matrix,
// so that word 4d + i holds the activations of code i of the four code bytes of code dword d.
template <int FMT, int M, bool ARITH = false>
__device__ __forceinline__ void load_xf(const Ctx &x, uint32_t voff, uint32_t (&xf)[M][Fmt<FMT>::kXWords]) {
    if constexpr (FMT == TG_FMT_T5B) {
        // the block's 160 activation bytes (ten 16-byte loads; past k they meet padding weights of
        // zero, so whatever they read adds nothing), then the five-trit permutation over 32 bytes
        uint32_t xr[M][40];
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
#pragma unroll
            for (int j = 0; j < 10; ++j) {
                const u32x4 v = ld4(x.rx, voff + 16u * j, (uint32_t)(mi * x.k));
                xr[mi][4 * j] = v.x;
                xr[mi][4 * j + 1] = v.y;
                xr[mi][4 * j + 2] = v.z;
                xr[mi][4 * j + 3] = v.w;
            }
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            auto xw = [&](int w) -> uint32_t { return w < 40 ? xr[mi][w] : 0u; };
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int w = (5 * j) >> 2, o = (5 * j) & 3;
                xf[mi][j] = o == 0 ? xw(w) : __builtin_amdgcn_alignbit(xw(w + 1), xw(w), 8 * o);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t lo = __builtin_amdgcn_perm(xw(5 * q + 2), xw(5 * q + 1), 0x0C0C0500u);
                const uint32_t hi = __builtin_amdgcn_perm(xw(5 * q + 4), xw(5 * q + 3), 0x0C0C0702u);
                xf[mi][32 + q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
        }
        return;
    }
    uint32_t xr[M][32];
    load_x<M>(x, voff, xr);
    if constexpr (FMT == TG_FMT_2BIT && ARITH) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t r0 = xr[mi][4 * d], r1 = xr[mi][4 * d + 1], r2 = xr[mi][4 * d + 2], r3 = xr[mi][4 * d + 3];
                const uint32_t a = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
                const uint32_t b = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
                const uint32_t c = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
                const uint32_t e = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
                xf[mi][4 * d] = __builtin_amdgcn_perm(c, a, 0x05040100u);      // byte 0 of r0..r3
                xf[mi][4 * d + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // byte 1
                xf[mi][4 * d + 2] = __builtin_amdgcn_perm(e, b, 0x05040100u);  // byte 2
                xf[mi][4 * d + 3] = __builtin_amdgcn_perm(e, b, 0x07060302u);  // byte 3
            }
    } else if constexpr (FMT == TG_FMT_2BIT) {
#pragma unroll
        for (int mi = 0; mi < M; ++mi)
#pragma unroll
            for (int j = 0; j < 32; ++j) xf[mi][j] = xr[mi][j];
    } else {
#pragma unroll
        for (int mi = 0; mi < M; ++mi) {
            auto xw = [&](int w) -> uint32_t { return w < 32 ? xr[mi][w] : 0u; };
#pragma unroll
            for (int j = 0; j < 26; ++j) {
                const int w = (5 * j) >> 2, o = (5 * j) & 3;
                xf[mi][j] = o == 0 ? xw(w) : __builtin_amdgcn_alignbit(xw(w + 1), xw(w), 8 * o);
            }
#pragma unroll
            for (int q = 0; q < 7; ++q) {
                // activation bytes 20q+4, 20q+9, 20q+14, 20q+19: byte 0 of word 5q+1, byte 1 of 5q+2,
                // byte 2 of 5q+3, byte 3 of 5q+4 (zero past the group)
                const uint32_t lo = __builtin_amdgcn_perm(xw(5 * q + 2), xw(5 * q + 1), 0x0C0C0500u);
                const uint32_t hi = __builtin_amdgcn_perm(xw(5 * q + 4), xw(5 * q + 3), 0x0C0C0702u);
                xf[mi][26 + q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
        }
    }
}

template <int FMT, int M>
__device__ __forceinline__ void wait_xf(const uint32_t (&xf)[M][Fmt<FMT>::kXWords]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi)
#pragma unroll
        for (int j = 0; j < Fmt<FMT>::kXWords; ++j) asm volatile("" ::"v"(xf[mi][j]));
}

// int32 sums of the lane's 128 weights times x, per activation row.
template <int FMT, int M>
__device__ __forceinline__ void decode_fixed(const CodeBuf &b, const uint32_t (&xf)[M][Fmt<FMT>::kXWords],
                                             const char *lds, uint32_t laneoff, int (&acc)[M]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) acc[mi] = 0;
    uint32_t w[8] = {b.c[0].x, b.c[0].y, b.c[0].z, b.c[0].w, b.c[1].x, b.c[1].y, b.c[1].z, b.c[1].w};
    if constexpr (FMT == TG_FMT_2BIT) {
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // (byte << 8) | (lane % 64) * 4: lane's copy of the byte's entry
                const uint32_t a = __builtin_amdgcn_perm(w[d], laneoff, 0x0C0C0000u | ((4u + i) << 8));
                const uint32_t e = *reinterpret_cast<const uint32_t *>(lds + a);
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(e, xf[mi][4 * d + i], acc[mi]);
            }
    } else {
        // five-trit: realign (the group's 26 bytes start at bit sh, 0 or 16, of w[0]); t5b blocks of
        // 32 bytes are aligned
        constexpr int kBytes = FMT == TG_FMT_T5B ? 32 : 26;
        constexpr int kRuns = (kBytes + 3) / 4;
        if constexpr (FMT == TG_FMT_5TRIT) {
#pragma unroll
            for (int d = 0; d < 7; ++d) w[d] = __builtin_amdgcn_alignbit(w[d + 1], w[d], b.sh);
        }
#pragma unroll
        for (int q = 0; q < kRuns; ++q) {
            uint32_t hi4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * q + i;  // code byte
                if (j < kBytes) {
                    const uint32_t a = __builtin_amdgcn_perm(w[q], laneoff, 0x0C0C0000u | ((4u + i) << 8));
                    const uint2 e = *reinterpret_cast<const uint2 *>(lds + a);
#pragma unroll
                    for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(e.x, xf[mi][j], acc[mi]);
                    hi4[i] = e.y;
                } else {
                    hi4[i] = 0;
                }
            }
            const uint32_t lo = __builtin_amdgcn_perm(hi4[1], hi4[0], 0x0C0C0400u);
            const uint32_t hi = __builtin_amdgcn_perm(hi4[3], hi4[2], 0x0C0C0400u);
            const uint32_t w4 = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
#pragma unroll
            for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(w4, xf[mi][kBytes + q], acc[mi]);
        }
    }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Table-free decode of the five-trit code ("Sub-Two-Bit Ternary Weight Storage with Table-Free
// Arithmetic Decoding", abstract: the depth-one arithmetic decode). Digit i of a code byte c is
// floor(c / 3^i) - 3 floor(c / 3^(i+1)); every floor comes straight from c with one multiply and one
// shift (f = (c * M) >> s with M / 2^s just above 3^-i, exact for every c < 243; all products stay
// below 2^16), so no digit waits for another. Two codes are decoded together, one in each 16-bit half
// of cp (c in the half's low byte); d[i] holds digit i of both.
__device__ __forceinline__ void t5_digit_pairs(uint32_t cp, u16x2 (&d)[5]) {
    const u16x2 c = __builtin_bit_cast(u16x2, cp);
    const u16x2 f1 = (c * (unsigned short)171) >> (unsigned short)9;   // floor(c / 3)
    const u16x2 f2 = (c * (unsigned short)57) >> (unsigned short)9;    // floor(c / 9)
    const u16x2 f3 = (c * (unsigned short)19) >> (unsigned short)9;    // floor(c / 27)
    const u16x2 f4 = (c * (unsigned short)203) >> (unsigned short)14;  // floor(c / 81)
    const unsigned short m3 = (unsigned short)0xFFFDu;                 // -3 modulo 2^16
    d[0] = f1 * m3 + c;
    d[1] = f2 * m3 + f1;
    d[2] = f3 * m3 + f2;
    d[3] = f4 * m3 + f3;
    d[4] = f4;
}

// Sums of the lane's weights times x with the table-free decode: the digits or codes (0, 1, 2) are
// contracted as they are and sx, the sum of the group's activations, is taken off once, since
// weight = digit - 1 = code - 1.
// Five-trit: four code bytes give four words of digits 0..3 (one per code, against xa[j]) and one
// word of their fifth digits (against xb[q]), as in the table path.
// 2-bit (the shift, mask and subtract decode, without expanding a code to its weight): code i of the
// four bytes of code dword d is (w >> 2i) & 0x03030303, contracted against the transposed activation
// word 4d + i.
template <int FMT, int M>
__device__ __forceinline__ void decode_fixed_arith(const CodeBuf &b, const uint32_t (&xf)[M][Fmt<FMT>::kXWords],
                                                   const int (&sx)[M], int (&acc)[M]) {
    if constexpr (FMT == TG_FMT_2BIT) {
        const uint32_t w[8] = {b.c[0].x, b.c[0].y, b.c[0].z, b.c[0].w, b.c[1].x, b.c[1].y, b.c[1].z, b.c[1].w};
#pragma unroll
        for (int mi = 0; mi < M; ++mi) acc[mi] = -sx[mi];
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c = (w[d] >> (2 * i)) & 0x03030303u;
#pragma unroll
                for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(c, xf[mi][4 * d + i], acc[mi]);
            }
    } else {
        static_assert(FMT == TG_FMT_5TRIT || FMT == TG_FMT_T5B, "five-trit codes");
        constexpr int kBytes = FMT == TG_FMT_T5B ? 32 : 26;
        constexpr int kRuns = (kBytes + 3) / 4;
        uint32_t w[8] = {b.c[0].x, b.c[0].y, b.c[0].z, b.c[0].w, b.c[1].x, b.c[1].y, b.c[1].z, b.c[1].w};
        if constexpr (FMT == TG_FMT_5TRIT) {
#pragma unroll
            for (int d = 0; d < 7; ++d) w[d] = __builtin_amdgcn_alignbit(w[d + 1], w[d], b.sh);
        }
#pragma unroll
        for (int mi = 0; mi < M; ++mi) acc[mi] = -sx[mi];
#pragma unroll
        for (int q = 0; q < kRuns; ++q) {
            uint32_t fifth[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // codes 4q + 2h and 4q + 2h + 1 into the low bytes of the two halves
                const uint32_t cp = __builtin_amdgcn_perm(w[q], w[q], h ? 0x0C030C02u : 0x0C010C00u);
                u16x2 dg[5];
                t5_digit_pairs(cp, dg);
                const uint32_t e0 = __builtin_bit_cast(uint32_t, dg[0]), e1 = __builtin_bit_cast(uint32_t, dg[1]);
                const uint32_t e2 = __builtin_bit_cast(uint32_t, dg[2]), e3 = __builtin_bit_cast(uint32_t, dg[3]);
                const uint32_t t01 = __builtin_amdgcn_perm(e1, e0, 0x06040200u);  // d0 lo, d0 hi, d1 lo, d1 hi
                const uint32_t t23 = __builtin_amdgcn_perm(e3, e2, 0x06040200u);  // d2 lo, d2 hi, d3 lo, d3 hi
                fifth[h] = __builtin_bit_cast(uint32_t, dg[4]);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int j = 4 * q + 2 * h + c;  // code byte
                    if (j < kBytes) {
                        const uint32_t dw = __builtin_amdgcn_perm(t23, t01, c ? 0x07050301u : 0x06040200u);
#pragma unroll
                        for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(dw, xf[mi][j], acc[mi]);
                    }
                }
            }
            // fifth digits of the run's four codes (a five-trit group's last run reaches two bytes of the
            // next group, whose digits meet activation positions past 127, which are zero)
            const uint32_t w4 = __builtin_amdgcn_perm(fifth[1], fifth[0], 0x06040200u);
#pragma unroll
            for (int mi = 0; mi < M; ++mi) acc[mi] = dot4(w4, xf[mi][kBytes + q], acc[mi]);
        }
    }
}

// Sum of the activations of the lane's group (the words of xf hold each of them once).
template <int FMT, int M>
__device__ __forceinline__ void xf_sums(const uint32_t (&xf)[M][Fmt<FMT>::kXWords], int (&sx)[M]) {
#pragma unroll
    for (int mi = 0; mi < M; ++mi) {
        int s = 0;
#pragma unroll
        for (int j = 0; j < Fmt<FMT>::kXWords; ++j) s = dot4(0x01010101u, xf[mi][j], s);
        sx[mi] = s;
    }
}

// Pipeline over the steps of units [u0, u1) of one GEMV: in half-step h, step h - 3 is decoded and
// the codes of step h are loaded (four code buffers rotate with the four half-steps of the loop
// body). Every stage runs on every half-step; dead steps use dead offsets and decode into tile slots
// a live step overwrites first.
template <int FMT, int M, bool ACC, int NB, bool CHUNKED, bool XS, bool ARITH>
__device__ __forceinline__ void run_fixed(const Problem &p, int u0, int u1, const char *lds, double *tile) {
    constexpr uint32_t GB = Fmt<FMT>::kGroupBytes;
    constexpr int XW = Fmt<FMT>::kXWords;
    const int lane = threadIdx.x & 63;
    // weight scale of a group: its fp16 scale, or the tensor scale of t5b
    const double tscale = (double)p.tscale;
    auto gscale = [&](const CodeBuf &b) -> double {
        return FMT == TG_FMT_T5B ? tscale : (double)half_bits_to_float(b.scale);
    };
    Ctx x;
    x.n = p.n;
    x.k = p.k;
    x.ng = p.ng;
    x.nch = p.nch;
    x.G = p.G;
    x.R = p.R;
    x.glast = p.glast;
    // a five-trit group's last load reaches up to 6 bytes past its 26; the packed buffer keeps at least
    // 16 zero bytes after the codes section, so the resource covers them
    x.rbm = make_rsrc(p.codes, p.codes_bytes + 16u);
    // t5b has no per-group scales: its tensor scale comes with the GEMV
    x.rsc = make_rsrc(p.scales, ACC || FMT == TG_FMT_T5B ? 0u : (uint32_t)p.n * (uint32_t)p.ng * 2u);
    x.rx = make_rsrc(p.x, (uint32_t)M * (uint32_t)p.k);
    x.ry = make_rsrc(p.y, ACC ? 0u : (uint32_t)M * (uint32_t)p.n * 4u);
    x.racc = make_rsrc(p.acc, ACC ? (uint32_t)M * (uint32_t)p.n * (uint32_t)p.ng * 4u : 0u);
    x.rxs = make_rsrc(p.xs, XS ? (uint32_t)M * (uint32_t)p.ng * 4u : 0u);
    const uint32_t laneoff = FMT == TG_FMT_2BIT ? (uint32_t)lane << 2 : (uint32_t)(lane & 31) << 3;
    const int rpu = p.rpu;
    const int row_begin = (u0 - p.unit_begin) * rpu;
    const int row_end = min(p.n, (u1 - p.unit_begin) * rpu);
    const uint32_t ng = (uint32_t)p.ng;

    uint32_t xf[M][XW];
    float xsv[M];  // activation group scales of the lane's group (1 without them)
    int T;
    uint32_t voff_sc, voff_acc, voff_x, lane_grp;  // lane_grp: the lane's group index offset in a step
    bool act;
    Red red;
    if constexpr (!CHUNKED) {
        const int ql = (int)(((uint32_t)lane * p.gmagic) >> 16);
        const int jl = lane - ql * x.G;
        act = lane < x.R * x.G;
        lane_grp = (uint32_t)lane;  // ql * ng + jl with ng = G
        voff_sc = act ? (uint32_t)lane * 2u : kOffOff;
        voff_acc = act ? (uint32_t)lane * 4u : kOffOff;
        voff_x = act ? (uint32_t)jl * Fmt<FMT>::kXBytes : kOffOff;
        T = (u1 - u0) * NB;
        red = make_red(NB * x.R, x.R, x.G, p.rmagic);
    } else {
        act = true;
        lane_grp = (uint32_t)lane;
        voff_sc = (uint32_t)lane * 2u;
        voff_acc = (uint32_t)lane * 4u;
        voff_x = (uint32_t)lane * Fmt<FMT>::kXBytes;
        T = (u1 - u0) * NB * x.nch;
        red = make_red(NB, 1, 64, p.rmagic);
    }
    load_xf<FMT, M, ARITH>(x, voff_x, xf);
    load_xs<M, XS>(x, voff_x, xsv);
    wait_xf<FMT, M>(xf);
    wait_xs<M, XS>(xsv);
    int sx[M];  // table-free decode: the group's activation sum (recomputed when a pass reloads xf)
    if constexpr (ARITH) xf_sums<FMT, M>(xf, sx);

    CodeBuf cb[4] = {};
    int cD = 0, rD = row_begin, cB = 0, rB = row_begin;

    for (int it = 0; 4 * it - 3 < T; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = 4 * it + j;
            // ---- decode step h - 3 (buffer cb[(j + 1) & 3]) ----
            {
                const int s = h - 3;
                const bool live = s >= 0 && s < T;
                const CodeBuf &b = cb[(j + 1) & 3];
                int acc[M];
                const int slot = (j + 1) % NB;
                if constexpr (ARITH) {
                    if constexpr (CHUNKED) {
                        if (slot == 0) xf_sums<FMT, M>(xf, sx);  // static: first step of a pass
                    }
                    decode_fixed_arith<FMT, M>(b, xf, sx, acc);
                } else {
                    decode_fixed<FMT, M>(b, xf, lds, laneoff, acc);
                }
                if constexpr (!CHUNKED) {
                    const int row0 = row_begin + s * x.R;
                    const bool va = live && act && row0 + (int)(((uint32_t)lane * p.gmagic) >> 16) < row_end;
                    emit<M, ACC, NB, XS>(x, acc, gscale(b), xsv, tile, slot, false, va ? voff_acc : kOffOff,
                                     live_or_dead(live, (uint32_t)row0 * ng * 4u));
                    if constexpr (!ACC) {
                        if (slot == NB - 1) reduce_store<M, NB>(x, red, tile, row0 - (NB - 1) * x.R, row_end, live);
                    }
                } else {
                    const int row = rD + slot;
                    const int gc = cD == x.nch - 1 ? x.glast : 64;
                    const bool va = live && lane < gc && row < row_end;
                    emit<M, ACC, NB, XS>(x, acc, gscale(b), xsv, tile, slot, cD != 0, va ? voff_acc : kOffOff,
                                     live_or_dead(live, ((uint32_t)row * ng + (uint32_t)cD * 64u) * 4u));
                    if (slot == NB - 1) {  // static: last step of a chunk pass
                        if constexpr (!ACC) reduce_store<M, NB>(x, red, tile, rD, row_end, live && cD == x.nch - 1);
                        const bool wrap = live && cD == x.nch - 1;
                        rD = wrap ? rD + NB : rD;
                        cD = live ? (wrap ? 0 : cD + 1) : cD;
                        TG_SCHED_FENCE();
                        const int gcn = cD == x.nch - 1 ? x.glast : 64;
                        const uint32_t vx =
                            lane < gcn ? voff_x + (uint32_t)cD * (64u * Fmt<FMT>::kXBytes) : kOffOff;
                        load_xf<FMT, M, ARITH>(x, vx, xf);
                        load_xs<M, XS>(x, vx, xsv);
                    }
                }
            }
            TG_SCHED_FENCE();
            // ---- codes and scale of step h -> cb[j] ----
            {
                const int s = h;
                const bool live = s < T;
                uint32_t grp, soff_sc;  // global group index of the lane's group, scale offset
                bool la;
                if constexpr (!CHUNKED) {
                    const int row0 = row_begin + s * x.R;
                    grp = (uint32_t)row0 * ng + lane_grp;
                    soff_sc = (uint32_t)row0 * ng * 2u;
                    la = live && act;
                } else {
                    const int slot = j % NB;
                    const int gc = cB == x.nch - 1 ? x.glast : 64;
                    grp = (uint32_t)(rB + slot) * ng + (uint32_t)cB * 64u + lane_grp;
                    soff_sc = ((uint32_t)(rB + slot) * ng + (uint32_t)cB * 64u) * 2u;
                    la = live && lane < gc;
                    if (slot == NB - 1) {
                        const bool wrap = live && cB == x.nch - 1;
                        rB = wrap ? rB + NB : rB;
                        cB = live ? (wrap ? 0 : cB + 1) : cB;
                    }
                }
                const uint32_t off = grp * GB;
                const uint32_t a4 = la ? off & ~3u : kOffOff;
                cb[j].c[0] = ld4(x.rbm, a4, 0u);
                cb[j].c[1] = ld4(x.rbm, a4 + 16u, 0u);
                cb[j].sh = (off & 3u) << 3;
                // 2-bit scales with the non-temporal policy (one instruction reads each 128-byte line
                // whole: +0.6 % on the layer set; five-trit unchanged, so it keeps the default)
                const uint32_t sdo = live_or_dead(live, soff_sc), svo = la ? voff_sc : kOffOff;
                cb[j].scale = ACC || FMT == TG_FMT_T5B ? (uint16_t)0
                              : FMT == TG_FMT_2BIT    ? ldhs(x.rsc, svo, sdo)
                                                      : ldh(x.rsc, svo, sdo);
            }
            TG_SCHED_FENCE();
        }
    }
}

// ARITH: the table-free decode of the five-trit and 2-bit codes (no LDS table, so no table fill either).
template <int FMT, int M, bool ACC, bool XS, bool ARITH = false>
__global__ __launch_bounds__((Cfg<M, FMT>::BLOCK)) void fixed_gemv_kernel(GroupArgs ga) {
    using C = Cfg<M, FMT>;
    constexpr int NB = C::NB, WAVES = C::WAVES, BLOCK = C::BLOCK;
    __shared__ uint4 s_lut[ARITH ? 1 : kLutBytes / 16];
    __shared__ double s_tile[ACC ? 1 : WAVES * M * NB * 64];
    // The table fill goes out first, straight from global memory into LDS (global_load_lds_dwordx4:
    // lane l of a wave writes its 16 bytes at the wave's LDS base + 16 l; 1 KB per instruction holds
    // the copies of four code bytes); the wave's unit range and first GEMV descriptor (two dependent
    // scalar round trips) are read while it is in flight.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if constexpr (!ARITH) {
        constexpr int kChunks = (int)(kLutBytes / 1024);
        const int lane = (int)(threadIdx.x & 63);
        const uint4 *src = reinterpret_cast<const uint4 *>(FMT == TG_FMT_2BIT ? &kFixedTables.b2[0][0]
                                                                             : &kFixedTables.t5[0][0]);
        typedef __attribute__((address_space(3))) void *lds_ptr;
        for (int c = wave; c < kChunks; c += WAVES)
            __builtin_amdgcn_global_load_lds(src + 4 * c + (lane >> 4), (lds_ptr)(s_lut + 64 * c), 16, 0, 0);
    }
    TG_SCHED_FENCE();
    int u, u_end, pi;
    wave_range<WAVES>(ga, wave, u, u_end, pi);
    const bool bad0 = ga.table && pi >= ga.count;
    const Problem p0 = uniform_problem(launch_problem(ga, bad0 ? 0 : pi));
    if constexpr (!ARITH) {
        lds_copies_landed();
        __syncthreads();
    }
    const char *lds = reinterpret_cast<const char *>(s_lut);
    double *tile = s_tile + (ACC ? 0 : wave * M * NB * 64);
    bool first = true;
    while (u < u_end) {
        if (ga.table && pi >= ga.count) break;  // ranges inconsistent with the table: stop
        const Problem p = first ? p0 : uniform_problem(launch_problem(ga, pi));
        first = false;
        const int u1 = min(u_end, p.unit_begin + p.nunits);
        if (u < u1) {
            if (p.nch == 1)
                run_fixed<FMT, M, ACC, NB, false, XS, ARITH>(p, u, u1, lds, tile);
            else
                run_fixed<FMT, M, ACC, NB, true, XS, ARITH>(p, u, u1, lds, tile);
        }
        u = max(u, u1);
        ++pi;
    }
}

template <int FMT, int M>
hipError_t launch_fixed_m(const GroupArgs &g, int out, hipStream_t s) {
    using C = Cfg<M, FMT>;
    const int blocks = grid_blocks<C::WAVES>(g);
    if (blocks < 1) return hipErrorInvalidValue;
    if (out == kOutAcc)
        hipLaunchKernelGGL((fixed_gemv_kernel<FMT, M, true, false>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    else if (out == kOutYxs) {
        if constexpr (FMT == TG_FMT_T5B)
            return hipErrorInvalidValue;  // t5b has no activation group scales
        else
            hipLaunchKernelGGL((fixed_gemv_kernel<FMT, M, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    }
    else
        hipLaunchKernelGGL((fixed_gemv_kernel<FMT, M, false, false>), dim3(blocks), dim3(C::BLOCK), 0, s, g);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fixed(const GroupArgs &g, int out, hipStream_t s) {
    switch (g.m) {
        case 1: return launch_fixed_m<FMT, 1>(g, out, s);
        case 2: return launch_fixed_m<FMT, 2>(g, out, s);
        case 3: return launch_fixed_m<FMT, 3>(g, out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_t5(const GroupArgs &g, int out, hipStream_t s) {
    return launch_fixed<TG_FMT_5TRIT>(g, out, s);
}

hipError_t launch_b2(const GroupArgs &g, int out, hipStream_t s) {
    return launch_fixed<TG_FMT_2BIT>(g, out, s);
}

hipError_t launch_table_free(int fmt, const GroupArgs &g, int out, hipStream_t s) {
    if (g.m != 1 || (out != kOutY && out != kOutAcc) ||
        (fmt != TG_FMT_5TRIT && fmt != TG_FMT_T5B && fmt != TG_FMT_2BIT))
        return hipErrorInvalidValue;
    if (fmt == TG_FMT_2BIT) {
        using C = Cfg<1, TG_FMT_2BIT>;
        const int blocks = grid_blocks<C::WAVES>(g);
        if (blocks < 1) return hipErrorInvalidValue;
        if (out == kOutAcc)
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_2BIT, 1, true, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s,
                               g);
        else
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_2BIT, 1, false, false, true>), dim3(blocks), dim3(C::BLOCK), 0,
                               s, g);
    } else if (fmt == TG_FMT_5TRIT) {
        using C = Cfg<1, TG_FMT_5TRIT>;
        const int blocks = grid_blocks<C::WAVES>(g);
        if (blocks < 1) return hipErrorInvalidValue;
        if (out == kOutAcc)
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_5TRIT, 1, true, false, true>), dim3(blocks), dim3(C::BLOCK), 0,
                               s, g);
        else
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_5TRIT, 1, false, false, true>), dim3(blocks), dim3(C::BLOCK),
                               0, s, g);
    } else {
        using C = Cfg<1, TG_FMT_T5B>;
        const int blocks = grid_blocks<C::WAVES>(g);
        if (blocks < 1) return hipErrorInvalidValue;
        if (out == kOutAcc)
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_T5B, 1, true, false, true>), dim3(blocks), dim3(C::BLOCK), 0, s,
                               g);
        else
            hipLaunchKernelGGL((fixed_gemv_kernel<TG_FMT_T5B, 1, false, false, true>), dim3(blocks), dim3(C::BLOCK), 0,
                               s, g);
    }
    return hipGetLastError();
}

hipError_t launch_t5b(const GroupArgs &g, int out, hipStream_t s) {
    if (out == kOutYxs) return hipErrorInvalidValue;  // no activation group scales for t5b
    return launch_fixed<TG_FMT_T5B>(g, out, s);
}

}  // namespace tg
