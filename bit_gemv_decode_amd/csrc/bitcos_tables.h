// LDS decode tables of the BITCOS kernels ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec.
// II-A and Fig. 4: the deposit of compact signs onto present positions, done here by lookup).
//
// Entry (pb, s) holds the 8 ternary weights, as int8, of presence byte pb with compact signs s (its
// popcount(pb) sign bits, first sign lowest; a set sign bit gives -1, a clear one +1, absent
// positions 0): 3^8 = 6561 entries of 8 bytes. The entries of one presence byte form a block of
// 2^popcount(pb) entries, and blocks are laid out in decreasing size, so each block starts at a
// multiple of its own size: the LDS address of an entry is (window & mask) | base, where window
// holds the compact signs at bits 3 and up, mask = (2^popcount(pb) - 1) << 3 and base is the block's
// LDS byte address. (mask, base) per presence byte come from a 256-entry table kept in 32 copies,
// one per LDS bank: lane l reads copy l % 32 at (pb << 8) | (l % 32) << 3, so these reads never
// conflict.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace tg {
namespace {

constexpr int kEntries = 6561;                 // sum over presence bytes of 2^popcount = 3^8
constexpr uint32_t kInfoBytes = 256 * 32 * 8;  // per-byte (mask, base) in 32 bank-spread copies
constexpr uint32_t kEntOff = kInfoBytes;       // LDS byte offset of the entry table
constexpr uint32_t kEntBytes = kEntries * 8;
constexpr uint32_t kTabBytes = (kEntOff + kEntBytes + 255) / 256 * 256;

struct alignas(16) Tables {
    uint64_t ent[kEntries + 1];  // padded to an even count for 16-byte copies
    uint32_t info[256][2];       // per presence byte: mask (popcount ones, shifted left 3), LDS base
};

constexpr int popc8(uint32_t v) {
    int c = 0;
    for (int i = 0; i < 8; ++i) c += (v >> i) & 1;
    return c;
}

// Blocks of entries in decreasing size: every block then starts at a multiple of its own size, so
// a block's base has zero bits where (window & mask) has its ones. Entry bytes are `pos` for +1 and
// `neg` for -1: the int8 weights (0x01, 0xFF), or for fp16 activations the high bytes of the binary16
// weights +1.0 and -1.0 (0x3C, 0xBC; their low bytes are zero).
constexpr Tables make_tables(uint64_t pos = 0x01, uint64_t neg = 0xFF) {
    Tables t{};
    uint32_t e = 0;
    for (int c = 8; c >= 0; --c) {
        for (uint32_t pb = 0; pb < 256; ++pb) {
            if (popc8(pb) != c) continue;
            t.info[pb][0] = ((1u << c) - 1u) << 3;
            t.info[pb][1] = kEntOff + 8 * e;
            for (uint32_t sc = 0; sc < (1u << c); ++sc) {
                uint64_t v = 0;
                uint32_t rank = 0;
                for (uint32_t i = 0; i < 8; ++i) {
                    if ((pb >> i) & 1) {
                        const uint64_t byte = ((sc >> rank) & 1) ? neg : pos;
                        v |= byte << (8 * i);
                        ++rank;
                    }
                }
                t.ent[e + sc] = v;
            }
            e += 1u << c;
        }
    }
    return t;
}

__device__ const Tables kTables = make_tables();
__device__ const Tables kTablesF16 = make_tables(0x3C, 0xBC);

// Copy both tables into LDS (s_tab: kTabBytes); the caller synchronises the block afterwards. Each
// thread issues all of its loads before any LDS write (one 8-byte load serves 8 consecutive (mask,
// base) copies of one presence byte), so the fill costs about one memory round trip (0.7-1 us per
// launch on MI355X, measured with a kernel that stops after the fill).
template <int BLOCK, bool F16 = false>
__device__ __forceinline__ void load_bitcos_tables(uint4 *s_tab) {
    // (mask, base) copies in units of 8 consecutive copies of one presence byte (64 bytes)
    constexpr int kUnits = 256 * 32 / 8;
    constexpr int kUnitPer = (kUnits + BLOCK - 1) / BLOCK;
    constexpr int kEntVec = (kEntries + 1) / 2;  // 16-byte vectors of the entry table
    constexpr int kEntPer = (kEntVec + BLOCK - 1) / BLOCK;
    const int t = threadIdx.x;
    const Tables &tab = F16 ? kTablesF16 : kTables;
    const uint2 *inf = reinterpret_cast<const uint2 *>(tab.info);
    const uint4 *src = reinterpret_cast<const uint4 *>(tab.ent);
    uint2 iv[kUnitPer];
    uint4 ev[kEntPer];
#pragma unroll
    for (int r = 0; r < kUnitPer; ++r) {
        const int u = t + r * BLOCK;
        iv[r] = u < kUnits ? inf[u >> 2] : make_uint2(0, 0);
    }
#pragma unroll
    for (int r = 0; r < kEntPer; ++r) {
        const int i = t + r * BLOCK;
        ev[r] = i < kEntVec ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < kUnitPer; ++r) {
        const int u = t + r * BLOCK;
        if (u < kUnits) {
#pragma unroll
            for (int c = 0; c < 4; ++c) s_tab[u * 4 + c] = make_uint4(iv[r].x, iv[r].y, iv[r].x, iv[r].y);
        }
    }
#pragma unroll
    for (int r = 0; r < kEntPer; ++r) {
        const int i = t + r * BLOCK;
        if (i < kEntVec) s_tab[kEntOff / 16 + i] = ev[r];
    }
}


// Nibble-keyed lookup ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-D, Eq. 4): the key is
// a presence nibble n (bits 0..3) and the next four compact sign bits s (bits 4..7); the entry holds
// the nibble's 4 weights as int8, weight i = 0 where n_i = 0, else -1 or +1 by sign bit r_i of s, where
// r_i counts the present weights before i. 256 entries of 4 bytes, kept in LDS in 32 copies: entry
// key of copy c at byte (key << 7) | (c << 2), so lane l reading copy l % 32 never conflicts.
constexpr uint32_t kNibCopies = 32;
constexpr uint32_t kNibBytes = 256 * 4 * kNibCopies;

struct NibTable {
    uint32_t ent[256];
};

constexpr NibTable make_nib_table() {
    NibTable t{};
    for (uint32_t key = 0; key < 256; ++key) {
        const uint32_t n = key & 15u, sg = key >> 4;
        uint32_t v = 0, r = 0;
        for (uint32_t i = 0; i < 4; ++i) {
            if ((n >> i) & 1u) {
                v |= (((sg >> r) & 1u) ? 0xFFu : 0x01u) << (8 * i);
                ++r;
            }
        }
        t.ent[key] = v;
    }
    return t;
}

__device__ const NibTable kNibTable = make_nib_table();

// Copy the nibble table's 32 copies into LDS (s_tab: at least kNibBytes); the caller synchronises.
template <int BLOCK>
__device__ __forceinline__ void load_nib_table(uint4 *s_tab) {
    constexpr int kWords = (int)(kNibBytes / 4);
    constexpr int kPer = (kWords + BLOCK - 1) / BLOCK;
    uint32_t *dst = reinterpret_cast<uint32_t *>(s_tab);
    uint32_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int w = (int)threadIdx.x + i * BLOCK;
        v[i] = w < kWords ? kNibTable.ent[w / (int)kNibCopies] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int w = (int)threadIdx.x + i * BLOCK;
        if (w < kWords) dst[w] = v[i];
    }
}

}  // namespace
}  // namespace tg
