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
    uint32_t info[256][4];       // per presence byte: mask (popcount ones, shifted left 3), LDS base;
                                 // twice, so that one 16-byte copy fills two bank copies
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
            t.info[pb][0] = t.info[pb][2] = ((1u << c) - 1u) << 3;
            t.info[pb][1] = t.info[pb][3] = kEntOff + 8 * e;
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

// Copy both tables into LDS (s_tab: kTabBytes); the caller waits (lds_copies_landed) and synchronises the
// block afterwards. The
// copies go from global memory straight into LDS (global_load_lds_dwordx4: lane l of a wave writes
// the 16 bytes it loads at the wave's LDS base + 16 l), 1 KB per wave instruction and no registers
// in between: 64 instructions for the (mask, base) copies (one presence byte's 32 copies are 16
// lanes' loads of the same doubled entry) and 52 for the entry table, spread over the block's waves,
// all issued before the first completes, so the fill is about one memory round trip.
template <int BLOCK, bool F16 = false>
__device__ __forceinline__ void load_bitcos_tables(uint4 *s_tab) {
    constexpr int kWaves = BLOCK / 64;
    constexpr int kInfoChunks = (int)(kInfoBytes / 1024);  // 4 presence bytes per chunk
    constexpr int kEntVec = (kEntries + 1) / 2;            // 16-byte vectors of the entry table
    constexpr int kEntChunks = (kEntVec + 63) / 64;
    static_assert(kInfoBytes % 1024 == 0 && kEntOff % 16 == 0, "whole chunks");
    const int lane = (int)(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const Tables &tab = F16 ? kTablesF16 : kTables;
    const uint4 *inf = reinterpret_cast<const uint4 *>(tab.info);
    const uint4 *ent = reinterpret_cast<const uint4 *>(tab.ent);
    typedef __attribute__((address_space(3))) void *lds_ptr;
    for (int c = wave; c < kInfoChunks; c += kWaves)
        __builtin_amdgcn_global_load_lds(inf + 4 * c + (lane >> 4), (lds_ptr)(s_tab + 64 * c), 16, 0, 0);
    for (int c = wave; c < kEntChunks; c += kWaves) {
        // the last chunk is partial: its lanes past the table load nothing
        if (64 * c + lane < kEntVec)
            __builtin_amdgcn_global_load_lds(ent + 64 * c + lane, (lds_ptr)(s_tab + kEntOff / 16 + 64 * c), 16, 0, 0);
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
