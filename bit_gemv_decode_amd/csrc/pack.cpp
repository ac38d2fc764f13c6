// Host packers, descriptor checks, validation and unpacking for the three weight formats.
//
// BITCOS ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-A, Fig. 2): presence bitmap with
// one bit per weight plus a compacted sign stream holding one bit per non-zero weight in bitmap
// order. Bits are LSB-first (the Sec. II-C Eq. (2)-(3) example maps the first element to bit 0) and a
// sign bit of 1 means -1. The bitmap is row-major; the per-row sign positions (rowoff) let a GPU
// wave start a row without scanning earlier rows.
// Five-trit (same paper, Sec. I; "Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic
// Decoding", abstract): 26 bytes per 128 weights, digit = weight + 1, first weight least significant.
// 2-bit (Table I): code = weight + 1, four codes per byte, first weight in the low bits.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "tg_internal.h"

namespace tg {
namespace {

int worker_count(int64_t work) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t by_work = work / (1 << 22) + 1;
    return (int)std::max<int64_t>(1, std::min<int64_t>(std::min<unsigned>(hw ? hw : 1, 32), by_work));
}

template <class F>
void parallel_rows(int64_t n, int64_t work, F &&f) {
    int t = worker_count(work);
    if (t <= 1) { f(0, n); return; }
    std::vector<std::thread> th;
    int64_t step = (n + t - 1) / t;
    for (int i = 0; i < t; i++) {
        int64_t lo = i * step, hi = std::min(n, lo + step);
        if (lo >= hi) break;
        th.emplace_back([&f, lo, hi] { f(lo, hi); });
    }
    for (auto &x : th) x.join();
}

// Compact the bits of `v` selected by `mask` into the low bits of the result (bit extraction in
// mask order). Loop over the set bits; BMI2 hosts use the hardware instruction.
inline uint64_t extract_bits_portable(uint64_t v, uint64_t mask) {
    uint64_t out = 0;
    int j = 0;
    while (mask) {
        int b = __builtin_ctzll(mask);
        out |= ((v >> b) & 1ull) << j++;
        mask &= mask - 1;
    }
    return out;
}

__attribute__((target("bmi2"))) inline uint64_t extract_bits_bmi2(uint64_t v, uint64_t mask) {
    return __builtin_ia32_pext_di(v, mask);
}

bool have_bmi2() {
    static const bool b = __builtin_cpu_supports("bmi2");
    return b;
}

// Presence and negative masks of 64 consecutive weights; false if a value is not ternary.
inline bool masks64(const int8_t *w, uint64_t *present, uint64_t *negative) {
    uint64_t p = 0, q = 0;
    bool ok = true;
    for (int b = 0; b < 64; b++) {
        int8_t v = w[b];
        ok &= (v >= -1 && v <= 1);
        p |= (uint64_t)(v != 0) << b;
        q |= (uint64_t)(v < 0) << b;
    }
    *present = p;
    *negative = q;
    return ok;
}

bool all_ternary(const int8_t *w, int64_t count) {
    std::atomic<bool> ok{true};
    parallel_rows(count / 4096 + 1, count, [&](int64_t lo, int64_t hi) {
        int64_t a = lo * 4096, b = std::min(count, hi * 4096);
        for (int64_t i = a; i < b; i++)
            if (w[i] < -1 || w[i] > 1) { ok = false; return; }
    });
    return ok;
}

void fill_header(tg_desc *d, int fmt, int64_t n, int64_t k, uint64_t nnz) {
    memset(d, 0, sizeof(*d));
    d->magic = TG_MAGIC;
    d->version = TG_VERSION;
    d->fmt = fmt;
    d->group = TG_GROUP;
    d->n = n;
    d->k = k;
    d->nnz = nnz;
}

int shape_ok(const int8_t *w, int64_t n, int64_t k, size_t *out_bytes) {
    if (!w || !out_bytes) return TG_EINVAL;
    if (n < 1 || k < 1 || k % TG_GROUP) return TG_ESHAPE;
    if (n > (1ll << 31) - 1 || k > (1ll << 31) - 1 || n > (int64_t)(UINT64_MAX / 4) / k) return TG_ESHAPE;
    return TG_OK;
}

uint64_t count_nonzero(const int8_t *w, int64_t n, int64_t k, std::vector<uint32_t> *row_nnz) {
    row_nnz->assign(n, 0);
    parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
        for (int64_t r = lo; r < hi; r++) {
            uint32_t c = 0;
            const int8_t *row = w + r * k;
            for (int64_t i = 0; i < k; i++) c += row[i] != 0;
            (*row_nnz)[r] = c;
        }
    });
    uint64_t t = 0;
    for (uint32_t c : *row_nnz) t += c;
    return t;
}

}  // namespace

int check_desc(const tg_desc *d, uint64_t limit) {
    if (!d) return TG_EINVAL;
    if (d->magic != TG_MAGIC || d->version != TG_VERSION) return TG_EFORMAT;
    if (d->fmt != TG_FMT_BITCOS && d->fmt != TG_FMT_5TRIT && d->fmt != TG_FMT_2BIT && d->fmt != TG_FMT_T5B)
        return TG_EFORMAT;
    if (d->group != (d->fmt == TG_FMT_T5B ? kT5bBlock : TG_GROUP)) return TG_EFORMAT;
    if (d->n < 1 || d->k < 1 || d->k % TG_GROUP || d->n > (1ll << 31) - 1 || d->k > (1ll << 31) - 1) return TG_ECORRUPT;
    uint64_t n = (uint64_t)d->n, k = (uint64_t)d->k;
    if (n > UINT64_MAX / 4 / k) return TG_ECORRUPT;
    if (d->nnz > n * k) return TG_ECORRUPT;
    if (limit && d->bytes_total > limit) return TG_ECORRUPT;
    auto section_ok = [&](uint64_t off, uint64_t bytes, uint64_t min_off) {
        return off >= min_off && off % kAlign == 0 && bytes <= d->bytes_total && off <= d->bytes_total - bytes;
    };
    if (!section_ok(d->off_codes, d->bytes_codes, TG_HEADER_BYTES)) return TG_ECORRUPT;
    if (d->fmt == TG_FMT_BITCOS) {
        if (d->nnz > 0xFFFFFFFFull) return TG_ECORRUPT;
        if (d->bytes_codes != n * k / 8) return TG_ECORRUPT;
        uint64_t sign_bytes = (d->nnz + 7) / 8;
        if (d->bytes_signs < sign_bytes + kSignPad || d->bytes_signs % 4) return TG_ECORRUPT;
        if (!section_ok(d->off_signs, d->bytes_signs, d->off_codes + d->bytes_codes)) return TG_ECORRUPT;
        if (d->bytes_index != 4 * (n + 1)) return TG_ECORRUPT;
        if (!section_ok(d->off_index, d->bytes_index, d->off_signs + d->bytes_signs)) return TG_ECORRUPT;
        if (d->bytes_payload != d->bytes_codes + sign_bytes + d->bytes_index) return TG_ECORRUPT;
        if ((d->bytes_signs / 4) > 0xFFFFFFFFull) return TG_ECORRUPT;
        if (d->empty_rows > n) return TG_ECORRUPT;
    } else {
        if (d->empty_rows) return TG_ECORRUPT;
        uint64_t want = d->fmt == TG_FMT_5TRIT ? n * (k / TG_GROUP) * 26
                        : d->fmt == TG_FMT_T5B ? n * t5b_blocks(k) * 32
                                               : n * k / 4;
        if (d->bytes_codes != want || d->bytes_signs || d->bytes_index) return TG_ECORRUPT;
        if (d->bytes_total - d->off_codes - d->bytes_codes < kSignPad) return TG_ECORRUPT;  // read slack
        if (d->bytes_payload != want) return TG_ECORRUPT;
    }
    return TG_OK;
}

}  // namespace tg

using namespace tg;

extern "C" int tg_pack_bitcos(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes) {
    int e = shape_ok(w, n, k, out_bytes);
    if (e) return e;
    if (!all_ternary(w, n * k)) return TG_ENOTTERNARY;
    std::vector<uint32_t> row_nnz;
    uint64_t nnz = count_nonzero(w, n, k, &row_nnz);
    if (nnz > 0xFFFFFFFFull) return TG_ESHAPE;
    tg_desc d;
    fill_header(&d, TG_FMT_BITCOS, n, k, nnz);
    d.empty_rows = (uint32_t)std::count(row_nnz.begin(), row_nnz.end(), 0u);
    uint64_t sign_bytes = (nnz + 7) / 8;
    d.off_codes = TG_HEADER_BYTES;
    d.bytes_codes = (uint64_t)n * k / 8;
    d.off_signs = align_up(d.off_codes + d.bytes_codes, kAlign);
    d.bytes_signs = align_up(sign_bytes + kSignPad, 8);
    d.off_index = align_up(d.off_signs + d.bytes_signs, kAlign);
    d.bytes_index = 4 * ((uint64_t)n + 1);
    d.bytes_total = align_up(d.off_index + d.bytes_index, kAlign);
    d.bytes_payload = d.bytes_codes + sign_bytes + d.bytes_index;
    *out_bytes = d.bytes_total;
    if (!out) return TG_OK;
    if (out_cap < d.bytes_total) return TG_ENOSPACE;

    uint8_t *base = (uint8_t *)out;
    memset(base, 0, TG_HEADER_BYTES);
    memcpy(base, &d, sizeof(d));
    uint64_t *bitmap = (uint64_t *)(base + d.off_codes);
    uint64_t *signs = (uint64_t *)(base + d.off_signs);
    uint32_t *rowoff = (uint32_t *)(base + d.off_index);
    memset(base + d.off_signs, 0, d.off_index - d.off_signs);
    memset(base + d.off_index + d.bytes_index, 0, d.bytes_total - d.off_index - d.bytes_index);
    uint32_t pos = 0;
    for (int64_t r = 0; r < n; r++) { rowoff[r] = pos; pos += row_nnz[r]; }
    rowoff[n] = pos;

    // Rows are packed in parallel. A row's sign bits start at rowoff[r]; interior 64-bit words of a
    // row range belong to one thread, the first and last word of each range may be shared with a
    // neighbour and are merged with an atomic OR.
    const bool bmi2 = have_bmi2();
    const int64_t words_per_row = k / 64;
    const int64_t sign_words = (int64_t)(d.bytes_signs / 8);
    parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
        if (lo >= hi) return;
        uint64_t first_bit = rowoff[lo], last_bit = rowoff[hi];
        int64_t w_first = (int64_t)(first_bit / 64), w_last = (int64_t)((last_bit + 63) / 64);
        std::vector<uint64_t> local((size_t)std::max<int64_t>(1, w_last - w_first + 1), 0);
        uint64_t bitpos = first_bit;
        for (int64_t r = lo; r < hi; r++) {
            const int8_t *row = w + r * k;
            for (int64_t j = 0; j < words_per_row; j++) {
                uint64_t p, q;
                masks64(row + 64 * j, &p, &q);
                bitmap[r * words_per_row + j] = p;
                int c = __builtin_popcountll(p);
                if (!c) continue;
                uint64_t bits = bmi2 ? extract_bits_bmi2(q, p) : extract_bits_portable(q, p);
                uint64_t li = bitpos / 64 - (uint64_t)w_first;
                int sh = (int)(bitpos % 64);
                local[li] |= bits << sh;
                if (sh && sh + c > 64) local[li + 1] |= bits >> (64 - sh);
                bitpos += (uint64_t)c;
            }
        }
        for (int64_t i = w_first; i < w_last && i < sign_words; i++) {
            uint64_t v = local[(size_t)(i - w_first)];
            if (!v) continue;
            if (i == w_first || i == w_last - 1)
                __atomic_fetch_or(&signs[i], v, __ATOMIC_RELAXED);
            else
                signs[i] = v;
        }
    });
    return TG_OK;
}

extern "C" int tg_pack_5trit(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes) {
    int e = shape_ok(w, n, k, out_bytes);
    if (e) return e;
    if (!all_ternary(w, n * k)) return TG_ENOTTERNARY;
    std::vector<uint32_t> row_nnz;
    uint64_t nnz = count_nonzero(w, n, k, &row_nnz);
    tg_desc d;
    fill_header(&d, TG_FMT_5TRIT, n, k, nnz);
    const int64_t ng = k / TG_GROUP;
    d.off_codes = TG_HEADER_BYTES;
    d.bytes_codes = (uint64_t)n * ng * 26;
    d.bytes_total = align_up(d.off_codes + d.bytes_codes + kSignPad, kAlign);
    d.bytes_payload = d.bytes_codes;
    *out_bytes = d.bytes_total;
    if (!out) return TG_OK;
    if (out_cap < d.bytes_total) return TG_ENOSPACE;
    uint8_t *base = (uint8_t *)out;
    memset(base, 0, TG_HEADER_BYTES);
    memcpy(base, &d, sizeof(d));
    memset(base + d.off_codes + d.bytes_codes, 0, d.bytes_total - d.off_codes - d.bytes_codes);
    uint8_t *codes = base + d.off_codes;
    parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
        for (int64_t r = lo; r < hi; r++)
            for (int64_t g = 0; g < ng; g++) {
                const int8_t *src = w + r * k + g * TG_GROUP;
                uint8_t *dst = codes + (r * ng + g) * 26;
                for (int b = 0; b < 26; b++) {
                    // Horner from the last digit: value = d0 + 3 (d1 + 3 (d2 + 3 (d3 + 3 d4)))
                    unsigned v = 0;
                    for (int i = 4; i >= 0; i--) {
                        int idx = 5 * b + i;
                        unsigned digit = idx < TG_GROUP ? (unsigned)(src[idx] + 1) : 1u;
                        v = v * 3 + digit;
                    }
                    dst[b] = (uint8_t)v;
                }
            }
    });
    return TG_OK;
}

extern "C" int tg_pack_2bit(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes) {
    int e = shape_ok(w, n, k, out_bytes);
    if (e) return e;
    if (!all_ternary(w, n * k)) return TG_ENOTTERNARY;
    std::vector<uint32_t> row_nnz;
    uint64_t nnz = count_nonzero(w, n, k, &row_nnz);
    tg_desc d;
    fill_header(&d, TG_FMT_2BIT, n, k, nnz);
    d.off_codes = TG_HEADER_BYTES;
    d.bytes_codes = (uint64_t)n * k / 4;
    d.bytes_total = align_up(d.off_codes + d.bytes_codes + kSignPad, kAlign);
    d.bytes_payload = d.bytes_codes;
    *out_bytes = d.bytes_total;
    if (!out) return TG_OK;
    if (out_cap < d.bytes_total) return TG_ENOSPACE;
    uint8_t *base = (uint8_t *)out;
    memset(base, 0, TG_HEADER_BYTES);
    memcpy(base, &d, sizeof(d));
    memset(base + d.off_codes + d.bytes_codes, 0, d.bytes_total - d.off_codes - d.bytes_codes);
    uint8_t *codes = base + d.off_codes;
    parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo * (k / 4); i < hi * (k / 4); i++) {
            const int8_t *src = w + 4 * i;
            codes[i] = (uint8_t)((src[0] + 1) | ((src[1] + 1) << 2) | ((src[2] + 1) << 4) | ((src[3] + 1) << 6));
        }
    });
    return TG_OK;
}

extern "C" int tg_pack_t5b(const int8_t *w, int64_t n, int64_t k, float scale, void *out, size_t out_cap,
                           size_t *out_bytes) {
    int e = shape_ok(w, n, k, out_bytes);
    if (e) return e;
    if (!(scale == scale) || scale - scale != 0.0f) return TG_EINVAL;  // NaN or infinite
    if (!all_ternary(w, n * k)) return TG_ENOTTERNARY;
    std::vector<uint32_t> row_nnz;
    uint64_t nnz = count_nonzero(w, n, k, &row_nnz);
    tg_desc d;
    fill_header(&d, TG_FMT_T5B, n, k, nnz);
    d.group = kT5bBlock;
    memcpy(&d.tensor_scale, &scale, 4);
    const int64_t nb = (int64_t)t5b_blocks((uint64_t)k);
    d.off_codes = TG_HEADER_BYTES;
    d.bytes_codes = (uint64_t)n * nb * 32;
    d.bytes_total = align_up(d.off_codes + d.bytes_codes + kSignPad, kAlign);
    d.bytes_payload = d.bytes_codes;
    *out_bytes = d.bytes_total;
    if (!out) return TG_OK;
    if (out_cap < d.bytes_total) return TG_ENOSPACE;
    uint8_t *base = (uint8_t *)out;
    memset(base, 0, TG_HEADER_BYTES);
    memcpy(base, &d, sizeof(d));
    memset(base + d.off_codes + d.bytes_codes, 0, d.bytes_total - d.off_codes - d.bytes_codes);
    uint8_t *codes = base + d.off_codes;
    parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
        for (int64_t r = lo; r < hi; r++)
            for (int64_t b = 0; b < nb; b++) {
                uint8_t *dst = codes + (r * nb + b) * 32;
                for (int j = 0; j < 32; j++) {
                    // Horner from the last digit; positions past k hold the weight-0 digit
                    unsigned v = 0;
                    for (int i = 4; i >= 0; i--) {
                        const int64_t col = kT5bBlock * b + 5 * j + i;
                        const unsigned digit = col < k ? (unsigned)(w[r * k + col] + 1) : 1u;
                        v = v * 3 + digit;
                    }
                    dst[j] = (uint8_t)v;
                }
            }
    });
    return TG_OK;
}

extern "C" int tg_describe(const void *packed, size_t bytes, tg_desc *out) {
    if (!packed || !out) return TG_EINVAL;
    if (bytes < TG_HEADER_BYTES) return TG_EFORMAT;
    tg_desc d;
    memcpy(&d, packed, sizeof(d));
    int e = check_desc(&d, bytes);
    if (e) return e;
    *out = d;
    return TG_OK;
}

namespace {

int validate_contents(const uint8_t *base, const tg_desc &d) {
    const int64_t n = d.n, k = d.k, ng = k / TG_GROUP;
    const uint8_t *codes = base + d.off_codes;
    std::atomic<int> err{TG_OK};
    std::atomic<uint64_t> nnz{0};
    if (d.fmt == TG_FMT_BITCOS) {
        const uint64_t *bm = (const uint64_t *)codes;
        const uint32_t *rowoff = (const uint32_t *)(base + d.off_index);
        if (rowoff[0] != 0 || rowoff[n] != d.nnz) return TG_ECORRUPT;
        std::atomic<uint64_t> empty{0};
        parallel_rows(n, n * k / 8, [&](int64_t lo, int64_t hi) {
            uint64_t e = 0;
            for (int64_t r = lo; r < hi; r++) {
                uint64_t c = 0;
                for (int64_t j = 0; j < k / 64; j++) c += (uint64_t)__builtin_popcountll(bm[r * (k / 64) + j]);
                if (rowoff[r + 1] < rowoff[r] || rowoff[r + 1] - rowoff[r] != c) err = TG_ECORRUPT;
                e += c == 0;
            }
            empty += e;
        });
        if (err) return err;
        return empty.load() == d.empty_rows ? TG_OK : TG_ECORRUPT;
    }
    parallel_rows(n, n * k / 4, [&](int64_t lo, int64_t hi) {
        uint64_t local = 0;
        for (int64_t r = lo; r < hi; r++) {
            if (d.fmt == TG_FMT_T5B) {
                const int64_t nb = (int64_t)t5b_blocks((uint64_t)k);
                for (int64_t b = 0; b < nb; b++) {
                    const uint8_t *src = codes + (r * nb + b) * 32;
                    for (int j = 0; j < 32; j++) {
                        unsigned v = src[j];
                        if (v >= 243) { err = TG_ECORRUPT; return; }
                        for (int i = 0; i < 5; i++) {
                            unsigned digit = v % 3;
                            v /= 3;
                            if (kT5bBlock * b + 5 * j + i < k) local += digit != 1;
                            else if (digit != 1) { err = TG_ECORRUPT; return; }
                        }
                    }
                }
            } else if (d.fmt == TG_FMT_5TRIT) {
                for (int64_t g = 0; g < ng; g++) {
                    const uint8_t *src = codes + (r * ng + g) * 26;
                    for (int b = 0; b < 26; b++) {
                        unsigned v = src[b];
                        if (v >= 243) { err = TG_ECORRUPT; return; }
                        for (int i = 0; i < 5; i++) {
                            unsigned digit = v % 3;
                            v /= 3;
                            if (5 * b + i < TG_GROUP) local += digit != 1;
                            else if (digit != 1) { err = TG_ECORRUPT; return; }
                        }
                    }
                }
            } else {
                for (int64_t i = r * (k / 4); i < (r + 1) * (k / 4); i++) {
                    unsigned v = codes[i];
                    for (int j = 0; j < 4; j++) {
                        unsigned c = (v >> (2 * j)) & 3;
                        if (c == 3) { err = TG_ECORRUPT; return; }
                        local += c != 1;
                    }
                }
            }
        }
        nnz += local;
    });
    if (err) return err;
    return nnz.load() == d.nnz ? TG_OK : TG_ECORRUPT;
}

}  // namespace

extern "C" int tg_validate(const void *packed, size_t bytes) {
    tg_desc d;
    int e = tg_describe(packed, bytes, &d);
    if (e) return e;
    return validate_contents((const uint8_t *)packed, d);
}

extern "C" int tg_unpack(const void *packed, size_t bytes, int8_t *w_out) {
    if (!w_out) return TG_EINVAL;
    int e = tg_validate(packed, bytes);
    if (e) return e;
    tg_desc d;
    memcpy(&d, packed, sizeof(d));
    const uint8_t *base = (const uint8_t *)packed;
    const int64_t n = d.n, k = d.k, ng = k / TG_GROUP;
    const uint8_t *codes = base + d.off_codes;
    if (d.fmt == TG_FMT_BITCOS) {
        const uint64_t *bm = (const uint64_t *)codes;
        const uint8_t *signs = base + d.off_signs;
        const uint32_t *rowoff = (const uint32_t *)(base + d.off_index);
        parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
            for (int64_t r = lo; r < hi; r++) {
                uint64_t pos = rowoff[r];
                for (int64_t j = 0; j < k / 64; j++) {
                    uint64_t p = bm[r * (k / 64) + j];
                    for (int b = 0; b < 64; b++) {
                        int8_t v = 0;
                        if ((p >> b) & 1) {
                            v = ((signs[pos >> 3] >> (pos & 7)) & 1) ? -1 : 1;
                            pos++;
                        }
                        w_out[r * k + 64 * j + b] = v;
                    }
                }
            }
        });
    } else if (d.fmt == TG_FMT_T5B) {
        const int64_t nb = (int64_t)t5b_blocks((uint64_t)k);
        parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
            for (int64_t r = lo; r < hi; r++)
                for (int64_t b = 0; b < nb; b++)
                    for (int j = 0; j < 32; j++) {
                        unsigned v = codes[(r * nb + b) * 32 + j];
                        for (int i = 0; i < 5; i++, v /= 3) {
                            const int64_t col = kT5bBlock * b + 5 * j + i;
                            if (col < k) w_out[r * k + col] = (int8_t)((int)(v % 3) - 1);
                        }
                    }
        });
    } else if (d.fmt == TG_FMT_5TRIT) {
        parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
            for (int64_t r = lo; r < hi; r++)
                for (int64_t g = 0; g < ng; g++)
                    for (int b = 0; b < 26; b++) {
                        unsigned v = codes[(r * ng + g) * 26 + b];
                        for (int i = 0; i < 5 && 5 * b + i < TG_GROUP; i++, v /= 3)
                            w_out[r * k + g * TG_GROUP + 5 * b + i] = (int8_t)((int)(v % 3) - 1);
                    }
        });
    } else {
        parallel_rows(n, n * k, [&](int64_t lo, int64_t hi) {
            for (int64_t i = lo * k; i < hi * k; i++)
                w_out[i] = (int8_t)((int)((codes[i >> 2] >> (2 * (i & 3))) & 3) - 1);
        });
    }
    return TG_OK;
}

extern "C" const char *tg_strerror(int code) {
    switch (code) {
        case TG_OK: return "success";
        case TG_EINVAL: return "invalid argument (null pointer, bad enum value or m out of range)";
        case TG_ENOTTERNARY: return "weight outside {-1, 0, +1}";
        case TG_ESHAPE: return "bad shape (n, k < 1, k not a multiple of 128, or too large for the format)";
        case TG_EFORMAT: return "not a packed ternary buffer of this version";
        case TG_ECORRUPT: return "packed buffer contents contradict its descriptor";
        case TG_ENOSPACE: return "output buffer too small";
        case TG_EHIP: return "HIP runtime error while enqueuing";
        default: return "unknown error";
    }
}

extern "C" uint32_t tg_version(void) { return TG_VERSION; }
