/*
 * oracle.c -- plain, slow CPU oracle for the ternary GEMV. TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load this file's
 * library. The product path (the HIP library and its Python binding) never calls it and shares no
 * code with it: no headers, helpers, tables or constants.
 *
 * What it computes, and where the pages define it:
 *   - BITCOS ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-A and Fig. 2): a ternary
 *     tensor is a presence bitmap (one bit per weight, set where the weight is non-zero) plus a
 *     sign vector holding one bit per non-zero weight, in tensor order; the j-th sign bit belongs
 *     to the j-th set bit of the bitmap. Sign polarity and bit order follow the Eq. (2)-(3) worked
 *     example of Sec. II-C: the first element is the least significant bit, and a stored sign bit
 *     of 1 marks a negative weight.
 *   - pdep (Sec. II-B, Fig. 4): deposit the low bits of a source, in order, at the set positions
 *     of a mask. Unpacking BITCOS is pdep applied over the whole stream.
 *   - five-trit bytes (same paper, Sec. I; "Sub-Two-Bit Ternary Weight Storage with Table-Free
 *     Arithmetic Decoding", abstract): five ternary digits per byte, 3^5 = 243 <= 256, and a block
 *     of 128 weights takes ceil(128/5) = 26 bytes.
 *   - 2-bit packing (Table I, "2-bit packing" column): two bits per weight.
 *   - t5b ("Sub-Two-Bit Ternary Weight Storage ...", abstract): the five-trit construction in blocks
 *     of 160 weights (32 bytes, 1.600 bits per weight) with one scale per tensor.
 *   - the GEMV contract (Sec. II-C, discussion after Fig. 5): int8 activations, dot products
 *     accumulated in int32 per group of 128 reduction elements, the group's 16-bit scale applied
 *     once per group. The oracle computes the dense definition: acc = sum of W*x over the group,
 *     then y = sum over groups of scale*acc in double precision, rounded once to float.
 *
 * Readings where the pages leave a step open (each is also listed in the design notes):
 *   - row-major orientation: W is n rows by k reduction elements, y = W x;
 *   - the bitmap and sign stream are bit streams in (row, k) order, packed LSB-first into bytes;
 *     with k a multiple of 64 this is the same byte image as little-endian 64-bit words per row;
 *   - five-trit digit map: digit = weight + 1, the first weight is the least-significant digit;
 *     byte 25 of a 128-block holds weights 125..127 and two padding digits of value 1 (weight 0);
 *   - 2-bit code: code = weight + 1, four codes per byte, the first weight in the lowest two bits;
 *     code 3 is invalid;
 *   - scales are IEEE binary16, decoded here from the format's definition.
 *   - activation quantisation (Sec. II-C, discussion after Fig. 5: activations are quantised to int8
 *     per group of 128 on the int8 path; the quantiser itself is not given): symmetric absmax per
 *     group of 128 consecutive k of one activation row, sigma = max|x| / 127 and q = x / sigma
 *     rounded to nearest-even, clamped to [-127, 127]; an all-zero group has sigma = 0 and q = 0.
 *     Both divisions are single-precision IEEE operations, so the integer codes are decided in fp32.
 *     The group's activation scale multiplies its term once, beside the weight scale.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_GROUP 128

/* ---------- bit-stream helpers (LSB-first within each byte) ---------- */

static int get_bit(const uint8_t *buf, int64_t i) { return (buf[i >> 3] >> (i & 7)) & 1; }

static void set_bit(uint8_t *buf, int64_t i) { buf[i >> 3] = (uint8_t)(buf[i >> 3] | (1u << (i & 7))); }

/* ---------- IEEE binary16 -> double, from the format's definition ---------- */

double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = (double)f; /* subnormal: f * 2^-24 */
        for (int i = 0; i < 24; i++) v *= 0.5;
    } else if (e == 31) {
        v = f ? (0.0 / 0.0) : (1.0 / 0.0);
    } else {
        v = 1.0 + (double)f / 1024.0;
        int p = e - 15;
        while (p > 0) { v *= 2.0; p--; }
        while (p < 0) { v *= 0.5; p++; }
    }
    return sign ? -v : v;
}

/* ---------- pdep, as Fig. 4 defines it ---------- */

uint64_t oracle_pdep64(uint64_t src, uint64_t mask) {
    uint64_t dst = 0;
    int taken = 0;
    for (int pos = 0; pos < 64; pos++) {
        if ((mask >> pos) & 1) {
            if ((src >> taken) & 1) dst |= (uint64_t)1 << pos;
            taken++;
        }
    }
    return dst;
}

/* ---------- BITCOS ---------- */

/* Number of non-zero weights; -1 if any value is outside {-1, 0, +1}. */
int64_t oracle_count_nonzero(const int8_t *w, int64_t count) {
    int64_t nnz = 0;
    for (int64_t i = 0; i < count; i++) {
        if (w[i] < -1 || w[i] > 1) return -1;
        if (w[i] != 0) nnz++;
    }
    return nnz;
}

/*
 * Pack W[n][k] into BITCOS. bitmap receives n*k bits, signs receives nnz bits (both zero-filled
 * by this function over their full byte length), rowoff[r] is the sign-stream position of row r's
 * first non-zero and rowoff[n] = nnz. Returns nnz, or -1 for a non-ternary value.
 */
int64_t oracle_bitcos_pack(const int8_t *w, int64_t n, int64_t k, uint8_t *bitmap, int64_t bitmap_bytes,
                           uint8_t *signs, int64_t signs_bytes, uint32_t *rowoff) {
    int64_t nnz = oracle_count_nonzero(w, n * k);
    if (nnz < 0) return -1;
    if (bitmap_bytes * 8 < n * k || signs_bytes * 8 < nnz) return -1;
    memset(bitmap, 0, (size_t)bitmap_bytes);
    memset(signs, 0, (size_t)signs_bytes);
    int64_t j = 0;
    for (int64_t r = 0; r < n; r++) {
        if (rowoff) rowoff[r] = (uint32_t)j;
        for (int64_t c = 0; c < k; c++) {
            int8_t v = w[r * k + c];
            if (v != 0) {
                set_bit(bitmap, r * k + c);
                if (v < 0) set_bit(signs, j);
                j++;
            }
        }
    }
    if (rowoff) rowoff[n] = (uint32_t)j;
    return nnz;
}

/*
 * Unpack BITCOS: walk the bitmap in storage order and hand each set bit the next sign bit
 * (pdep over the whole stream). Returns the number of sign bits consumed.
 */
int64_t oracle_bitcos_unpack(const uint8_t *bitmap, const uint8_t *signs, int64_t n, int64_t k, int8_t *w) {
    int64_t j = 0;
    for (int64_t i = 0; i < n * k; i++) {
        if (get_bit(bitmap, i)) {
            w[i] = get_bit(signs, j) ? -1 : 1;
            j++;
        } else {
            w[i] = 0;
        }
    }
    return j;
}

/* ---------- five-trit bytes ---------- */

int64_t oracle_t5_bytes(int64_t n, int64_t k) { return n * (k / ORACLE_GROUP) * 26; }

int oracle_t5_pack(const int8_t *w, int64_t n, int64_t k, uint8_t *out) {
    if (k % ORACLE_GROUP) return -1;
    if (oracle_count_nonzero(w, n * k) < 0) return -1;
    int64_t ng = k / ORACLE_GROUP;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t g = 0; g < ng; g++) {
            const int8_t *src = w + r * k + g * ORACLE_GROUP;
            uint8_t *dst = out + (r * ng + g) * 26;
            for (int b = 0; b < 26; b++) {
                int value = 0, place = 1;
                for (int i = 0; i < 5; i++) {
                    int idx = 5 * b + i;
                    int digit = idx < ORACLE_GROUP ? src[idx] + 1 : 1;
                    value += digit * place;
                    place *= 3;
                }
                dst[b] = (uint8_t)value;
            }
        }
    }
    return 0;
}

/* Returns 0, or -1 if a byte is >= 243 or a padding digit is not the weight-0 digit. */
int oracle_t5_unpack(const uint8_t *in, int64_t n, int64_t k, int8_t *w) {
    if (k % ORACLE_GROUP) return -1;
    int64_t ng = k / ORACLE_GROUP;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t g = 0; g < ng; g++) {
            const uint8_t *src = in + (r * ng + g) * 26;
            int8_t *dst = w + r * k + g * ORACLE_GROUP;
            for (int b = 0; b < 26; b++) {
                int value = src[b];
                if (value >= 243) return -1;
                for (int i = 0; i < 5; i++) {
                    int digit = value % 3;
                    value /= 3;
                    int idx = 5 * b + i;
                    if (idx < ORACLE_GROUP) dst[idx] = (int8_t)(digit - 1);
                    else if (digit != 1) return -1;
                }
            }
        }
    }
    return 0;
}

/* ---------- t5b: five-trit bytes in blocks of 160 weights, one scale per tensor ---------- */

/*
 * "Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic Decoding" (abstract): the same
 * base-3 construction at a block length of 160 (32 bytes, 1.600 bits per weight), the scale carried
 * once per tensor. Readings: blocks run along each row, block b of row r holding weights
 * 160b .. 160b + 159; byte j of a block holds weights 160b + 5j .. 160b + 5j + 4 as digits weight + 1,
 * the first weight least significant; positions at or past k are padding digits of value 1
 * (weight 0).
 */
int64_t oracle_t5b_blocks(int64_t k) { return (k + 159) / 160; }

int oracle_t5b_pack(const int8_t *w, int64_t n, int64_t k, uint8_t *out) {
    if (k < 1 || oracle_count_nonzero(w, n * k) < 0) return -1;
    int64_t nb = oracle_t5b_blocks(k);
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nb; b++)
            for (int j = 0; j < 32; j++) {
                int value = 0, place = 1;
                for (int i = 0; i < 5; i++) {
                    int64_t col = 160 * b + 5 * j + i;
                    int digit = col < k ? w[r * k + col] + 1 : 1;
                    value += digit * place;
                    place *= 3;
                }
                out[(r * nb + b) * 32 + j] = (uint8_t)value;
            }
    return 0;
}

/* Returns 0, or -1 if a byte is >= 243 or a padding digit is not the weight-0 digit. */
int oracle_t5b_unpack(const uint8_t *in, int64_t n, int64_t k, int8_t *w) {
    int64_t nb = oracle_t5b_blocks(k);
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nb; b++)
            for (int j = 0; j < 32; j++) {
                int value = in[(r * nb + b) * 32 + j];
                if (value >= 243) return -1;
                for (int i = 0; i < 5; i++) {
                    int digit = value % 3;
                    value /= 3;
                    int64_t col = 160 * b + 5 * j + i;
                    if (col < k) w[r * k + col] = (int8_t)(digit - 1);
                    else if (digit != 1) return -1;
                }
            }
    return 0;
}

/* acc[mi][r][b] = sum over the k of block b (160 b <= k < min(160 b + 160, k)) of W[r][k] * x[mi][k]. */
void oracle_gemv_acc_blocks(const int8_t *w, int64_t n, int64_t k, const int8_t *x, int64_t m, int32_t *acc) {
    int64_t nb = oracle_t5b_blocks(k);
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++)
            for (int64_t b = 0; b < nb; b++) {
                int32_t s = 0;
                for (int64_t c = 160 * b; c < 160 * (b + 1) && c < k; c++)
                    s += (int32_t)w[r * k + c] * (int32_t)x[mi * k + c];
                acc[(mi * n + r) * nb + b] = s;
            }
}

/* y[mi][r] = (float)((double) scale * (double) sum_b acc[mi][r][b]): the per-tensor scale applied to
 * the exact integer row sum, rounded once. */
void oracle_combine_tensor(const int32_t *acc, float scale, int64_t n, int64_t nb, int64_t m, float *y) {
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++) {
            int64_t s = 0;
            for (int64_t b = 0; b < nb; b++) s += acc[(mi * n + r) * nb + b];
            y[mi * n + r] = (float)((double)scale * (double)s);
        }
}

/* ---------- 2-bit codes ---------- */

int oracle_b2_pack(const int8_t *w, int64_t n, int64_t k, uint8_t *out) {
    if (k % 4) return -1;
    if (oracle_count_nonzero(w, n * k) < 0) return -1;
    for (int64_t i = 0; i < n * k / 4; i++) {
        int value = 0;
        for (int j = 0; j < 4; j++) value |= (w[4 * i + j] + 1) << (2 * j);
        out[i] = (uint8_t)value;
    }
    return 0;
}

int oracle_b2_unpack(const uint8_t *in, int64_t n, int64_t k, int8_t *w) {
    if (k % 4) return -1;
    for (int64_t i = 0; i < n * k / 4; i++) {
        for (int j = 0; j < 4; j++) {
            int code = (in[i] >> (2 * j)) & 3;
            if (code == 3) return -1;
            w[4 * i + j] = (int8_t)(code - 1);
        }
    }
    return 0;
}

/* ---------- the GEMV definition ---------- */

/* acc[mi][r][g] = sum over the 128 k of group g of W[r][k] * x[mi][k], exact in int32. */
void oracle_gemv_acc(const int8_t *w, int64_t n, int64_t k, const int8_t *x, int64_t m, int32_t *acc) {
    int64_t ng = k / ORACLE_GROUP;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++)
            for (int64_t g = 0; g < ng; g++) {
                int32_t s = 0;
                for (int64_t c = g * ORACLE_GROUP; c < (g + 1) * ORACLE_GROUP; c++)
                    s += (int32_t)w[r * k + c] * (int32_t)x[mi * k + c];
                acc[(mi * n + r) * ng + g] = s;
            }
}

/* y[mi][r] = (float) sum_g (double) scale[r][g] * (double) acc[mi][r][g], groups in ascending order. */
void oracle_combine(const int32_t *acc, const uint16_t *scales, int64_t n, int64_t ng, int64_t m, float *y) {
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++) {
            double s = 0.0;
            for (int64_t g = 0; g < ng; g++)
                s += oracle_half_to_double(scales[r * ng + g]) * (double)acc[(mi * n + r) * ng + g];
            y[mi * n + r] = (float)s;
        }
}

/* ---------- fp16 activations ---------- */

/*
 * The GEMV against fp16 activations: the weights are rebuilt as +-scale or 0 and multiplied with the
 * activations in floating point ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-B and
 * II-D: the AVX-512 path expands each ternary weight to +-s in fp16, the Xe2 kernel feeds fp16
 * weights and activations to its matrix engine). Here the definition is computed exactly: x is
 * decoded from IEEE binary16, each group's sum of +-x is exact in double (binary16 values span at
 * most 40 bits of significance), the group scale multiplies it exactly, groups are added in
 * ascending order and the row is rounded once to float. x16: binary16 bits [m][k].
 */
void oracle_gemv_f16(const int8_t *w, const uint16_t *scales, const uint16_t *x16, int64_t n, int64_t k, int64_t m,
                     float *y) {
    int64_t ng = k / ORACLE_GROUP;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++) {
            double total = 0.0;
            for (int64_t g = 0; g < ng; g++) {
                double s = 0.0;
                for (int64_t c = g * ORACLE_GROUP; c < (g + 1) * ORACLE_GROUP; c++)
                    s += (double)w[r * k + c] * oracle_half_to_double(x16[mi * k + c]);
                total += oracle_half_to_double(scales[r * ng + g]) * s;
            }
            y[mi * n + r] = (float)total;
        }
}

/* ---------- per-group int8 activation quantisation ---------- */

/* x: float [m][k] (finite values), k a multiple of 128. xq: int8 [m][k]; xs: float [m][k/128], the
 * group's activation scale sigma. Per group: a = max |x|; sigma = a / 127 (fp32); each code is
 * x / sigma (fp32) rounded to nearest-even and clamped to [-127, 127]; a = 0 gives sigma = 0 and
 * codes 0. */
void oracle_quantize_x(const float *x, int64_t m, int64_t k, int8_t *xq, float *xs) {
    int64_t ng = k / ORACLE_GROUP;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t g = 0; g < ng; g++) {
            const float *v = x + mi * k + g * ORACLE_GROUP;
            int8_t *q = xq + mi * k + g * ORACLE_GROUP;
            float a = 0.0f;
            for (int c = 0; c < ORACLE_GROUP; c++) {
                float t = fabsf(v[c]);
                if (t > a) a = t;
            }
            volatile float sigma = a / 127.0f; /* volatile: keep the fp32 rounding of each step */
            xs[mi * ng + g] = sigma;
            for (int c = 0; c < ORACLE_GROUP; c++) {
                int code = 0;
                if (a > 0.0f) {
                    volatile float ratio = v[c] / sigma;
                    float r = nearbyintf(ratio); /* default rounding mode: nearest, ties to even */
                    code = r > 127.0f ? 127 : r < -127.0f ? -127 : (int)r;
                }
                q[c] = (int8_t)code;
            }
        }
}

/* y[mi][r] = (float) sum_g ((double) scale[r][g] * (double) acc[mi][r][g]) * (double) xs[mi][g]:
 * the definition with each group's activation scale applied beside its weight scale, groups in
 * ascending order, rounded once. */
void oracle_combine_xs(const int32_t *acc, const uint16_t *scales, const float *xs, int64_t n, int64_t ng, int64_t m,
                       float *y) {
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t r = 0; r < n; r++) {
            double s = 0.0;
            for (int64_t g = 0; g < ng; g++)
                s += (oracle_half_to_double(scales[r * ng + g]) * (double)acc[(mi * n + r) * ng + g]) *
                     (double)xs[mi * ng + g];
            y[mi * n + r] = (float)s;
        }
}

/*
 * Row-at-a-time GEMV from packed bytes: decode one row with the unpackers above, then apply the
 * definition. This is what the CPU baseline times. Rows are independent, so they are spread over
 * threads when the library is built with OpenMP. fmt: 1 = BITCOS, 2 = five-trit, 3 = 2-bit.
 * For BITCOS, `a` is the bitmap, `b` the sign stream and rowoff the per-row sign positions;
 * for the other formats `a` holds the codes and `b`, rowoff are unused. Returns 0 or -1.
 */
int oracle_gemv_packed(int fmt, const uint8_t *a, const uint8_t *b, const uint32_t *rowoff, const uint16_t *scales,
                       int64_t n, int64_t k, const int8_t *x, int64_t m, float *y) {
    if (k % ORACLE_GROUP) return -1;
    int64_t ng = k / ORACLE_GROUP;
    int bad = 0;
#pragma omp parallel
    {
        int8_t wrow[65536];
        int32_t acc[512];
#pragma omp for schedule(static)
        for (int64_t r = 0; r < n; r++) {
            if (k > 65536) { bad = 1; continue; }
            if (fmt == 1) {
                int64_t j = rowoff[r];
                for (int64_t c = 0; c < k; c++) {
                    if (get_bit(a, r * k + c)) { wrow[c] = get_bit(b, j) ? -1 : 1; j++; }
                    else wrow[c] = 0;
                }
                if (j != (int64_t)rowoff[r + 1]) bad = 1;
            } else if (fmt == 2) {
                if (oracle_t5_unpack(a + r * ng * 26, 1, k, wrow)) bad = 1;
            } else if (fmt == 3) {
                if (oracle_b2_unpack(a + r * (k / 4), 1, k, wrow)) bad = 1;
            } else {
                bad = 1;
            }
            for (int64_t mi = 0; mi < m; mi++) {
                oracle_gemv_acc(wrow, 1, k, x + mi * k, 1, acc);
                double s = 0.0;
                for (int64_t g = 0; g < ng; g++) s += oracle_half_to_double(scales[r * ng + g]) * (double)acc[g];
                y[mi * n + r] = (float)s;
            }
        }
    }
    return bad ? -1 : 0;
}

/* Threads later parallel regions of this library use (n >= 1; no effect without OpenMP). Used to time
 * the CPU baseline on one core and on all cores; it changes no result. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads an OpenMP parallel region of this library uses (1 without OpenMP). */
int oracle_threads(void) {
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
