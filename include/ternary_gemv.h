/*
 * ternary_gemv.h -- C ABI of the MI355X (gfx950) ternary GEMV library.
 *
 * The operation ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C, the int8 path after
 * Fig. 5): int8 activations times a ternary {-1, 0, +1} weight matrix whose groups of 128 consecutive
 * reduction elements share one 16-bit scale. Dot products accumulate exactly in int32 per group and
 * the group scale is applied once per group:
 *
 *     acc[m][n][g] = sum_{k = 128 g}^{128 g + 127} W[n][k] * x[m][k]              (int32, exact)
 *     y[m][n]      = sum_g scale[n][g] * acc[m][n][g]                            (fp64 sum, fp32 store)
 *
 * W is n rows by k reduction elements (k a multiple of 128), x is m rows of k int8, y is m rows of
 * n floats. The weights are read straight from one of three packed formats:
 *
 *   TG_FMT_BITCOS -- "BITmap and COmpacted Signs" (same paper, Sec. II-A, Fig. 2, Eq. 1): a presence
 *       bitmap with one bit per weight (set where the weight is non-zero) plus a sign stream with one
 *       bit per non-zero weight, in the bitmap's storage order (the j-th sign bit belongs to the j-th
 *       set bit). 2 - z bits per weight at zero density z. Layout here: the bitmap is row-major, bit
 *       (r*k + c) of the bit stream is weight (r, c), packed LSB-first (the Eq. (2)-(3) example maps
 *       the first element to the least-significant bit); a sign bit of 1 marks -1. An index of n+1
 *       unsigned 32-bit sign positions (rowoff[r] = sign-stream position of row r's first non-zero,
 *       rowoff[n] = nnz) lets a row start decoding without scanning the rows before it.
 *   TG_FMT_5TRIT -- five ternary digits per byte (same paper, Sec. I; "Sub-Two-Bit Ternary Weight
 *       Storage with Table-Free Arithmetic Decoding", abstract): 3^5 = 243 <= 256, 26 bytes per
 *       128-weight group (1.625 bits per weight). Byte b of a group holds weights 5b..5b+4 as base-3
 *       digits d = w + 1, the first weight least significant; byte 25 holds weights 125..127 and two
 *       padding digits of value 1. Bytes >= 243 are invalid.
 *   TG_FMT_2BIT -- two bits per weight (Table I's "2-bit packing"): code c = w + 1, four codes per
 *       byte, the first weight in the lowest two bits. Code 3 is invalid.
 *   TG_FMT_T5B -- the five-trit code in blocks of 160 weights with one scale per tensor ("Sub-Two-Bit
 *       Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract: t5b, 32 bytes per
 *       block, 1.600 bits per weight). Block b of a row holds weights 160b .. 160b + 159; byte j of
 *       a block holds weights 160b + 5j .. + 4 as digits w + 1, the first weight least significant;
 *       positions past k are padding digits of value 1. The fp32 tensor scale is stored in the
 *       descriptor (tensor_scale); there are no per-group scales, and the per-group quantities
 *       (accumulators) are per 160-weight block: acc[m][n][ceil(k/160)], y = scale * sum_k W x.
 *
 * Scales are IEEE binary16, row-major [n][k/128], and are passed separately from the packed weights.
 *
 * Conventions
 *   - Every buffer is owned by the caller. The library allocates no device memory. Its only
 *     global state is a per-device cache of the compute-unit count (written once per device with
 *     the device's fixed value, atomically); all functions are re-entrant and thread-safe.
 *   - Functions return TG_OK (0) or a negative TG_E* code; tg_strerror() names it. Argument,
 *     descriptor and shape errors are detected before anything is enqueued, also for calls that
 *     issue several launches (five-trit, 2-bit and t5b with m > 3 run up to six launches of at
 *     most three activation rows: all of them are set up and checked before the first is
 *     enqueued). Only a failure of the HIP runtime itself while enqueuing (TG_EHIP) can leave
 *     earlier launches of such a call enqueued; their outputs are then partial.
 *   - Host functions (tg_pack_*, tg_describe, tg_validate, tg_unpack) take host pointers and are
 *     synchronous.
 *   - ternary_gemv / ternary_gemv_acc take a HOST copy of the packed buffer's descriptor and DEVICE
 *     pointers for everything else; they enqueue on `stream` (a hipStream_t passed as void*, NULL =
 *     the default stream) and return without synchronising. The format is not a separate argument:
 *     it is desc->fmt, and the descriptor carries what a bare format code could not (shape, zero
 *     count and section offsets within W), so a call cannot pair a format with the wrong layout.
 */
#ifndef TERNARY_GEMV_H
#define TERNARY_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_GROUP 128         /* reduction elements per scale group */
#define TG_MAX_M 16          /* most activation rows one ternary_gemv call accepts */
#define TG_MAGIC 0x53444754u /* "TGDS" little-endian: first word of every packed buffer */
#define TG_VERSION 1u
#define TG_HEADER_BYTES 256u /* the descriptor occupies the first 256 bytes of a packed buffer */

typedef enum { TG_FMT_BITCOS = 1, TG_FMT_5TRIT = 2, TG_FMT_2BIT = 3, TG_FMT_T5B = 4 } tg_fmt;

enum {
    TG_OK = 0,
    TG_EINVAL = -1,       /* null pointer, bad enum value, m outside [1, TG_MAX_M] */
    TG_ENOTTERNARY = -2,  /* a weight outside {-1, 0, +1} was given to a packer */
    TG_ESHAPE = -3,       /* n < 1, k < 1, k not a multiple of 128, or sizes that overflow the format */
    TG_EFORMAT = -4,      /* the buffer is not a packed buffer of this library/version */
    TG_ECORRUPT = -5,     /* a packed buffer whose contents contradict its descriptor */
    TG_ENOSPACE = -6,     /* the output buffer is smaller than required */
    TG_EHIP = -7          /* the HIP runtime reported an error while enqueuing */
};

/*
 * Descriptor stored in the first TG_HEADER_BYTES of every packed buffer (host byte order, i.e.
 * little-endian). Section offsets are in bytes from the start of the buffer and are 256-aligned.
 *   BITCOS: codes = bitmap (n*k/8 bytes), signs = sign stream (ceil(nnz/8) bytes followed by zero
 *           padding up to bytes_signs), index = rowoff (4*(n+1) bytes).
 *   5TRIT:  codes = n * (k/128) * 26 bytes, row-major by (row, group). No signs or index.
 *   2BIT:   codes = n * k / 4 bytes, row-major. No signs or index.
 *   T5B:    codes = n * ceil(k/160) * 32 bytes, row-major by (row, block). No signs or index;
 *           group = 160 (the block length; every other format has group = TG_GROUP).
 */
typedef struct tg_desc {
    uint32_t magic;      /* TG_MAGIC */
    uint32_t version;    /* TG_VERSION */
    int32_t fmt;         /* tg_fmt */
    int32_t group;       /* TG_GROUP */
    int64_t n;           /* rows */
    int64_t k;           /* reduction elements per row */
    uint64_t nnz;        /* non-zero weights (all formats) */
    uint64_t off_codes, bytes_codes;
    uint64_t off_signs, bytes_signs;
    uint64_t off_index, bytes_index;
    uint64_t bytes_total; /* whole buffer, header included */
    uint64_t bytes_payload; /* algorithmic bytes: codes + ceil(nnz/8) sign bytes + index (no padding, no header) */
    uint32_t tensor_scale;  /* TG_FMT_T5B: the per-tensor scale, IEEE binary32 bits; 0 otherwise */
    uint32_t empty_rows;    /* TG_FMT_BITCOS: rows without a non-zero weight (rowoff[r + 1] == rowoff[r]),
                               written by tg_pack_bitcos; 0 for the other formats. A hint only: the
                               m = 1 kernel walks only the other rows of a GEMV that reports some (and
                               stores 0 for these), and any value up to n gives the same results. */
    uint64_t reserved;
} tg_desc;

/*
 * Packers: convert a host int8 matrix W[n][k] (values in {-1, 0, +1}) into a packed buffer
 * (descriptor + sections). Two-call pattern: with out == NULL only *out_bytes is written (the size
 * needed); otherwise out must hold out_cap >= that size, and *out_bytes receives the size written.
 * Errors: TG_EINVAL (w or out_bytes NULL), TG_ESHAPE (n < 1, k < 1, k % 128 != 0, or more than
 * 2^32 - 1 non-zeros for BITCOS), TG_ENOTTERNARY, TG_ENOSPACE.
 */
int tg_pack_bitcos(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes);
int tg_pack_5trit(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes);
int tg_pack_2bit(const int8_t *w, int64_t n, int64_t k, void *out, size_t out_cap, size_t *out_bytes);
/* t5b packer: as above, plus the per-tensor scale (finite; TG_EINVAL otherwise) stored in the
 * descriptor. k must be a multiple of 128 like every format of this library. */
int tg_pack_t5b(const int8_t *w, int64_t n, int64_t k, float scale, void *out, size_t out_cap, size_t *out_bytes);

/* Read and check the descriptor of a host packed buffer of `bytes` bytes (header fields only).
 * Errors: TG_EINVAL, TG_EFORMAT (magic/version/fmt/group wrong or bytes too small),
 * TG_ECORRUPT (sections that do not fit the buffer or do not match n, k, nnz). */
int tg_describe(const void *packed, size_t bytes, tg_desc *out);

/* Full content check of a host packed buffer: the descriptor, then every code (five-trit bytes < 243
 * with weight-0 padding digits, no 2-bit code 3) and, for BITCOS, rowoff[0] = 0, each row's index
 * step equal to that row's bitmap popcount, rowoff[n] = nnz. Returns TG_OK or the first error. */
int tg_validate(const void *packed, size_t bytes);

/* Decode a host packed buffer back to int8 W[n][k] (w_out holds n*k bytes); lossless. Validates
 * first (same errors as tg_validate). */
int tg_unpack(const void *packed, size_t bytes, int8_t *w_out);

/*
 * GPU GEMV (asynchronous). desc: host copy of the descriptor of the packed buffer whose device copy
 * is W (bytes_total bytes, the same image as the host buffer). scales: device fp16 [n][k/128] bit
 * patterns (TG_FMT_T5B: must be NULL, the tensor scale comes from the descriptor). x: device int8
 * [m][k]. y: device float [m][n]. 1 <= m <= TG_MAX_M.
 * Paths: the vector kernels (int8 dot products in int32, "Breaking the 1.58-bit Barrier for Ternary
 * LLMs", Sec. II-C) take up to three activation rows per launch; five-trit, 2-bit and t5b with m > 3
 * run them in launches of up to three rows. BITCOS with m >= 3, or m = 2 with k > 8192, takes the
 * thin-batch path instead: one launch decodes each weight once into int8
 * operands of int8 matrix-core products against X padded to 16 rows (a batch turns the GEMV into a
 * matrix product; the untitled page on a NUMA-aware decode engine for ternary models, Sec. 6.5 and
 * its appendix "Ternary GEMM on AMX", expands ternary weights into int8 matrix-engine tiles the same
 * way). Every path produces the same exact int32 group sums and the same fp32 outputs.
 * The kernels trust W's contents as far as its descriptor describes them (validate host buffers
 * with tg_validate before upload); every device read stays inside the sections the descriptor
 * names even for corrupt contents, so a corrupt buffer gives wrong numbers, not a fault.
 * Alignment: W and x 16-byte aligned, y / acc 4-byte aligned, scales 2-byte aligned.
 * Errors: TG_EINVAL (null or misaligned pointer, m out of range), TG_EFORMAT / TG_ECORRUPT
 * (descriptor), TG_EHIP (launch failure).
 */
int ternary_gemv(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                 int32_t m, void *stream);

/* Same contraction, but writes the exact int32 per-group accumulators acc[m][n][k/128] instead of y
 * (no scales). This is the bit-exact parity entry point. */
int ternary_gemv_acc(const tg_desc *desc, const void *W, const int8_t *x, int32_t *acc, int32_t m, void *stream);

/*
 * Activations quantised per group ("Breaking the 1.58-bit Barrier for Ternary LLMs", Sec. II-C, the
 * int8 path after Fig. 5: activations are quantised to int8 per group of 128 and each group's scale
 * is applied once per group, beside the weight scale). The page does not spell out the quantiser;
 * this library uses the symmetric absmax form.
 *
 * tg_quantize_x (device, asynchronous): x is device float [m][k] (finite values), k a multiple of 128,
 *   1 <= m <= TG_MAX_M. For each group of 128 consecutive elements of a row:
 *       sigma = max |x| / 127                       (IEEE fp32 division, nearest-even)
 *       xq    = clamp(rint_even(x / sigma), -127, 127)   (IEEE fp32 division), 0 where sigma = 0
 *   and writes xq (device int8 [m][k]) and xs (device float [m][k/128], the sigmas). The codes are
 *   decided in fp32, so they are exact and reproducible. Alignment: x 8 bytes, xq 2, xs 4.
 *   Errors: TG_EINVAL (null or misaligned pointer, m out of range), TG_ESHAPE (k < 128, k % 128 != 0
 *   or k > 2^30), TG_EHIP.
 *
 * ternary_gemv_xs (device, asynchronous): ternary_gemv on quantised activations xq with their group
 *   scales xs (device float [m][k/128], 4-byte aligned):
 *       y[m][n] = sum_g scale[n][g] * xs[m][g] * acc[m][n][g]     (each term exact in fp64, fp32 store)
 *   Same paths, arguments and errors as ternary_gemv; a null or misaligned xs is TG_EINVAL.
 */
int tg_quantize_x(const float *x, int32_t m, int64_t k, int8_t *xq, float *xs, void *stream);
int ternary_gemv_xs(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *xq, const float *xs,
                    float *y, int32_t m, void *stream);

/*
 * ternary_gemv_f16 (device, asynchronous): the BITCOS GEMV against fp16 activations ("Breaking the
 * 1.58-bit Barrier for Ternary LLMs", Sec. II-B: ternary weights rebuilt as +-1 or 0 in 16-bit
 * floating point and multiplied with the activations; Sec. II-D: lookup entries holding fp16
 * weights). x16: device binary16 [m][k] bit patterns (finite values), 16-byte aligned.
 *       y[m][n] = sum_g scale[n][g] * sum_{k in g} W[n][k] * x16[m][k]
 *   Each group sum is accumulated in fp32 (products exact, at most 128 roundings of partial sums no
 *   larger than sum_{k in g} |W x|), multiplied by the group scale in fp64 (exact), summed over
 *   groups in fp64 and stored as fp32:
 *       |y - y_exact| <= 2^-24 |y_exact| + 2^-17 * sum_g |scale[n][g]| * sum_{k in g} |W x|,
 *   and the parity checks accept |y - y_ref| <= 2^-22 |y_ref| + 2^-17 * sum_g |scale[n][g]| *
 *   sum_{k in g} |W x| against the correctly rounded value y_ref (derived in oracle/bounds.py).
 *   1 <= m <= TG_MAX_M. Paths: m = 1, and m = 2 with k <= 8192, run the vector kernel
 *   (v_dot2_f32_f16); from m = 3, and at m = 2 with k > 8192, one launch takes all rows on matrix
 *   cores (v_mfma_f32_16x16x32_f16, the decoded fp16 weights as the B operand, X padded to 16 rows
 *   as A). Non-finite activations are outside the
 *   contract.
 *   Errors: TG_EINVAL (null or misaligned pointer, m out of range, a format other than BITCOS),
 *   TG_EFORMAT / TG_ECORRUPT (descriptor), TG_ESHAPE (2 * m * k > 2^30), TG_EHIP.
 */
int ternary_gemv_f16(const tg_desc *desc, const void *W, const uint16_t *scales, const uint16_t *x16, float *y,
                     int32_t m, void *stream);

/*
 * Grouped launch: several GEMVs of one format and one activation-row count m (1 <= m <= 3; BITCOS
 * 1 <= m <= TG_MAX_M) run as
 * one persistent kernel. This is the batched form of the same operation (each GEMV is computed
 * exactly as ternary_gemv / ternary_gemv_acc compute it); it removes the per-launch ramp and lets
 * the memory pipeline stay full across matrices, e.g. the q/k/v or gate/up projections of a decode
 * step, or a whole layer stack in a benchmark.
 *
 * tg_plan_table_bytes(count): bytes of device memory the table of `count` GEMVs needs.
 * tg_plan_init: checks every descriptor and pointer (the same rules as ternary_gemv; all formats
 *   equal), chooses one path for the launch (BITCOS: the thin-batch kernel from m = 3, and at m = 2
 *   when GEMVs with k > 8192 hold most of the weights; at m = 2 with no such GEMV the vector kernel's
 *   12-wave build; else the vector kernels; plan->path records it), then writes the
 *   table into `table` (caller-owned DEVICE memory of at least tg_plan_table_bytes(count) bytes,
 *   16-byte aligned) with a synchronous host-to-device copy, and
 *   fills the host struct *plan. descs, W, scales, x, y, acc are host arrays of `count` entries;
 *   W/scales/x/y/acc entries are device pointers. Pass acc == NULL for fp32 outputs y (then y and
 *   scales are required), or acc != NULL for int32 accumulators (y and scales may be NULL).
 *   Errors: TG_EINVAL (null or misaligned pointer, mixed formats, count < 1, m outside the range
 *   above,
 *   table too small), TG_EFORMAT / TG_ECORRUPT (a descriptor), TG_ESHAPE (a section beyond 4 GiB),
 *   TG_EHIP (the copy failed). The plan stays valid while the table and every buffer it names do.
 * ternary_gemv_plan: enqueues all GEMVs of the plan on `stream` as one launch (asynchronous).
 *   The table splits the work for the GPU that was current at tg_plan_init; run the plan there.
 *   Errors: TG_EINVAL (not an initialised plan, or one made for a GPU with another CU count),
 *   TG_EHIP.
 */
#define TG_PLAN_MAGIC 0x4E4C5054u /* "TPLN" */

typedef struct tg_plan {
    uint32_t magic;      /* TG_PLAN_MAGIC once initialised */
    int32_t fmt;         /* tg_fmt shared by every GEMV */
    int32_t m;           /* activation rows of every GEMV */
    int32_t count;       /* GEMVs in the table */
    int32_t units;       /* work units over all GEMVs */
    int32_t rows_per_unit;
    int32_t acc_mode;    /* 0: fp32 y; 1: int32 accumulator outputs; 2: fp32 y with activation group scales */
    int32_t waves;       /* waves of the launch the table's work split was made for */
    int32_t path;        /* 0: vector kernels; 1: thin-batch matrix-core kernel (BITCOS); 2 / 3: fp16
                            activations on the vector / matrix-core kernel; 4: the vector kernel at 12
                            waves per CU with two-step units (BITCOS, m = 2, no GEMV with more than 64
                            groups per row) */
    int32_t decode;      /* TG_DECODE_BYTE, _NIBBLE or _ARITH (tg_plan_init*: _ARITH for 2-bit plans
                            that may take it, else _BYTE) */
    int32_t live_rows;   /* 1: the launch (BITCOS, m = 1, vector path, fp32 outputs, byte-keyed
                            decode) takes the row-walk kernel, because some GEMV reports rows without
                            non-zeros (tg_desc.empty_rows) or has rows of 5120 weights: it walks only
                            the non-empty rows of the GEMVs with one row per step, storing 0 for the
                            empty ones, and runs 5120-weight rows with a lane per 80 weights; 0
                            otherwise */
    uint32_t table_gen;  /* 0 for a caller-owned table; tg_plan_init_noalloc: the generation of the
                            library's static table this plan was written into */
    void *table;         /* device table written by tg_plan_init */
} tg_plan;

size_t tg_plan_table_bytes(int32_t count);
int tg_plan_init(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                 const void *const *W, const uint16_t *const *scales, const int8_t *const *x, float *const *y,
                 int32_t *const *acc, int32_t m);
/* tg_plan_init for ternary_gemv_xs outputs: every GEMV of the plan takes quantised activations xq[i]
 * and their group scales xs[i] (device float [m][k/128], 4-byte aligned) and writes fp32 y[i]. Same
 * rules and errors as tg_plan_init with acc == NULL; a null xs array or entry is TG_EINVAL. */
int tg_plan_init_xs(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                    const void *const *W, const uint16_t *const *scales, const int8_t *const *xq,
                    const float *const *xs, float *const *y, int32_t m);

/* tg_plan_init for ternary_gemv_f16 outputs: every GEMV of the plan is BITCOS and takes fp16
 * activations x16[i] (device binary16 [m][k], 16-byte aligned), 1 <= m <= TG_MAX_M; the launch runs
 * the fp16 vector kernel (path 2) or the fp16 matrix-core kernel (path 3: from m = 3, and at m = 2
 * when GEMVs with k > 8192 hold most of the weights), and each y is computed as ternary_gemv_f16
 * computes it. Errors as tg_plan_init, plus TG_EINVAL for another
 * format and TG_ESHAPE for 2 * m * k > 2^30. */
int tg_plan_init_f16(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                     const void *const *W, const uint16_t *const *scales, const uint16_t *const *x16,
                     float *const *y, int32_t m);
int ternary_gemv_plan(const tg_plan *plan, void *stream);

/*
 * tg_plan_init_noalloc: tg_plan_init for callers that cannot allocate device memory (code that runs
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * checks, work split and results as tg_plan_init, without the table argument: the table is written
 * into the library's own static device array of TG_NOALLOC_TABLE_BYTES (one per GPU the library runs
 * on, held until the process ends), with a synchronous hipMemcpy from host memory. It calls no
 * hipMalloc or hipFree and no other allocating HIP or library routine. The plan is run with
 * ternary_gemv_plan as usual.
 * Limit: tg_plan_table_bytes(count) <= TG_NOALLOC_TABLE_BYTES (about 1400 GEMVs on a 256-CU GPU);
 * larger counts return TG_ENOSPACE and leave the static table untouched.
 * Sharing: every GPU has one static table, and it keeps what the last successful call wrote. Each
 * call on a GPU whose count fits (successful or not) invalidates every plan made earlier by this
 * function on that GPU: ternary_gemv_plan refuses them with TG_EINVAL. Calls and launches that
 * overlap on one GPU race: a launch of an earlier static plan must have finished before the next
 * call on that GPU, and two threads must not call it for one GPU at the same time.
 * Errors: those of tg_plan_init, TG_ENOSPACE, and TG_EHIP when the static table's address cannot be
 * obtained.
 */
#define TG_NOALLOC_TABLE_BYTES (256u * 1024u)
int tg_plan_init_noalloc(tg_plan *plan, int32_t count, const tg_desc *descs, const void *const *W,
                         const uint16_t *const *scales, const int8_t *const *x, float *const *y,
                         int32_t *const *acc, int32_t m);

/*
 * Decode strategy of a plan. TG_DECODE_BYTE (the default, except for 2-bit plans below): table
 * lookups in LDS (BITCOS: one per presence byte in a byte-keyed table of 6561 entries; five-trit and
 * t5b: one per code byte in a 243-entry table; 2-bit: one per code byte in a 256-entry table). TG_DECODE_NIBBLE (BITCOS): the nibble-keyed lookup of "Breaking the 1.58-bit
 * Barrier for Ternary LLMs", Sec. II-D, Eq. 4 (key: a presence nibble and the next four compact sign
 * bits; entry: the nibble's 4 weights), one lookup per nibble in a 256-entry table.
 * TG_DECODE_ARITH (five-trit, t5b, 2-bit): no table. Five-trit and t5b: each base-3 digit of a code
 * byte is computed from the byte directly by multiply and shift (the depth-one, table-free decode of
 * "Sub-Two-Bit Ternary Weight Storage with Table-Free Arithmetic Decoding", abstract); 2-bit: the codes
 * are isolated by shift and mask and contracted as they are (the 2-bit expansion of "Breaking the
 * 1.58-bit Barrier for Ternary LLMs", Sec. II-C). Either way the group's activation sum is subtracted
 * once (weight = code - 1). Every strategy gives the same exact int32 group sums and the same fp32
 * outputs; they differ in speed. Invalid codes (five-trit bytes of 243 and above, 2-bit code 3; see
 * tg_validate) decode to unspecified weights under TG_DECODE_ARITH, to zeros under the table.
 * tg_plan_init* gives 2-bit plans that may take TG_DECODE_ARITH (below) that decode by default, and a
 * ternary_gemv / ternary_gemv_acc call on 2-bit weights with m = 1 uses it too: measured faster from
 * HBM and from the caches. tg_plan_set_decode(plan, TG_DECODE_BYTE) selects the table.
 * tg_plan_set_decode: TG_DECODE_NIBBLE is accepted for initialised BITCOS plans, TG_DECODE_ARITH for
 * five-trit, t5b and 2-bit plans, each with m = 1 on the vector path (path 0) writing fp32 y or int32
 * accumulators (tg_plan_init; not _xs); TG_EINVAL otherwise (the plan is then unchanged). Host only;
 * takes effect at the next ternary_gemv_plan.
 */
#define TG_DECODE_BYTE 0
#define TG_DECODE_NIBBLE 1
#define TG_DECODE_ARITH 2
int tg_plan_set_decode(tg_plan *plan, int32_t decode);

/*
 * Bandwidth reference (not part of the GEMV): reads `bytes` bytes of device memory at buf
 * (16-byte aligned, a multiple of 16, at most 4 GiB) with `blocks` workgroups of 4 waves, each lane
 * keeping `unroll` (1, 2, 4 or 8) 16-byte loads in flight, and writes one XOR word per wave to
 * sink (device, blocks * 4 words). Asynchronous. The GEMVs' effective bandwidth is reported
 * against the rate this reaches on the same GPU. Errors: TG_EINVAL, TG_EHIP.
 */
int tg_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks, int32_t unroll, void *stream);

/*
 * Clock reference (not part of the GEMV): one wave writes four 64-bit counter samples to
 * out[4 slot .. 4 slot + 3] (device, 8-byte aligned, the caller sizes it): the constant 100 MHz
 * counter and the shader-clock counter at its start, and both again once spin_ticks (at most 10^8) of
 * the constant counter have passed. Enqueued between other launches on one stream, consecutive
 * probes bracket those launches (durations in 10 ns ticks), and each probe's two deltas give the
 * shader clock at that moment. Asynchronous. Errors: TG_EINVAL, TG_EHIP.
 */
int tg_clock_probe(uint64_t *out, uint32_t slot, uint32_t spin_ticks, void *stream);

/* Static string for a TG_* code ("unknown error" for anything else). */
const char *tg_strerror(int code);

/* TG_VERSION of the loaded library. */
uint32_t tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_GEMV_H */
