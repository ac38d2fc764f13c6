// Internal declarations shared by the host packers, the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ternary_gemv.h"

namespace tg {

constexpr uint64_t kAlign = 256;      // section alignment inside a packed buffer
// Zero bytes after the sign stream (and after the fixed codes). The kernels read these sections
// through buffer resources that end with the section (the thin-batch kernel's sign stretches: with the
// row index after it), so a window or stretch that runs past the stream's end reads zeros whatever its
// length (the vector kernels' 4-dword windows, the thin-batch kernel's 36-dword stretches); the pad
// keeps a 16-byte read that starts in the stream inside the packed buffer for plain loads too.
constexpr uint64_t kSignPad = 16;

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// t5b: weights per block (one group of the kernels' work geometry) and blocks per row of k weights.
constexpr int kT5bBlock = 160;
inline constexpr uint64_t t5b_blocks(uint64_t k) { return (k + kT5bBlock - 1) / kT5bBlock; }

// Per-row group count of a format: 128-weight scale groups, or t5b's 160-weight blocks.
inline constexpr int64_t groups_per_row(int fmt, int64_t k) {
    return fmt == TG_FMT_T5B ? (int64_t)t5b_blocks((uint64_t)k) : k / TG_GROUP;
}

// One GEMV as the kernels see it: device pointers into one packed buffer plus the caller's
// scales, activations and outputs. Filled on the host from a checked descriptor.
struct Problem {
    const uint8_t *codes;     // bitmap (BITCOS) or code bytes (5-trit, 2-bit)
    const uint32_t *signs;    // BITCOS sign stream as little-endian dwords
    const uint32_t *rowoff;   // BITCOS per-row sign positions, n + 1 entries
    const uint16_t *scales;   // fp16 [n][k/128] (value path)
    const int8_t *x;          // int8 [m][k] (fp16 [m][k] on the fp16-activation path)
    float *y;                 // float [m][n] (value path)
    int32_t *acc;             // int32 [m][n][groups] (accumulator path)
    const float *xs;          // float [m][k/128] activation group scales (value path with them), else null
    uint32_t codes_bytes;     // bytes of the codes section
    uint32_t sign_bytes;      // bytes of the sign section
    int32_t n, k;             // rows, reduction length (k % 128 == 0)
    int32_t unit_begin;       // index of this GEMV's first work unit within its launch
    int32_t nunits;           // work units of this GEMV
    // work geometry (filled by gemv_geometry)
    int32_t ng;               // 128-groups per row
    int32_t nch;              // chunks of at most 64 groups per row
    int32_t G;                // groups per row in a full chunk (ng when nch == 1, else 64)
    int32_t R;                // rows per step (64 / ng when nch == 1, else 1)
    int32_t glast;            // groups per row in the last chunk
    int32_t nbu;              // steps per chunk pass of a unit (row bundles per unit)
    int32_t rpu;              // rows per unit (nbu * R)
    uint32_t gmagic;          // ceil(65536 / G): lane / G as (lane * gmagic) >> 16 for lane < 64
    uint32_t rmagic;          // ceil(65536 / R): likewise for R
    float tscale;             // t5b: the per-tensor scale (other formats: unused)
    int32_t empty_rows;       // BITCOS: rows without non-zeros the descriptor reports (a hint)
};

// Work units a wave processes: [begin, end), starting in GEMV `problem` of the table.
struct WaveRange {
    int32_t begin, end, problem, reserved;
};

// Arguments of one launch: either a single GEMV passed by value (table == nullptr) or a device
// table of `count` GEMVs sharing one format and one m, processed by one persistent grid.
struct GroupArgs {
    const Problem *table;
    const WaveRange *ranges;  // per-wave unit ranges (table mode); nullptr: equal contiguous shares
    int32_t count;
    int32_t units;            // total work units over all GEMVs
    int32_t m;                // activation rows (1 .. 3 on the vector path)
    int32_t rows_per_unit;    // unused (each GEMV's rows per unit are in Problem::rpu)
    int32_t waves;            // waves the launch must have (table mode: ranges has this many entries)
    int32_t live;             // BITCOS, m = 1, fp32 outputs: some GEMV reports rows without non-zeros,
                              // and the launch walks only the other rows of such GEMVs
    int32_t short_units;      // BITCOS, m = 2, no chunked rows: the 12-wave build with two-step units
    Problem one;
};

// Waves per CU of a vector-path GEMV launch for m activation rows (one block per CU: the decode
// tables fill most of the LDS): 16 at m = 1 (128 registers per lane); 12 for five-trit at m = 2 (168
// registers) and 2-bit at m = 3 (168); else 8. Measured against 8 waves with identical outputs, on
// single matrices (96 copies) and on the Llama3-8B layer set as one plan: five-trit at m = 2
// 4096x4096 +12 %, 14336x4096 +8 %, 2560x2560 +22 %, layer set +0.1 % (its chunked down unchanged);
// 2-bit at m = 3 +8 %, +8 %, +22 %, layer set +29 % (with 4-row units). 2-bit at m = 2 gained on
// single matrices (+2 %, +3 %, +21 %) but lost 3.8 % on the layer set, and BITCOS at m = 2 fits 12
// waves only with two-step units (its tables leave no room for a deeper tile), whose chunked rows
// reload the activation slices twice as often: a layer-set plan at m = 2 ran 23 % slower. Both keep 8,
// except that a BITCOS launch at m = 2 with no chunked rows takes the 12-wave build with two-step
// units (kBitcosM2ShortWaves; single-chunk shapes +3-14 % in that measurement).
constexpr int gemv_waves(int fmt, int m) {
    return (fmt == TG_FMT_5TRIT && m == 2) || (fmt == TG_FMT_2BIT && m == 3) ? 12 : m > 1 ? 8 : 16;
}
constexpr int kBitcosM2ShortWaves = 12;
constexpr int kMaxWavesPerCu = 16;

// BITCOS rows of this many weights (40 groups) at m = 1 with fp32 outputs run on the row-walk build
// of the kernel with a lane per 80 weights, so that a row fills the wave instead of 40 of its 64
// lanes; a step of such a row costs about kWideLaneStepCost of a step of group lanes (ten presence
// bytes per lane instead of sixteen) in the planner's balance.
constexpr int64_t kWideLaneK = 5120;
constexpr double kWideLaneStepCost = 0.8;

// Rows per unit of chunked BITCOS GEMVs at m = 1 (their row sums live in registers, not the tile).
constexpr int kChunkRows1 = 8;
// ... or of kChunkRows1Fine rows when units of kChunkRows1 are fewer than a launch's waves (small
// plans, single calls), or of kChunkRows1Mid rows when they are enough but each is so long against a
// wave's share of the launch that the waves holding one set its time (one-layer plans).
constexpr int kChunkRows1Fine = 2;
constexpr int kChunkRows1Mid = 4;
// Unit sizes of chunked BITCOS rows at m = 1 (gemv_geometry's `chunk` argument).
enum ChunkUnits { kChunkCoarse = 0, kChunkMid = 1, kChunkFine = 2 };

// Fill the work geometry of p (p.n, p.k set) for m activation rows on the vector path (the same for
// every format, except that chunked BITCOS rows at m = 1 go in units of kChunkRows1 (or, by `chunk`,
// kChunkRows1Mid or kChunkRows1Fine) rows and BITCOS
// units at m = 3 are two steps long; f16: the fp16-activation kernel, four-step units).
// short_units: two-step units of the 12-wave BITCOS build at m = 2 (single-chunk rows only).
void gemv_geometry(Problem &p, int fmt, int m, int chunk = kChunkCoarse, bool f16 = false, bool short_units = false);

// Thin-batch BITCOS path on matrix cores: m in [kMfmaMinM, TG_MAX_M] activation rows in one launch,
// units of kMfmaTiles tiles of 16 rows each over the whole row, kMfmaWavesPerCu waves per CU. It is
// taken from m = 3, and at m = 2 for rows of more than 64 groups (measured on MI355X, z = 0.44:
// 4096 x 14336 at m = 2 and 3 runs 1.23x and 2.6x faster there than on the vector kernel,
// 14336 x 4096 at m = 3 1.06x faster, at m = 2 1.2x slower).
constexpr int kMfmaMinM = 2;
constexpr int kMfmaAlwaysM = 3;  // from this m every BITCOS GEMV takes the matrix-core path
constexpr int kMfmaLongRowGroups = 64;  // at m = 2, rows of more groups than this take it
constexpr int kMfmaTiles = 2;
constexpr int kMfmaWavesPerCu = 8;
// From kMfmaWideM activation rows (int8 activations) the units take kMfmaTilesWide tiles at
// kMfmaWavesWide waves per CU (the LDS holds no more stages): each activation operand load then
// serves 48 weight rows instead of 32. Measured on MI355X (gate 14336x4096 and down 4096x14336, 96
// copies, alternating builds, identical outputs): at m = 16 gate 2228 -> 2385 GB/s and down 2177 ->
// 2260; at m = 14 within 1 %; at m = 10, 12 3-10 % slower, at m = 4, 8 13-17 % slower.
constexpr int kMfmaWideM = 16;
constexpr int kMfmaTilesWide = 3;
constexpr int kMfmaWavesWide = 6;
constexpr int mfma_tiles(int m, bool f16) { return !f16 && m >= kMfmaWideM ? kMfmaTilesWide : kMfmaTiles; }
constexpr int mfma_waves(int tiles) { return tiles == kMfmaTilesWide ? kMfmaWavesWide : kMfmaWavesPerCu; }
void mfma_geometry(Problem &p, int tiles);
hipError_t launch_bitcos_mfma(const GroupArgs &g, int out, hipStream_t s);

// Host-side checks of a descriptor; `limit` is the buffer length when known (0 = trust bytes_total).
int check_desc(const tg_desc *d, uint64_t limit);

// Fill a Problem from a checked descriptor and the caller's pointers.
Problem make_problem(const tg_desc *d, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                     int32_t *acc, const float *xs = nullptr);


// What a GEMV launch writes: fp32 y, the int32 per-group accumulators, or fp32 y with each group's
// term also multiplied by its activation group scale xs[m][g].
enum OutMode { kOutY = 0, kOutAcc = 1, kOutYxs = 2 };

// Kernel launchers (asynchronous; return the HIP status of the launch). `g.one` or `g.table` holds
// the problems; the launchers set grid sizes themselves.
hipError_t launch_bitcos(const GroupArgs &g, int out, hipStream_t s);
hipError_t launch_t5(const GroupArgs &g, int out, hipStream_t s);
hipError_t launch_b2(const GroupArgs &g, int out, hipStream_t s);
hipError_t launch_t5b(const GroupArgs &g, int out, hipStream_t s);
// The table-free decode (five-trit, t5b or 2-bit; m = 1, fp32 y or int32 accumulators).
hipError_t launch_table_free(int fmt, const GroupArgs &g, int out, hipStream_t s);

// BITCOS GEMV at m = 1 with the nibble-keyed decode (fp32 y or int32 accumulators; same geometry).
hipError_t launch_bitcos_nibble(const GroupArgs &g, int out, hipStream_t s);

// BITCOS GEMV against fp16 activations (Problem::x then points to fp16 [m][k]; fp32 y): launches of
// at most kF16MaxM activation rows, f16_waves(m) waves per CU, vector-path geometry. At m = 1 the
// kernel fits 168 registers and 12 waves share a CU; two rows need 253 registers (8 waves).
constexpr int kF16MaxM = 2;
constexpr int f16_waves(int m) { return m == 1 ? 12 : 8; }
hipError_t launch_bitcos_f16(const GroupArgs &g, hipStream_t s);
// ... and on matrix cores (the thin-batch kernel with fp16 operands, mfma_geometry, 1 <= m <= 16),
// taken from kF16MfmaMinM activation rows, and at two rows for rows of more than kMfmaLongRowGroups
// groups.
constexpr int kF16MfmaMinM = 3;
hipError_t launch_bitcos_mfma_f16(const GroupArgs &g, hipStream_t s);

// Per-group int8 quantisation of `groups` runs of 128 fp32 activations (one wave per group).
hipError_t launch_quantize_x(const float *x, int64_t groups, int8_t *xq, float *xs, hipStream_t s);

// Streaming-read reference kernel (bandwidth ceiling probe).
hipError_t launch_stream_read(const void *buf, uint32_t bytes, uint32_t *sink, int blocks, int unroll, hipStream_t s);
// Clock probe: one wave writes four counter samples to out[4 slot .. 4 slot + 3].
hipError_t launch_clock_probe(uint64_t *out, uint32_t slot, uint32_t spin, hipStream_t s);

// Number of compute units of the current device (cached).
int device_cus();

// tg_plan_init writing its table into `table` (the body shared with tg_plan_init_noalloc).
int plan_init_into(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                   const void *const *W, const uint16_t *const *scales, const int8_t *const *x, float *const *y,
                   int32_t *const *acc, int32_t m);

// Whether `table` is the current device's static plan table and still holds generation `gen` (the
// contents tg_plan_init_noalloc wrote for the plan that carries it).
bool static_table_current(const void *table, uint32_t gen);

}  // namespace tg
