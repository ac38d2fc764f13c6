// C ABI entry points that enqueue GPU work: argument checks, then dispatch to the kernels.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "tg_internal.h"

namespace tg {

int device_cus() {
    // One entry per device ordinal: the compute-unit count is a fixed property of the device, so the
    // cache is written at most once per entry with the same value, and concurrent first calls on
    // several threads only race to store that value (relaxed atomics keep the accesses well defined).
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
    if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

Problem make_problem(const tg_desc *d, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                     int32_t *acc, const float *xs) {
    const uint8_t *base = (const uint8_t *)W;
    Problem p{};
    p.codes = base + d->off_codes;
    p.codes_bytes = (uint32_t)d->bytes_codes;
    if (d->fmt == TG_FMT_BITCOS) {
        p.signs = (const uint32_t *)(base + d->off_signs);
        p.sign_bytes = (uint32_t)d->bytes_signs;
        p.rowoff = (const uint32_t *)(base + d->off_index);
    }
    p.scales = scales;
    p.x = x;
    p.y = y;
    p.acc = acc;
    p.xs = xs;
    p.n = (int32_t)d->n;
    p.k = (int32_t)d->k;
    if (d->fmt == TG_FMT_T5B) memcpy(&p.tscale, &d->tensor_scale, 4);
    if (d->fmt == TG_FMT_BITCOS) p.empty_rows = (int32_t)d->empty_rows;
    return p;
}

}  // namespace tg

using namespace tg;

namespace {

constexpr int kVectorMaxM = 3;  // activation rows one vector-path launch handles

// The kernels address each section with 32-bit byte offsets, and their switched-off accesses use
// offsets of 2^31 and more: bitmaps/codes, scales and outputs must stay below 1 GiB, sign windows
// (positions counted in bits) below 512 MiB.
bool fits_offsets(const tg_desc *d, int32_t m) {
    const uint64_t lim = 1ull << 30;
    const uint64_t ng = (uint64_t)groups_per_row(d->fmt, d->k);
    return d->bytes_codes < lim && d->bytes_signs < (lim >> 1) && (uint64_t)d->n * ng * 4 * (uint64_t)m < lim &&
           (uint64_t)d->n * 4 * (uint64_t)m < lim &&
           (uint64_t)m * (uint64_t)d->k <= lim;
}

// Whether a BITCOS GEMV with m activation rows and k-long rows runs on the matrix-core kernel (in one
// launch for all m rows): always from kMfmaAlwaysM rows, and at kMfmaMinM rows for long rows.
bool use_mfma(int fmt, int32_t m, int64_t k) {
    return fmt == TG_FMT_BITCOS &&
           (m >= kMfmaAlwaysM || (m >= kMfmaMinM && k / TG_GROUP > kMfmaLongRowGroups));
}

// The same choice for fp16 activations: matrix cores from kF16MfmaMinM rows, and at two rows for
// long rows (measured on MI355X, z = 0.44, 96 copies: 4096 x 14336 at m = 2 runs 1.27 TB/s on the
// fp16 vector kernel, whose chunked rows reload 256-byte activation slices per pass, against
// 2.34 TB/s for the matrix-core kernel at m = 4).
bool use_mfma_f16(int32_t m, int64_t k) {
    return m >= kF16MfmaMinM || (m == 2 && k / TG_GROUP > kMfmaLongRowGroups);
}

// Work geometry of one GEMV for a launch of m activation rows on the chosen path (chunk: the unit
// size of chunked BITCOS rows at m = 1).
void geometry(Problem &p, int fmt, int32_t m, bool mfma, int chunk = kChunkCoarse, bool f16 = false,
              bool short_units = false) {
    if (mfma)
        mfma_geometry(p, mfma_tiles(m, f16));
    else
        gemv_geometry(p, fmt, m, chunk, f16, short_units);
}

// A BITCOS launch of two activation rows on the vector path runs 12 waves per CU with two-step units
// when none of its GEMVs has chunked rows (more than 64 groups per row): with two-step units chunked
// rows would reload their activation slices twice as often (measured on MI355X: a Llama3-8B layer plan
// at m = 2 23 % slower), while single-chunk shapes gained 3-14 % (4096x4096 +7-9 %, 1024x4096 +13 %,
// 2560x2560 +14 %) over 8 waves with four-step units.
bool short_units_ok(int fmt, int32_t m, int64_t max_groups_per_row) {
    return fmt == TG_FMT_BITCOS && m == 2 && max_groups_per_row <= 64;
}

// Extra cost per row of a chunk pass of the vector path, in steps: the lanes reload their activation
// slice once per pass of a unit, shared by its rows (measured on MI355X over the Llama3-8B layer set:
// about two steps per pass for BITCOS, whose steps are longer, four for the fixed-size codes).
double pass_cost(int fmt, int rows_per_unit) { return (fmt == TG_FMT_BITCOS ? 2.0 : 4.0) / rows_per_unit; }

// Cost of a whole unit of p in steps (the last unit may be shorter), as unit_cost counts it without
// empty-row credit.
double full_unit_cost(const Problem &p, int fmt) {
    if (p.nch == 1) return (double)p.nbu;
    return (double)p.rpu * ((double)p.nch + pass_cost(fmt, p.rpu));
}

// Unit size of chunked BITCOS rows at m = 1 for a launch over these GEMVs (coarse geometry filled in).
// Fine units when the coarse ones are fewer than the launch's waves: some waves would get none and
// the few holding chunked units (a whole 8-row unit each) set the launch time (measured on MI355X: a
// single 4096 x 14336 call 18.1 -> 14.7 us, a plan of 32 such GEMVs 24.0 -> 19.7 us per launch). Mid
// units when there are enough units but a coarse chunked unit costs more than 1.5 times a wave's
// share of the launch: a one-layer Llama3-8B plan (7 GEMVs, ~7 steps per wave) gives each 4096 x 14336
// unit 18 steps, and the waves holding one finish ~10 us after the median wave (per-wave timestamps).
int chunk_units(const std::vector<Problem> &ps, int fmt, int32_t m, bool mfma, int waves) {
    if (mfma || fmt != TG_FMT_BITCOS || m != 1) return kChunkCoarse;
    int64_t units = 0;
    bool chunked = false;
    double total = 0, longest = 0;
    for (const Problem &p : ps) {
        units += p.nunits;
        chunked = chunked || p.nch > 1;
        const double c = full_unit_cost(p, fmt);
        total += c * (double)p.nunits;
        if (p.nch > 1) longest = std::max(longest, c);
    }
    if (!chunked) return kChunkCoarse;
    if (units < waves) return kChunkFine;
    return longest > 1.5 * total / (double)waves ? kChunkMid : kChunkCoarse;
}

hipError_t launch(int fmt, const GroupArgs &g, int out, bool mfma, hipStream_t s) {
    if (mfma) return launch_bitcos_mfma(g, out, s);
    switch (fmt) {
        case TG_FMT_BITCOS: return launch_bitcos(g, out, s);
        case TG_FMT_5TRIT: return launch_t5(g, out, s);
        case TG_FMT_2BIT: return launch_b2(g, out, s);
        case TG_FMT_T5B: return launch_t5b(g, out, s);
        default: return hipErrorInvalidValue;
    }
}

int gemv_common(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, const float *xs,
                float *y, int32_t *acc, int32_t m, void *stream, int out) {
    const bool acc_out = out == kOutAcc;
    if (!desc || !W || !x || m < 1 || m > TG_MAX_M) return TG_EINVAL;
    // t5b carries its scale in the descriptor: no per-group scales, and no activation group scales
    // (its 160-weight blocks do not follow the activations' 128-groups)
    const bool t5b = desc->fmt == TG_FMT_T5B;
    if (t5b && (scales || out == kOutYxs)) return TG_EINVAL;
    if (acc_out ? !acc : (!y || (!t5b && !scales))) return TG_EINVAL;
    if (out == kOutYxs && (!xs || ((uintptr_t)xs & 3))) return TG_EINVAL;
    // 16-byte vector loads of W sections and x rows; 4-byte stores of y / acc; 2-byte scales.
    if (((uintptr_t)W & 15) || ((uintptr_t)x & 15)) return TG_EINVAL;
    if (acc_out ? ((uintptr_t)acc & 3) : (((uintptr_t)y & 3) || ((uintptr_t)scales & 1))) return TG_EINVAL;
    int e = check_desc(desc, 0);
    if (e) return e;
    if (!fits_offsets(desc, m)) return TG_ESHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n = desc->n, k = desc->k, ng = groups_per_row(desc->fmt, k);
    // Activation rows go in launches of at most three on the vector path (each launch reads the
    // weights once); the matrix-core path takes all of them in one launch. Every launch is set up and
    // checked before the first one is enqueued, so an argument or geometry error enqueues nothing.
    const bool mfma = use_mfma(desc->fmt, m, desc->k);
    const int32_t step = mfma ? m : kVectorMaxM;
    GroupArgs gs[(TG_MAX_M + kVectorMaxM - 1) / kVectorMaxM];
    int nl = 0;
    const int cus = device_cus();
    for (int32_t m0 = 0; m0 < m; m0 += step) {
        const int32_t mt = std::min<int32_t>(step, m - m0);
        GroupArgs &g = gs[nl++];
        g = GroupArgs{};
        g.one = make_problem(desc, W, scales, x + (size_t)m0 * k, acc_out ? nullptr : y + (size_t)m0 * n,
                             acc_out ? acc + (size_t)m0 * n * ng : nullptr,
                             out == kOutYxs ? xs + (size_t)m0 * ng : nullptr);
        g.count = 1;
        g.m = mt;
        g.one.unit_begin = 0;
        g.short_units = !mfma && short_units_ok(desc->fmt, mt, ng) ? 1 : 0;
        geometry(g.one, desc->fmt, mt, mfma, kChunkCoarse, false, g.short_units != 0);
        const int chunk = chunk_units({g.one}, desc->fmt, mt, mfma, cus * gemv_waves(desc->fmt, mt));
        if (chunk != kChunkCoarse) geometry(g.one, desc->fmt, mt, mfma, chunk);
        g.rows_per_unit = g.one.rpu;
        g.units = g.one.nunits;
        g.live = desc->fmt == TG_FMT_BITCOS && (desc->empty_rows > 0 || desc->k == kWideLaneK) && mt == 1 && !mfma &&
                 out != kOutAcc;
        if (g.units < 1) return TG_ESHAPE;
    }
    // a 2-bit call of one activation row with fp32 or int32 outputs takes the table-free decode, as
    // 2-bit plans do by default
    const bool table_free = desc->fmt == TG_FMT_2BIT && m == 1 && !mfma && (out == kOutY || out == kOutAcc);
    for (int i = 0; i < nl; ++i)
        if ((table_free ? launch_table_free(desc->fmt, gs[i], out, s) : launch(desc->fmt, gs[i], out, mfma, s)) !=
            hipSuccess)
            return TG_EHIP;
    return TG_OK;
}

}  // namespace

extern "C" int ternary_gemv(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                            int32_t m, void *stream) {
    return gemv_common(desc, W, scales, x, nullptr, y, nullptr, m, stream, kOutY);
}

extern "C" int ternary_gemv_xs(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *xq,
                               const float *xs, float *y, int32_t m, void *stream) {
    return gemv_common(desc, W, scales, xq, xs, y, nullptr, m, stream, kOutYxs);
}

extern "C" int tg_quantize_x(const float *x, int32_t m, int64_t k, int8_t *xq, float *xs, void *stream) {
    if (!x || !xq || !xs || m < 1 || m > TG_MAX_M) return TG_EINVAL;
    if (((uintptr_t)x & 7) || ((uintptr_t)xq & 1) || ((uintptr_t)xs & 3)) return TG_EINVAL;
    if (k < TG_GROUP || k % TG_GROUP || k > (int64_t)1 << 30) return TG_ESHAPE;
    return launch_quantize_x(x, (int64_t)m * (k / TG_GROUP), xq, xs, (hipStream_t)stream) == hipSuccess ? TG_OK
                                                                                                      : TG_EHIP;
}

extern "C" int ternary_gemv_f16(const tg_desc *desc, const void *W, const uint16_t *scales, const uint16_t *x16,
                                float *y, int32_t m, void *stream) {
    if (!desc || !W || !scales || !x16 || !y || m < 1 || m > TG_MAX_M) return TG_EINVAL;
    if (desc->fmt != TG_FMT_BITCOS) return TG_EINVAL;
    if (((uintptr_t)W & 15) || ((uintptr_t)x16 & 15) || ((uintptr_t)y & 3) || ((uintptr_t)scales & 1))
        return TG_EINVAL;
    int e = check_desc(desc, 0);
    if (e) return e;
    // the fp16 rows take twice the bytes of int8 ones
    if (!fits_offsets(desc, m) || (uint64_t)m * (uint64_t)desc->k * 2 > (1ull << 30)) return TG_ESHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n = desc->n, k = desc->k;
    if (use_mfma_f16(m, k)) {  // all rows in one launch on matrix cores
        GroupArgs g{};
        g.one = make_problem(desc, W, scales, reinterpret_cast<const int8_t *>(x16), y, nullptr);
        g.count = 1;
        g.m = m;
        g.one.unit_begin = 0;
        mfma_geometry(g.one, mfma_tiles(m, true));
        g.rows_per_unit = g.one.rpu;
        g.units = g.one.nunits;
        return launch_bitcos_mfma_f16(g, s) == hipSuccess ? TG_OK : TG_EHIP;
    }
    for (int32_t m0 = 0; m0 < m; m0 += kF16MaxM) {
        const int32_t mt = std::min<int32_t>(kF16MaxM, m - m0);
        GroupArgs g{};
        g.one = make_problem(desc, W, scales, reinterpret_cast<const int8_t *>(x16 + (size_t)m0 * k),
                             y + (size_t)m0 * n, nullptr);
        g.count = 1;
        g.m = mt;
        g.one.unit_begin = 0;
        gemv_geometry(g.one, TG_FMT_BITCOS, mt, kChunkCoarse, true);
        const int chunk = chunk_units({g.one}, TG_FMT_BITCOS, mt, false, device_cus() * f16_waves(mt));
        if (chunk != kChunkCoarse) gemv_geometry(g.one, TG_FMT_BITCOS, mt, chunk, true);
        g.rows_per_unit = g.one.rpu;
        g.units = g.one.nunits;
        if (launch_bitcos_f16(g, s) != hipSuccess) return TG_EHIP;
    }
    return TG_OK;
}

extern "C" int ternary_gemv_acc(const tg_desc *desc, const void *W, const int8_t *x, int32_t *acc, int32_t m,
                                void *stream) {
    return gemv_common(desc, W, nullptr, x, nullptr, nullptr, acc, m, stream, kOutAcc);
}

namespace {

// Waves of a persistent launch on this device for m activation rows; a plan's per-wave ranges are
// sized for it (the table has room for the largest count).
// Waves of a vector-path (f16 = false) or matrix-core launch of m activation rows.
int plan_waves(int fmt, int m, bool mfma, bool f16 = false) {
    return device_cus() * (mfma ? mfma_waves(mfma_tiles(m, f16)) : gemv_waves(fmt, m));
}
int plan_waves_max() { return device_cus() * std::max(kMaxWavesPerCu, kMfmaWavesPerCu); }

// Largest m a plan of this format takes (one launch per plan).
int plan_max_m(int fmt) { return fmt == TG_FMT_BITCOS ? TG_MAX_M : kVectorMaxM; }

size_t ranges_offset(int32_t count) { return ((size_t)count * sizeof(Problem) + 255) / 256 * 256; }

// Relative time of work unit u of p, for splitting a plan's units across waves. Every step of the
// vector path costs about the same (one 128-weight group per lane, however many lanes are busy), so a
// unit costs its step count, plus the activation reloads of chunked rows; a unit of the matrix-core
// path costs its chunk count (all units of one plan take the same path).
// Steps per wave from which a launch takes the strong age-class shares (below). One-layer plans of
// the Llama3-8B-shaped layer (~7 steps per wave) run slower with them; one GPU's 8-way shard of the
// 32-layer set (~26 steps per wave) runs faster (+3.3 % in the first launches from idle, +2.6 %
// settled, against a threshold of 64), as do the longer launches.
constexpr double kLongRangeSteps = 16.0;

// Whether a launch's wave ranges are long (at least kLongRangeSteps of cost per wave) and not a
// row-walk build: such launches take the stronger issue-order shares.
bool long_ranges_of(double total_cost, int nw, bool live) {
    return !live && total_cost >= kLongRangeSteps * (double)nw;
}

double unit_cost(const Problem &p, int fmt, bool mfma, int64_t u, bool live) {
    const int64_t row0 = (u - p.unit_begin) * (int64_t)p.rpu;
    const int64_t rows = std::min<int64_t>(p.rpu, (int64_t)p.n - row0);
    if (mfma) return (double)((p.ng + 7) / 8);
    // A launch that walks only the rows with non-zeros skips the empty ones, but an empty row's step
    // costs less than a full one on the plain walk too (every lane reads the same table entries) and
    // the walk adds a little per step: counting an empty row as half a step balanced best on MI355X
    // (the 32B-shaped stack, against no credit and a full one, identical outputs).
    if (live && p.nch == 1 && p.k == kWideLaneK)
        return (double)rows * kWideLaneStepCost * (1.0 - 0.5 * (double)p.empty_rows / (double)p.n);
    if (live && p.nch == 1 && p.R == 1 && p.empty_rows > 0)
        return (double)rows * (1.0 - 0.5 * (double)p.empty_rows / (double)p.n);
    if (p.nch == 1) return (double)((rows + p.R - 1) / p.R);
    return (double)rows * ((double)p.nch + pass_cost(fmt, p.rpu));
}

}  // namespace

extern "C" size_t tg_plan_table_bytes(int32_t count) {
    return count > 0 ? ranges_offset(count) + (size_t)plan_waves_max() * sizeof(WaveRange) : 0;
}

namespace {

// Plan paths (tg_plan::path).
enum PlanPath { kPathVector = 0, kPathMfma = 1, kPathF16 = 2, kPathF16Mfma = 3, kPathVectorShort = 4 };

// Waves of a launch on `path`.
int path_waves(int fmt, int m, int path) {
    if (path == kPathF16) return device_cus() * f16_waves(m);
    if (path == kPathVectorShort) return device_cus() * kBitcosM2ShortWaves;
    return plan_waves(fmt, m, path == kPathMfma || path == kPathF16Mfma, path == kPathF16Mfma);
}

// Whether a plan may run the table-free decode (defined with tg_plan_set_decode below).
bool arith_ok(const tg_plan *p);

// f16: the x are fp16 activations (BITCOS, fp32 outputs; the fp16 vector kernel for m <= kF16MaxM,
// the fp16 matrix-core kernel from kF16MfmaMinM rows).
int plan_init_common(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                     const void *const *W, const uint16_t *const *scales, const int8_t *const *x,
                     const float *const *xs, float *const *y, int32_t *const *acc, int32_t m, bool f16 = false) {
    if (!plan || !table || !descs || !W || !x || count < 1 || m < 1) return TG_EINVAL;
    if (f16 && (descs[0].fmt != TG_FMT_BITCOS || acc || xs || m > TG_MAX_M)) return TG_EINVAL;
    const bool acc_mode = acc != nullptr;
    const int fmt = descs[0].fmt;
    const bool t5b = fmt == TG_FMT_T5B;  // scale in the descriptor; no activation group scales
    if (t5b && (scales || xs)) return TG_EINVAL;
    if (acc_mode ? xs != nullptr : (!y || (!t5b && !scales))) return TG_EINVAL;
    if (((uintptr_t)table & 15) || table_bytes < tg_plan_table_bytes(count)) return TG_EINVAL;
    if (m > plan_max_m(fmt)) return TG_EINVAL;
    std::vector<Problem> host((size_t)count);
    int rpu = 1;  // largest rows per unit (informational)
    for (int32_t i = 0; i < count; ++i) {
        const tg_desc *d = &descs[i];
        int e = check_desc(d, 0);
        if (e) return e;
        if (d->fmt != fmt) return TG_EINVAL;
        if (!fits_offsets(d, m) || (f16 && (uint64_t)m * (uint64_t)d->k * 2 > (1ull << 30))) return TG_ESHAPE;
        if (!W[i] || !x[i] || ((uintptr_t)W[i] & 15) || ((uintptr_t)x[i] & 15)) return TG_EINVAL;
        if (acc_mode ? (!acc[i] || ((uintptr_t)acc[i] & 3))
                     : (!y[i] || ((uintptr_t)y[i] & 3) || (!t5b && (!scales[i] || ((uintptr_t)scales[i] & 1)))))
            return TG_EINVAL;
        if (xs && (!xs[i] || ((uintptr_t)xs[i] & 3))) return TG_EINVAL;
    }
    for (int32_t i = 0; i < count; ++i) {
        const tg_desc *d = &descs[i];
        host[i] = make_problem(d, W[i], acc_mode || t5b ? nullptr : scales[i], x[i], acc_mode ? nullptr : y[i],
                               acc_mode ? acc[i] : nullptr, xs ? xs[i] : nullptr);
    }
    // One launch takes one path: the matrix-core kernel when every GEMV would take it on its own, or
    // (at m = kMfmaMinM) when the GEMVs that would take it hold most of the plan's weights.
    double w_mfma = 0, w_all = 0;
    for (int32_t i = 0; i < count; ++i) {
        const double wts = (double)descs[i].n * (double)descs[i].k;
        w_all += wts;
        if (f16 ? use_mfma_f16(m, descs[i].k) : use_mfma(fmt, m, descs[i].k)) w_mfma += wts;
    }
    const bool mfma = f16 ? m >= kF16MfmaMinM || (m == 2 && 2 * w_mfma > w_all)
                          : fmt == TG_FMT_BITCOS && m >= kMfmaMinM && (m >= kMfmaAlwaysM || 2 * w_mfma > w_all);
    int64_t max_groups = 0;
    for (int32_t i = 0; i < count; ++i) max_groups = std::max<int64_t>(max_groups, groups_per_row(fmt, descs[i].k));
    const bool short_units = !f16 && !mfma && short_units_ok(fmt, m, max_groups);
    const int path = f16 ? (mfma ? kPathF16Mfma : kPathF16) : mfma ? kPathMfma : short_units ? kPathVectorShort : kPathVector;
    // the row-walk build: some GEMV has empty rows to skip or rows of kWideLaneK weights (wide lanes)
    bool walk = false;
    for (int32_t i = 0; i < count; ++i) walk = walk || host[i].empty_rows > 0 || host[i].k == kWideLaneK;
    const bool live = fmt == TG_FMT_BITCOS && m == 1 && path == kPathVector && !acc_mode && walk;
    for (int32_t i = 0; i < count; ++i) geometry(host[i], fmt, m, mfma, kChunkCoarse, f16, short_units);
    {
        int64_t ub = 0;
        for (int32_t i = 0; i < count; ++i) {
            host[i].unit_begin = (int32_t)std::min<int64_t>(ub, 0x7FFFFFFF);
            ub += host[i].nunits;
        }
    }
    const int chunk = chunk_units(host, fmt, m, mfma, path_waves(fmt, m, path));
    if (chunk != kChunkCoarse)
        for (int32_t i = 0; i < count; ++i) geometry(host[i], fmt, m, mfma, chunk, f16, short_units);
    for (int32_t i = 0; i < count; ++i) rpu = std::max(rpu, (int)host[i].rpu);
    // Work order: GEMVs of one shape next to each other (by k, then n; the caller's order within a
    // shape). Each Problem carries its own pointers, so the order changes no result; on MI355X it
    // keeps the waves of a CU and of an XCD on one kind of work, which measured 15 % faster on the
    // Llama3-8B layer set than the layer-by-layer order (mixed shapes per CU run slower than the
    // same units grouped by shape).
    std::stable_sort(host.begin(), host.end(), [](const Problem &a, const Problem &b) {
        return a.k != b.k ? a.k < b.k : a.n < b.n;
    });
    int64_t units = 0;
    for (int32_t i = 0; i < count; ++i) {
        host[i].unit_begin = (int32_t)units;
        units += host[i].nunits;
        if (units > 0x7FFFFFFF) return TG_ESHAPE;
    }
    double total_cost = 0;
    for (int32_t i = 0; i < count; ++i)
        for (int64_t u = host[i].unit_begin; u < host[i].unit_begin + host[i].nunits; ++u)
            total_cost += unit_cost(host[i], fmt, mfma, u, live);
    // Contiguous unit ranges per wave, balanced by the cost model above and by the issue order of
    // the SIMDs: with 16 waves per CU, wave w of a block runs on SIMD w % 4, and a SIMD issues for its
    // oldest ready wave first, so of equal shares the block's waves 0-3 finish first and 12-15 last
    // (per-wave timestamps of the Llama3-8B layer-set step: 225, 252, 289 and 332 us, every CU alike).
    // Shares by wave w / 4 narrow that. Launches of many steps per wave take 1.30 : 1.10 : 0.90 : 0.70
    // (measured on MI355X against 1.12 : 1.04 : 0.96 : 0.88, alternating builds, three runs: the
    // Llama3-8B step +2.1-2.3 % in the first launches from idle and +1.9-2.8 % settled; 1.40 : ... : 0.60
    // no better), launches of few steps per wave the milder ones (one-layer plans, ~7 steps per wave,
    // ran 1.8-2.6 % slower with the strong shares), and so do launches of the row-walk build (the
    // 32B-shaped stack: +1.6 % in the first launches but -0.4 to -1.4 % settled with the strong ones)
    // and 2-bit plans (the layer set with the LDS table: -6.1 % in the first launches and -4.0 %
    // settled with the strong shares; table-free +0.3 / +0.4 %; five-trit gains +0.7 / +2.7 %, t5b
    // +3.9 / +2.9 %). The same order holds with 12 waves per CU (three per SIMD: m = 2 with two-step
    // units) and 8 (two per SIMD: the thin-batch matrix-core launches of two-tile units); for their
    // long launches, measured on 96-copy plans of 14336 x 4096 and 4096 x 14336 (settled, alternating
    // builds, two runs): 12 waves with 1.30 : 1.00 : 0.70 +3.6-3.7 % against equal shares (1.20 : 1.00
    // : 0.80 +1.2-3.6 %); 8 waves with 1.15 : 0.85 +0.3-2.7 % for 4096 x 14336 at m = 2, 4, 8 and -1.0
    // to +0.7 % for 14336 x 4096 (1.20 : 0.80: -3 to -6 %); the fp16 matrix-core launches (8 waves)
    // with 1.15 : 0.85 +3.2-3.5 % at m = 4, +1.4-2.0 % at m = 8, -0.5-0 % at m = 16 (both shapes).
    // The other 12- and 8-wave launches against equal shares (same plans): fp16 activations at m = 1
    // (12 waves) +4.9 / +2.6 % (14336 x 4096 / 4096 x 14336) and m = 2 +4.9 / +5.1 %, five-trit
    // m = 2 (12) +7.0 / +3.0 % and m = 3 (8) +5.4 / +2.4 %; but 2-bit m = 2 (8) -8.4 / +2.4 % and
    // m = 3 (12) -14.3 / +1.8 %, so 2-bit plans keep equal shares there.
    // Their short launches keep milder or equal shares. Six-wave launches (three-tile units,
    // m >= 16) leave SIMDs 2 and 3 with one wave each,
    // which runs ahead of the two pairs: their long launches take per-wave shares 1.05, 1.05, 1.15,
    // 1.15, 0.80, 0.80 (4096 x 14336 and 14336 x 4096 at m = 16: +5.1 and +5.9 % against equal
    // shares; 1.05 / 1.20 / 0.75 +4.8 and +3.4 %, 1.10 / 1.20 / 0.70 +4.1 and +3.3 %, 1.10 / 1.40 /
    // 0.50 -4 and -6 %).
    const int nw = path_waves(fmt, m, path);
    std::vector<WaveRange> ranges((size_t)nw);
    {
        const int wpb = path == kPathF16 ? f16_waves(m) : path == kPathVector ? gemv_waves(fmt, m)
                        : path == kPathVectorShort ? kBitcosM2ShortWaves
                        : path == kPathMfma ? mfma_waves(mfma_tiles(m, false))
                        : path == kPathF16Mfma ? mfma_waves(mfma_tiles(m, true)) : 0;
        const bool by_age = (wpb == 16 || ((wpb == 12 || wpb == 8) && fmt != TG_FMT_2BIT)) && nw % wpb == 0;
        // six waves: SIMDs 0 and 1 hold waves 0, 4 and 1, 5; SIMDs 2 and 3 hold waves 2 and 3 alone
        const bool by_wave6 = path == kPathMfma && wpb == 6 && nw % 6 == 0 && long_ranges_of(total_cost, nw, live);
        const double wave6_share[6] = {1.05, 1.05, 1.15, 1.15, 0.80, 0.80};
        const bool long_ranges = long_ranges_of(total_cost, nw, live);
        const double age16_long[4] = {1.30, 1.10, 0.90, 0.70}, age16_mild[4] = {1.12, 1.04, 0.96, 0.88};
        // 2-bit launches of few steps per wave (one-layer plans, table-free decode: 16.91 -> 16.09 us
        // per launch against the mild shares; BITCOS and five-trit within 1 %)
        const double age16_2bit_short[4] = {1.08, 1.03, 0.97, 0.92};
        const double *age16_short = fmt == TG_FMT_2BIT && !live && total_cost < kLongRangeSteps * (double)nw
                                        ? age16_2bit_short : age16_mild;
        const double age12_long[3] = {1.30, 1.00, 0.70}, age12_short[3] = {1.10, 1.00, 0.90};
        const double age8_long[2] = {1.15, 0.85}, age8_short[2] = {1.0, 1.0};
        const double *age_share = wpb == 16 ? (long_ranges && fmt != TG_FMT_2BIT ? age16_long : age16_short)
                                  : wpb == 12 ? (long_ranges ? age12_long : age12_short)
                                  : (long_ranges ? age8_long : age8_short);
        std::vector<double> cum((size_t)nw + 1, 0.0);
        for (int w = 0; w < nw; ++w)
            cum[w + 1] = cum[w] + (by_age ? age_share[(w % wpb) / 4] : by_wave6 ? wave6_share[w % 6] : 1.0);
        int32_t pi = 0;
        int64_t u = 0;
        double done = 0;
        for (int w = 0; w < nw; ++w) {
            ranges[w].begin = (int32_t)u;
            ranges[w].problem = pi;
            const double target = total_cost * cum[w + 1] / cum[nw];
            while (u < units) {
                while (pi + 1 < count && u >= host[pi + 1].unit_begin) ++pi;
                const double cost = unit_cost(host[pi], fmt, mfma, u, live);
                if (done + 0.5 * cost > target && w + 1 < nw) break;
                done += cost;
                ++u;
            }
            if (w + 1 == nw) u = units;
            ranges[w].end = (int32_t)u;
            ranges[w].reserved = 0;
            if (ranges[w].begin == ranges[w].end) ranges[w].problem = 0;
        }
    }
    std::vector<uint8_t> img(tg_plan_table_bytes(count), 0);
    memcpy(img.data(), host.data(), (size_t)count * sizeof(Problem));
    memcpy(img.data() + ranges_offset(count), ranges.data(), ranges.size() * sizeof(WaveRange));
    if (hipMemcpy(table, img.data(), img.size(), hipMemcpyHostToDevice) != hipSuccess) return TG_EHIP;
    memset(plan, 0, sizeof(*plan));
    plan->magic = TG_PLAN_MAGIC;
    plan->fmt = fmt;
    plan->m = m;
    plan->count = count;
    plan->units = (int32_t)units;
    plan->rows_per_unit = rpu;
    plan->acc_mode = acc_mode ? kOutAcc : xs ? kOutYxs : kOutY;
    plan->waves = nw;
    plan->path = path;
    plan->live_rows = live ? 1 : 0;
    plan->table = table;
    // 2-bit plans that the table-free decode serves take it by default: it reads no LDS table and
    // issues two instructions per four codes (faster from HBM and from the caches, measured)
    if (fmt == TG_FMT_2BIT && arith_ok(plan)) plan->decode = TG_DECODE_ARITH;
    return TG_OK;
}

}  // namespace

namespace tg {

int plan_init_into(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                   const void *const *W, const uint16_t *const *scales, const int8_t *const *x, float *const *y,
                   int32_t *const *acc, int32_t m) {
    return plan_init_common(plan, table, table_bytes, count, descs, W, scales, x, nullptr, y, acc, m);
}

}  // namespace tg

extern "C" int tg_plan_init(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                            const void *const *W, const uint16_t *const *scales, const int8_t *const *x,
                            float *const *y, int32_t *const *acc, int32_t m) {
    return plan_init_common(plan, table, table_bytes, count, descs, W, scales, x, nullptr, y, acc, m);
}

extern "C" int tg_plan_init_xs(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                               const void *const *W, const uint16_t *const *scales, const int8_t *const *xq,
                               const float *const *xs, float *const *y, int32_t m) {
    if (!xs) return TG_EINVAL;
    return plan_init_common(plan, table, table_bytes, count, descs, W, scales, xq, xs, y, nullptr, m);
}

extern "C" int tg_plan_init_f16(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                                const void *const *W, const uint16_t *const *scales, const uint16_t *const *x16,
                                float *const *y, int32_t m) {
    return plan_init_common(plan, table, table_bytes, count, descs, W, scales,
                            reinterpret_cast<const int8_t *const *>(x16), nullptr, y, nullptr, m, true);
}

namespace {

// Whether a plan may run the nibble-keyed decode.
bool nibble_ok(const tg_plan *p) {
    return p->fmt == TG_FMT_BITCOS && p->m == 1 && p->path == kPathVector &&
           (p->acc_mode == kOutY || p->acc_mode == kOutAcc);
}

// Whether a plan may run the table-free decode.
bool arith_ok(const tg_plan *p) {
    return (p->fmt == TG_FMT_5TRIT || p->fmt == TG_FMT_T5B || p->fmt == TG_FMT_2BIT) && p->m == 1 &&
           p->path == kPathVector &&
           (p->acc_mode == kOutY || p->acc_mode == kOutAcc);
}

bool decode_ok(const tg_plan *p, int32_t decode) {
    return decode == TG_DECODE_BYTE || (decode == TG_DECODE_NIBBLE && nibble_ok(p)) ||
           (decode == TG_DECODE_ARITH && arith_ok(p));
}

}  // namespace

extern "C" int tg_plan_set_decode(tg_plan *plan, int32_t decode) {
    if (!plan || plan->magic != TG_PLAN_MAGIC || !decode_ok(plan, decode)) return TG_EINVAL;
    plan->decode = decode;
    return TG_OK;
}

extern "C" int ternary_gemv_plan(const tg_plan *plan, void *stream) {
    if (!plan || plan->magic != TG_PLAN_MAGIC || !plan->table || plan->count < 1 || plan->m < 1 ||
        plan->m > plan_max_m(plan->fmt) || plan->acc_mode < kOutY || plan->acc_mode > kOutYxs ||
        plan->path < kPathVector || plan->path > kPathVectorShort ||
        (plan->path == kPathVectorShort && (plan->fmt != TG_FMT_BITCOS || plan->m != 2)) ||
        (plan->path == kPathMfma && (plan->fmt != TG_FMT_BITCOS || plan->m < kMfmaMinM)) ||
        (plan->path == kPathF16 && (plan->fmt != TG_FMT_BITCOS || plan->m > kF16MaxM || plan->acc_mode != kOutY)) ||
        (plan->path == kPathF16Mfma &&
         (plan->fmt != TG_FMT_BITCOS || plan->m < 2 || plan->acc_mode != kOutY)) ||
        !decode_ok(plan, plan->decode) ||
        (plan->live_rows != 0 && (plan->live_rows != 1 || plan->fmt != TG_FMT_BITCOS || plan->m != 1 ||
                                  plan->path != kPathVector || plan->acc_mode == kOutAcc)) ||
        (plan->table_gen != 0 && !static_table_current(plan->table, plan->table_gen)))
        return TG_EINVAL;
    GroupArgs g{};
    g.table = (const Problem *)plan->table;
    const bool mfma = plan->path == kPathMfma;
    if (plan->waves != path_waves(plan->fmt, plan->m, plan->path)) return TG_EINVAL;  // built for another device
    g.ranges = (const WaveRange *)((const uint8_t *)plan->table + ranges_offset(plan->count));
    g.waves = plan->waves;
    g.count = plan->count;
    g.units = plan->units;
    g.m = plan->m;
    g.rows_per_unit = plan->rows_per_unit;
    g.live = plan->live_rows;
    g.short_units = plan->path == kPathVectorShort ? 1 : 0;
    if (plan->decode == TG_DECODE_NIBBLE)
        return launch_bitcos_nibble(g, plan->acc_mode, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
    if (plan->decode == TG_DECODE_ARITH)
        return launch_table_free(plan->fmt, g, plan->acc_mode, (hipStream_t)stream) == hipSuccess ? TG_OK
                                                                                                         : TG_EHIP;
    if (plan->path == kPathF16) return launch_bitcos_f16(g, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
    if (plan->path == kPathF16Mfma)
        return launch_bitcos_mfma_f16(g, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
    return launch(plan->fmt, g, plan->acc_mode, mfma, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
}

extern "C" int tg_clock_probe(uint64_t *out, uint32_t slot, uint32_t spin_ticks, void *stream) {
    if (!out || ((uintptr_t)out & 7) || spin_ticks > 100000000u) return TG_EINVAL;
    return launch_clock_probe(out, slot, spin_ticks, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
}

extern "C" int tg_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks, int32_t unroll,
                              void *stream) {
    if (!buf || !sink || blocks < 1 || ((uintptr_t)buf & 15) || bytes == 0 || bytes > 0xFFFFFFFFull || bytes % 16)
        return TG_EINVAL;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return TG_EINVAL;
    return launch_stream_read(buf, (uint32_t)bytes, sink, blocks, unroll, (hipStream_t)stream) == hipSuccess ? TG_OK
                                                                                                        : TG_EHIP;
}
