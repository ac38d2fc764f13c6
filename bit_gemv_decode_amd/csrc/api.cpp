// C ABI entry points that enqueue GPU work: argument checks, then dispatch to the kernels.
#include <string.h>

#include <algorithm>
#include <vector>

#include "tg_internal.h"

namespace tg {

int bitcos_rows_per_unit(int64_t n, int64_t k, int m);

int device_cus() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached = cus;
        else
            return 256;
    }
    return cached;
}

Problem make_problem(const tg_desc *d, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                     int32_t *acc) {
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
    p.n = (int32_t)d->n;
    p.k = (int32_t)d->k;
    return p;
}

int rows_per_unit(int fmt, int64_t n, int64_t k, int m) {
    return fmt == TG_FMT_BITCOS ? bitcos_rows_per_unit(n, k, m) : 1;
}

}  // namespace tg

using namespace tg;

namespace {

constexpr int kVectorMaxM = 3;  // activation rows one vector-path launch handles

// The kernels address every section with 32-bit byte offsets.
bool fits_offsets(const tg_desc *d, int32_t m) {
    const uint64_t lim = 0xFFFFFFFFull;
    return d->bytes_codes <= lim && d->bytes_signs <= lim && (uint64_t)d->n * (uint64_t)(d->k / TG_GROUP) * 2 <= lim &&
           (uint64_t)m * (uint64_t)d->k <= lim;
}

hipError_t launch(int fmt, const GroupArgs &g, bool acc_out, hipStream_t s) {
    switch (fmt) {
        case TG_FMT_BITCOS: return launch_bitcos(g, acc_out, s);
        case TG_FMT_5TRIT: return launch_t5(g, acc_out, s);
        case TG_FMT_2BIT: return launch_b2(g, acc_out, s);
        default: return hipErrorInvalidValue;
    }
}

int gemv_common(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, float *y, int32_t *acc,
                int32_t m, void *stream, bool acc_out) {
    if (!desc || !W || !x || m < 1 || m > TG_MAX_M) return TG_EINVAL;
    if (acc_out ? !acc : (!y || !scales)) return TG_EINVAL;
    // 16-byte vector loads of W sections and x rows; 4-byte stores of y / acc; 2-byte scales.
    if (((uintptr_t)W & 15) || ((uintptr_t)x & 15)) return TG_EINVAL;
    if (acc_out ? ((uintptr_t)acc & 3) : (((uintptr_t)y & 3) || ((uintptr_t)scales & 1))) return TG_EINVAL;
    int e = check_desc(desc, 0);
    if (e) return e;
    if (!fits_offsets(desc, m)) return TG_ESHAPE;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n = desc->n, k = desc->k, ng = k / TG_GROUP;
    // Activation rows go in launches of at most three (each launch reads the weights once).
    for (int32_t m0 = 0; m0 < m; m0 += kVectorMaxM) {
        const int32_t mt = std::min<int32_t>(kVectorMaxM, m - m0);
        GroupArgs g{};
        g.one = make_problem(desc, W, scales, x + (size_t)m0 * k, acc_out ? nullptr : y + (size_t)m0 * n,
                             acc_out ? acc + (size_t)m0 * n * ng : nullptr);
        g.count = 1;
        g.m = mt;
        g.rows_per_unit = rows_per_unit(desc->fmt, n, k, mt);
        g.units = (int32_t)((n + g.rows_per_unit - 1) / g.rows_per_unit);
        g.one.unit_begin = 0;
        if (launch(desc->fmt, g, acc_out, s) != hipSuccess) return TG_EHIP;
    }
    return TG_OK;
}

}  // namespace

extern "C" int ternary_gemv(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, float *y,
                            int32_t m, void *stream) {
    return gemv_common(desc, W, scales, x, y, nullptr, m, stream, false);
}

extern "C" int ternary_gemv_acc(const tg_desc *desc, const void *W, const int8_t *x, int32_t *acc, int32_t m,
                                void *stream) {
    return gemv_common(desc, W, nullptr, x, nullptr, acc, m, stream, true);
}

extern "C" size_t tg_plan_table_bytes(int32_t count) {
    return count > 0 ? (size_t)count * sizeof(Problem) : 0;
}

extern "C" int tg_plan_init(tg_plan *plan, void *table, size_t table_bytes, int32_t count, const tg_desc *descs,
                            const void *const *W, const uint16_t *const *scales, const int8_t *const *x,
                            float *const *y, int32_t *const *acc, int32_t m) {
    if (!plan || !table || !descs || !W || !x || count < 1 || m < 1 || m > kVectorMaxM) return TG_EINVAL;
    const bool acc_mode = acc != nullptr;
    if (acc_mode ? false : (!y || !scales)) return TG_EINVAL;
    if (((uintptr_t)table & 15) || table_bytes < tg_plan_table_bytes(count)) return TG_EINVAL;
    const int fmt = descs[0].fmt;
    std::vector<Problem> host((size_t)count);
    int rpu = 1;
    for (int32_t i = 0; i < count; ++i) {
        const tg_desc *d = &descs[i];
        int e = check_desc(d, 0);
        if (e) return e;
        if (d->fmt != fmt) return TG_EINVAL;
        if (!fits_offsets(d, m)) return TG_ESHAPE;
        if (!W[i] || !x[i] || ((uintptr_t)W[i] & 15) || ((uintptr_t)x[i] & 15)) return TG_EINVAL;
        if (acc_mode ? (!acc[i] || ((uintptr_t)acc[i] & 3))
                     : (!y[i] || !scales[i] || ((uintptr_t)y[i] & 3) || ((uintptr_t)scales[i] & 1)))
            return TG_EINVAL;
        rpu = std::max(rpu, rows_per_unit(fmt, d->n, d->k, m));
    }
    // A table has plenty of work: use the largest batch every GEMV allows.
    if (fmt == TG_FMT_BITCOS) rpu = m == 1 ? 8 : 4;
    int64_t units = 0;
    for (int32_t i = 0; i < count; ++i) {
        const tg_desc *d = &descs[i];
        host[i] = make_problem(d, W[i], acc_mode ? nullptr : scales[i], x[i], acc_mode ? nullptr : y[i],
                               acc_mode ? acc[i] : nullptr);
        host[i].unit_begin = (int32_t)units;
        units += (d->n + rpu - 1) / rpu;
        if (units > 0x7FFFFFFF) return TG_ESHAPE;
    }
    if (hipMemcpy(table, host.data(), tg_plan_table_bytes(count), hipMemcpyHostToDevice) != hipSuccess)
        return TG_EHIP;
    memset(plan, 0, sizeof(*plan));
    plan->magic = TG_PLAN_MAGIC;
    plan->fmt = fmt;
    plan->m = m;
    plan->count = count;
    plan->units = (int32_t)units;
    plan->rows_per_unit = rpu;
    plan->acc_mode = acc_mode ? 1 : 0;
    plan->table = table;
    return TG_OK;
}

extern "C" int ternary_gemv_plan(const tg_plan *plan, void *stream) {
    if (!plan || plan->magic != TG_PLAN_MAGIC || !plan->table || plan->count < 1 || plan->m < 1 ||
        plan->m > kVectorMaxM)
        return TG_EINVAL;
    GroupArgs g{};
    g.table = (const Problem *)plan->table;
    g.count = plan->count;
    g.units = plan->units;
    g.m = plan->m;
    g.rows_per_unit = plan->rows_per_unit;
    return launch(plan->fmt, g, plan->acc_mode != 0, (hipStream_t)stream) == hipSuccess ? TG_OK : TG_EHIP;
}
