// C ABI entry points that enqueue GPU work: argument checks, then dispatch to the kernels.
#include "tg_internal.h"

using namespace tg;

namespace {

int gemv_common(const tg_desc *desc, const void *W, const uint16_t *scales, const int8_t *x, float *y, int32_t *acc,
                int32_t m, void *stream, bool acc_out) {
    if (!desc || !W || !x || m < 1 || m > TG_MAX_M) return TG_EINVAL;
    if (acc_out ? !acc : (!y || !scales)) return TG_EINVAL;
    // 16-byte vector loads of W sections and x rows; 4-byte stores of y / acc; 2-byte scales.
    if (((uintptr_t)W & 15) || ((uintptr_t)x & 15)) return TG_EINVAL;
    if (acc_out ? ((uintptr_t)acc & 3) : (((uintptr_t)y & 3) || ((uintptr_t)scales & 1))) return TG_EINVAL;
    int e = check_desc(desc, 0);
    if (e) return e;
    const uint8_t *base = (const uint8_t *)W;
    GemvArgs a{};
    a.codes = base + desc->off_codes;
    a.signs = desc->fmt == TG_FMT_BITCOS ? (const uint32_t *)(base + desc->off_signs) : nullptr;
    a.rowoff = desc->fmt == TG_FMT_BITCOS ? (const uint32_t *)(base + desc->off_index) : nullptr;
    a.sign_dwords = (uint32_t)(desc->bytes_signs / 4);
    a.n = (int32_t)desc->n;
    a.k = (int32_t)desc->k;
    a.scales = scales;
    a.x = x;
    a.y = y;
    a.acc = acc;
    a.m = m;
    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    switch (desc->fmt) {
        case TG_FMT_BITCOS: err = launch_bitcos(a, acc_out, s); break;
        case TG_FMT_5TRIT: err = launch_t5(a, acc_out, s); break;
        case TG_FMT_2BIT: err = launch_b2(a, acc_out, s); break;
        default: return TG_EFORMAT;
    }
    return err == hipSuccess ? TG_OK : TG_EHIP;
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
