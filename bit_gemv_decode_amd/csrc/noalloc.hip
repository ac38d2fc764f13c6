// Plans whose table lives in the library's own static device memory, for callers that cannot
// allocate device memory (tg_plan_init_noalloc; the plan itself is the grouped launch of several
// GEMVs, each computed as ternary_gemv computes it).
//
// The table is a file-scope device array. In host code its name is only a stand-in for the symbol,
// not a device address: the address of each device's copy is obtained once per device with
// hipGetSymbolAddress (with that device current) and kept per device, and only that address is used
// from then on (it becomes the plan's table pointer, which the kernels receive as an argument).
#include <atomic>
#include <mutex>

#include "tg_internal.h"

namespace tg {
namespace {

static_assert(TG_NOALLOC_TABLE_BYTES % 256 == 0, "whole 256-byte blocks");

__device__ __align__(256) uint8_t scratch[TG_NOALLOC_TABLE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];    // each device's copy of `scratch`, once looked up
std::atomic<uint32_t> scratch_gen[kMaxDevices];   // generation of each device's table contents
std::mutex lookup_mutex;

// Address of the current device's copy of the static table (nullptr if it cannot be obtained).
void *scratch_for(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(lookup_mutex);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return nullptr;
        scratch_addr[dev].store(a, std::memory_order_release);
        p = a;
    }
    return p;
}

}  // namespace

bool static_table_current(const void *table, uint32_t gen) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    const void *p = scratch_addr[dev].load(std::memory_order_acquire);
    return p && p == table && scratch_gen[dev].load(std::memory_order_acquire) == gen;
}

}  // namespace tg

using namespace tg;

extern "C" int tg_plan_init_noalloc(tg_plan *plan, int32_t count, const tg_desc *descs, const void *const *W,
                                    const uint16_t *const *scales, const int8_t *const *x, float *const *y,
                                    int32_t *const *acc, int32_t m) {
    if (!plan || count < 1) return TG_EINVAL;
    if (tg_plan_table_bytes(count) > TG_NOALLOC_TABLE_BYTES) return TG_ENOSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TG_EHIP;
    void *table = scratch_for(dev);
    if (!table) return TG_EHIP;
    // the contents are about to change: earlier plans on this table are invalid from here on
    const uint32_t gen = scratch_gen[dev].fetch_add(1, std::memory_order_acq_rel) + 1;
    const int e = plan_init_into(plan, table, TG_NOALLOC_TABLE_BYTES, count, descs, W, scales, x, y, acc, m);
    if (e != TG_OK) return e;
    plan->table_gen = gen == 0 ? 1 : gen;
    if (gen == 0) scratch_gen[dev].store(1, std::memory_order_release);
    return TG_OK;
}
