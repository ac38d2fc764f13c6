// Internal declarations shared by the host packers, the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ternary_gemv.h"

namespace tg {

constexpr uint64_t kAlign = 256;      // section alignment inside a packed buffer
constexpr uint64_t kSignPad = 16;     // zero bytes after the sign stream (room for 2-dword windows)

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Arguments every GEMV kernel receives (device pointers into one packed buffer plus the
// caller's scales, activations and outputs).
struct GemvArgs {
    const uint8_t *codes;     // bitmap (BITCOS) or code bytes (5-trit, 2-bit)
    const uint32_t *signs;    // BITCOS sign stream as little-endian dwords
    const uint32_t *rowoff;   // BITCOS per-row sign positions, n + 1 entries
    uint32_t sign_dwords;     // dwords in the sign section (reads are clamped below this)
    int32_t n, k;             // rows, reduction length (k % 128 == 0)
    const uint16_t *scales;   // fp16 [n][k/128]
    const int8_t *x;          // int8 [m][k]
    float *y;                 // float [m][n] (value path)
    int32_t *acc;             // int32 [m][n][k/128] (accumulator path)
    int32_t m;                // activation rows handled by this launch
};

// Host-side checks of a descriptor; `limit` is the buffer length when known (0 = trust bytes_total).
int check_desc(const tg_desc *d, uint64_t limit);

// Kernel launchers (asynchronous; return the HIP status of the launch).
hipError_t launch_bitcos(const GemvArgs &a, bool acc_out, hipStream_t s);
hipError_t launch_t5(const GemvArgs &a, bool acc_out, hipStream_t s);
hipError_t launch_b2(const GemvArgs &a, bool acc_out, hipStream_t s);

}  // namespace tg
