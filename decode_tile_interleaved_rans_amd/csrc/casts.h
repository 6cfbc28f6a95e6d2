// Device-side number-format casts shared by the gfx950 kernels of the codec.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ep {

// OCP E4M3FN, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7FFFFFFFu;
    uint32_t r;
    if (u >= 0x43E00000u) {                              // >= 448 (448..464 rounds to 448 too)
        r = 0x7Eu;
    } else if (u < 0x3C800000u) {                        // below 2^-6: subnormal grid of 2^-9
        r = (uint32_t)__builtin_rintf(__uint_as_float(u) * 512.0f);   // 8 -> 0x08, smallest normal
    } else {
        u += 0x7FFFFu + ((u >> 20) & 1u);                // round the mantissa to 3 bits
        uint32_t e = (u >> 23) - 127u + 7u;
        r = (e << 3) | ((u >> 20) & 7u);
        if (r > 0x7Eu) r = 0x7Eu;
    }
    return r | sign;
}

}  // namespace ep
