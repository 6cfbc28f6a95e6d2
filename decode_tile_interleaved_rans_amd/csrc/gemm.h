// BF16 GEMM launch interface: Y = X W^T (+ bias), row-major, K contiguous in X and W.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ep {

struct GemmArgs {
    const uint16_t* X;      // [M][ldx] bf16
    const uint16_t* W;      // [N][ldw] bf16
    const uint16_t* bias;   // [N] bf16 or null
    uint16_t* Y;            // [M][ldy] bf16
    int M, N, K, ldx, ldw, ldy;
};

// Requires K % 8 == 0 and 16-byte aligned rows (ldx, ldw multiples of 8, aligned bases).
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

}  // namespace ep
