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

// FP8 GEMM: Y[m][n] = sx[m] * sw[n] * sum_k X[m][k] W[n][k] (+ bias[n]), X and W OCP E4M3 codes,
// fp32 accumulation, BF16 output.
struct GemmF8Args {
    const uint8_t* X;       // [M][ldx] E4M3
    const float* sx;        // [M]
    const uint8_t* W;       // [N][ldw] E4M3
    const float* sw;        // [N]
    const uint16_t* bias;   // [N] bf16 or null
    uint16_t* Y;            // [M][ldy] bf16
    int M, N, K, ldx, ldw, ldy;
};

// Requires K % 16 == 0 and 16-byte aligned rows (ldx, ldw multiples of 16, aligned bases).
hipError_t launch_gemm_f8(const GemmF8Args& g, hipStream_t stream);

// Per-row E4M3 quantization of BF16 rows: amax = max |x| (raised to 2^-100 when smaller and not
// zero), s = amax / 448, q = E4M3(x * (448 / amax)); a zero row gets s = 0 and codes 0.
// Requires K % 8 == 0 and 16-byte aligned rows.
hipError_t launch_quantize_rows_f8(const uint16_t* X, int M, int K, int ldx, uint8_t* Q, int ldq, float* s,
                                   hipStream_t stream);

}  // namespace ep
