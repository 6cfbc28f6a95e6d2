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
    int splits = 1;         // K splits (gemm_splits); above 1 the scratch below holds the partials
    float* part = nullptr;  // fp32 [splits][M][N] partial tiles
    size_t part_bytes = 0;  // its size
    int kc = 0;             // K columns per split (set by the launcher)
};

// Requires K % 8 == 0 and 16-byte aligned rows (ldx, ldw multiples of 8, aligned bases). With
// splits > 1 every 256 x 256 output tile is computed by `splits` blocks over consecutive K ranges
// of split_columns(K, splits) columns, whose fp32 partial tiles are then added in split order
// (deterministic; hipErrorInvalidValue when the scratch is missing or short).
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

// K splits for an M x N x K product: 1 for M <= 64 or when the 256 x 256 tiles fill the CUs, else
// as many as fill the CUs, at most 8, each at least 256 columns. The result of an output element
// depends only on (K, splits), so slices of N computed with the layer's count give the same bits.
int gemm_splits(int M, int N, int K);
int split_columns(int K, int splits);

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

// The product of launch_gemm (splits ignored) through hipBLASLt with up to ws_bytes of device
// workspace at `workspace`: hipErrorNotSupported when the library offers no algorithm for the shape
// (the caller then runs launch_gemm). Plans are cached per device and shape; calls from several threads are
// serialized while they are queued. (gemm_lt.cpp)
hipError_t lt_gemm(const GemmArgs& g, void* workspace, size_t ws_bytes, hipStream_t stream);
// The FP8 product of launch_gemm_f8 through hipBLASLt (E4M3 operands, the row scales as outer-vector
// scales), same contract.
hipError_t lt_gemm_f8(const GemmF8Args& g, void* workspace, size_t ws_bytes, hipStream_t stream);

// Per-row E4M3 quantization of BF16 rows: amax = max |x| (raised to 2^-100 when smaller and not
// zero), s = amax / 448, q = E4M3(x * (448 / amax)); a zero row gets s = 0 and codes 0.
// Requires K % 8 == 0 and 16-byte aligned rows.
hipError_t launch_quantize_rows_f8(const uint16_t* X, int M, int K, int ldx, uint8_t* Q, int ldq, float* s,
                                   hipStream_t stream);

}  // namespace ep
