// Launch interface of the decode fused into the compressed linear layer's matrix product
// (fused.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kernels.h"

namespace ep {

// Largest number of activation rows the fused kernel takes (one 16-row MFMA tile). Beyond it the
// decode-then-GEMM path is as fast or faster: the partial-sum registers of a second M tile push
// the kernel into register spills (measured at 32 and 64 rows).
constexpr int kFusedMaxRows = 16;
// The same for streams in the row layout (each rANS state on one tile row), whose kernel needs no
// transposition and keeps up to four 16-row M tiles.
constexpr int kFusedMaxRowsRowLayout = 64;

// Whether launch_fused takes this matrix and M (lossy, 16-row tiles, 1 <= M <= kFusedMaxRows, or
// kFusedMaxRowsRowLayout in the row layout, cols % 8 == 0 and 64 x cols BF16 rows addressable
// with 32-bit offsets).
bool fused_fits(const MatDesc& m, int64_t M);

// Bytes of fp32 partial sums the fused kernel writes for M activation rows of matrix m.
size_t fused_partial_bytes(const MatDesc& m, int64_t M);

// Y [M][rows] = X [M][cols] W^T (+ bias) for the activation rows fused_fits allows, of a lossy
// matrix with 16-row tiles: every tile pair is decoded once into registers and becomes the B
// operand of the BF16 MFMA (layout 0: transposed through LDS; row layout: straight from the
// decoder's registers, block step by block step), multiplied by X (bf16 [M][cols], cols % 8 == 0,
// 16-byte aligned); its fp32 partial sums go to `part` (fused_partial_bytes); a second kernel sums
// them per output in column order, adds the bias (bf16 [rows] or null) and rounds to BF16 into y
// (bf16 [M][rows]).
hipError_t launch_fused(const MatDesc& m, const uint16_t* x, int64_t M, float* part, const uint16_t* bias,
                        uint16_t* y, hipStream_t stream);

// Whether launch_fused_many takes these matrices and M: 1 to kMaxGroup matrices that fused_fits
// each, all in the row layout, with one probability precision and one input width.
bool fused_many_fits(const MatDesc* ms, int count, int64_t M);

// launch_fused for several matrices that take the same activations X (bf16 [M][cols]) in one
// decode + MFMA launch: matrix i writes its partial sums to parts[i] (fused_partial_bytes of it)
// and Y_i = X W_i^T (+ bias[i], bf16 or null) to y[i] (bf16 [M][rows_i]), each the same bits as
// launch_fused of that matrix alone.
hipError_t launch_fused_many(const MatDesc* ms, int count, const uint16_t* x, int64_t M, float* const* parts,
                             const uint16_t* const* bias, uint16_t* const* y, hipStream_t stream);

// launch_fused_many in FP8: the E4M3 codes xq [M][cols] and row scales xs [M] of the shared
// activations, each matrix finished with its own row scales (cols % 16 == 0), each y[i] the same
// bits as launch_fused_f8 of that matrix alone.
hipError_t launch_fused_many_f8(const MatDesc* ms, int count, const uint8_t* xq, const float* xs, int64_t M,
                                float* const* parts, const uint16_t* const* bias, uint16_t* const* y,
                                hipStream_t stream);

// FP8 variant: the tile pairs decoded into E4M3 codes (the FP8 container) multiplied by per-row
// E4M3 activation codes xq [M][cols] (scales xs [M]) on v_mfma_f32_16x16x128_f8f6f4 (layout 0) or
// v_mfma_f32_16x16x32_fp8_fp8 (row layout); y = (sum of the partials) x xs[m] x row_scale[n]
// (+ bias), BF16. Requires cols % 16 == 0.
hipError_t launch_fused_f8(const MatDesc& m, const uint8_t* xq, const float* xs, int64_t M, float* part,
                           const uint16_t* bias, uint16_t* y, hipStream_t stream);

}  // namespace ep
