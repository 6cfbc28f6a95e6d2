// Kernel launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ep {

// container codes (the first four equal the ep_dtype values)
enum Container : int { CT_BF16 = 1, CT_F16 = 2, CT_F8E4M3 = 3, CT_I8 = 4, CT_Q16 = 100 };

// Everything a decode kernel needs about one uploaded matrix and one output.
struct DecodeParams {
    const uint32_t* payload;    // tile payload, 4-byte units
    const uint32_t* index;      // [n_tiles + 1] tile offsets into payload
    const float* row_scale;     // [rows] (lossy)
    const uint16_t* row_qmax;   // [rows] (lossy)
    const uint8_t* tables;      // lut [n_tables][2^n] u8, then sym [n_tables][256] u64
    int mode, n_tables, prob_bits, tile_rows;
    int64_t rows, cols, tiles_c, pairs_c, n_pairs;
    float step;
    void* out;                  // [rows][cols] container elements
    float* scale_out;           // [rows] for FP8 / INT8
    int* err;                   // device error flag (bit 0: words, bit 1: final state)
};

// Size in bytes of the device table blob for a stream (lut + sym), a multiple of 16.
inline size_t table_blob_bytes(int n_tables, int prob_bits) {
    return ((size_t)n_tables << prob_bits) + (size_t)n_tables * 256 * 8;
}

hipError_t launch_decode(const DecodeParams& p, int container, hipStream_t stream);

}  // namespace ep
