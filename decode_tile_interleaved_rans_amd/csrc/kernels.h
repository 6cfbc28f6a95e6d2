// Kernel launch interface between the C ABI and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ep {

// container codes (the first four equal the ep_dtype values)
enum Container : int {
    CT_BF16 = 1, CT_F16 = 2, CT_F8E4M3 = 3, CT_I8 = 4, CT_Q16 = 100,
    // fused matrix-vector products W x[m] for m < 1, 2 or 4 activation rows (see launch_gemv)
    CT_GEMV1 = 101, CT_GEMV2 = 102, CT_GEMV4 = 104
};

constexpr int kMaxGroup = 32;        // matrices per grouped launch (kernel-argument space)

// One matrix of a grouped decode launch: the uploaded stream and its output.
struct MatDesc {
    const uint32_t* payload;    // tile payload, 4-byte units
    const uint32_t* index;      // [n_tiles + 1] tile offsets into payload
    const float* row_scale;     // [rows] (lossy)
    const uint16_t* row_qmax;   // [rows] (lossy)
    const uint8_t* raw;         // [Rp][Cp] sign/mantissa bytes (exponent-coded lossless BF16)
    const uint8_t* tables;      // decode tables (see table_blob_bytes)
    void* out;                  // [rows][cols] container elements
    union {
        float* scale_out;       // [rows] for FP8 / INT8, else unused
        const uint16_t* gemv_x; // fused matrix-vector product: X [gemv_m][cols] bf16 (out: fp32 partials)
    };
    int* err;                   // device error flag (bit 0: word count, bit 1: final state)
    uint32_t rows, cols, tiles_c, pairs_c;
    uint32_t payload_bytes;     // size of the tile payload (buffer-load bounds)
    float step;
    uint8_t prob_bits, tile_rows, container, n_tables;
    uint8_t mode;               // 0 lossy E8 coordinates, 1 lossless byte planes, 2 exponent-coded BF16
    uint8_t gemv_m;             // activation rows of a fused matrix-vector product
    uint16_t esc_tables;        // lossy: bit 2j + b set when coordinate table 1 + 2j + b can decode
                                // the escape symbol (its frequency is not zero)
    uint32_t pair_cost;         // relative decode time of one tile pair (load balancing)
    uint8_t layout;             // lossy tile layout: 0 lane = block column, 1 lane = tile row (block_of)
};

// Relative decode time of one tile pair, per tile row: a lossy row is 9 steps (coset + 8
// coordinates) at 9 units each; a lossless row is one step per byte plane per element (8
// elements) at 7.5 units, as measured on gfx950 (a lossless BF16 pair takes 1.47 times a lossy
// pair); an exponent-coded BF16 row (8 steps plus joining the raw bytes) takes 0.89 of a lossy
// row.
inline uint32_t pair_cost_of(int mode, int tile_rows, int n_tables) {
    return (uint32_t)tile_rows * (mode == 0 ? 81u : mode == 2 ? 72u : 60u * (uint32_t)n_tables);
}

struct GroupArgs {
    int32_t count;              // matrices in this launch (<= kMaxGroup)
    uint64_t block_cost;        // cost units per block (the last block may get fewer)
    uint64_t cost_start[kMaxGroup + 1];   // matrix-major prefix sums of pairs x pair_cost
    MatDesc m[kMaxGroup];
};

// Decode tables of one stream, in device memory:
//   lut [n_tables][2^n] u8      slot -> symbol
//   ent [n_tables][256] 2 x u32 {f | esc << 31, (c + base) | v << 16}: frequency f (bit 31 set
//                               for the escape symbol of a lossy coordinate table), cumulative
//                               frequency c, and the decoded value v (int16): the doubled lattice
//                               coordinate 2 (lo + s) + b of a lossy coordinate table, lo + s of
//                               the coset table, the byte s of a lossless plane.
// In LDS a lossy stream keeps only its coordinate tables 1..16 (the two-symbol coset table is
// decoded arithmetically from its frequencies), LUTs first, so coordinate table 1 + 2j + b has
// its LUT at LDS address (2j + b) << n. base is b << n for that table and 0 for the others, so
// that slot - c = address - (c + base) for a lookup address (slot | b << n) + (2j << n).
__host__ __device__ inline size_t table_blob_bytes(int n_tables, int prob_bits) {
    return ((size_t)n_tables << prob_bits) + (size_t)n_tables * 256 * 8;
}
__host__ __device__ inline size_t lds_table_bytes(int n_tables, int prob_bits, bool lossy) {
    return table_blob_bytes(lossy ? n_tables - 1 : n_tables, prob_bits);
}

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// Launch one grouped decode of up to kMaxGroup matrices (lossy and lossless may be mixed).
hipError_t launch_group(const MatDesc* mats, int count, hipStream_t stream);

// Fused decode and matrix-vector product of one lossy layout-0 matrix W [rows][cols] with
// gemv_m <= 4 BF16 activation rows: every wave multiplies the BF16 weights it has just decoded
// (bf16(q alpha_r), never stored) by the activations and writes each row's sums over its tile pair
// to the fp32 partials m.out [pairs_c][gemv_m][rows] (every entry of a row < rows written once).
// m.container must be CT_GEMV1, CT_GEMV2 or CT_GEMV4 (at least gemv_m) and cols a multiple of 8.
hipError_t launch_gemv(const MatDesc& m, hipStream_t stream);

// Y [M][N] bf16 = sum over p < pcs, in order, of part [p][M][N] (+ bias [N] bf16), rounded to
// nearest even; pcs = 0 gives the bias (or zeros) and reads no partials.
hipError_t launch_gemv_finish(const float* part, int64_t pcs, const uint16_t* bias, uint16_t* y, int64_t M, int64_t N,
                              hipStream_t stream);

static_assert(sizeof(GroupArgs) <= 4096, "kernel argument space");

}  // namespace ep
