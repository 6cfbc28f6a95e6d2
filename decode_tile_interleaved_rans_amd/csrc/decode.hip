// gfx950 decode kernels of the tile-rANS weight codec.
//
// The method codes lattice coordinates in tiles that decode independently, so that symbol
// decoding and weight reconstruction run fused on the GPU, into BF16, FP16, FP8 or INT8
// containers ("EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
// Bitrates", Abstract). Lossless byte-plane tiles implement the lossless tile-ANS option listed in
// "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Choose a
// compression contract"; exponent-coded BF16 tiles (the same section's DFloat11 config for
// lossless BF16, read after the published DFloat11 split) code only the exponent and join it with
// uncoded sign and mantissa bytes.
//
// Work mapping. A tile is tile_rows x 256 weights coded by 32 interleaved rANS states; lane l of
// a tile owns the 8-column block l of every tile row. One wave64 decodes two horizontally
// adjacent tiles of one tile row: lanes 0-31 the even tile, lanes 32-63 the odd one, so each
// decoded block row is one contiguous 1 KiB store (BF16) per wave and both halves share the
// row's scale. A launch covers up to 32 matrices (lossy and lossless alike); a persistent block
// of 16 waves per CU takes an equal share of the launch's decode cost, stages the decode tables
// of each matrix its share touches in LDS, and walks that matrix's tile pairs.
//
// Word staging. Every half-wave keeps a 1024-word LDS ring of its tile's word stream, filled by
// coalesced 512-byte chunk loads that are issued one chunk ahead, so the serial rANS chain only
// ever waits on LDS. Before each block row the ring is topped up until it holds more than a row
// can consume (9 steps x 64 words), so the steps need no bounds checks; a damaged stream can
// only read stale ring words, and is caught by the end-of-tile checks. Lossless tiles top up once
// per row (once per four elements for 4-byte elements).
//
// Per decoding step every lane looks up its slot in the LDS LUT (one byte read), then reads the
// symbol's 8-byte entry (frequency, cumulative frequency, decoded value) and updates its state;
// lanes whose state fell below 2^16 take the next word of their tile: a wave ballot, shifted to
// the lane's half and popcounted below the lane, gives each refilling lane its word index. Lanes
// that decoded the escape symbol then read their raw value the same way.


#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "decode_core.h"
#include "kernels.h"

namespace ep {
namespace {

// ----------------------------------------------------------------------------- stores
// Decoded coordinates are carried as fp32 values (exact: |q| < 2^17) for the floating-point
// containers and as int32 (the bit pattern kept in the same float slot) for INT8 and the raw
// coordinates, which then need no conversion to float and back.
template <int CT>
constexpr bool int_coords() { return CT == CT_I8 || CT == CT_Q16; }
template <int CT>
__device__ __forceinline__ float coord_of(int32_t q) {
    if constexpr (int_coords<CT>()) return __int_as_float(q);
    else return (float)q;
}
// The value field of a table entry (the doubled coordinate in the high half) as a coordinate.
template <int CT>
__device__ __forceinline__ float coord_of_entry(uint32_t ey) {
    if constexpr (int_coords<CT>()) return __int_as_float((int32_t)ey >> 16);
    else return hi16_to_f32(ey);
}
template <int CT>
struct Conv;
template <>
struct Conv<CT_BF16> {
    using T = uint16_t;
    __device__ static uint32_t f(float q, float alpha, float, uint32_t, uint32_t) { return bf16_rne(q * alpha); }
};
template <>
struct Conv<CT_F16> {
    using T = uint16_t;
    __device__ static uint32_t f(float q, float alpha, float, uint32_t, uint32_t) { return f16_rne(q * alpha); }
};
template <>
struct Conv<CT_F8E4M3> {
    using T = uint8_t;      // converted pairwise in store_block
};
template <>
struct Conv<CT_I8> {
    using T = uint8_t;
    // round-half-away(q / k) = floor((2|q| + k) / 2k), by a multiply with ceil(2^32 / 2k); exact
    // because (2|q| + k) * 2k < 2^32.
    __device__ static uint32_t f(float qf, float, float, uint32_t k, uint32_t magic) {
        const int32_t q = __float_as_int(qf);
        const uint32_t a = (uint32_t)(q < 0 ? -q : q);
        const int32_t v = (int32_t)__umulhi(2u * a + k, magic);
        return (uint32_t)(uint8_t)(int8_t)(q < 0 ? -v : v);
    }
};
template <>
struct Conv<CT_Q16> {
    using T = uint16_t;
    __device__ static uint32_t f(float q, float, float, uint32_t, uint32_t) { return (uint32_t)(uint16_t)__float_as_int(q); }
};

// The 8 container values of one block.
template <int CT>
__device__ __forceinline__ void convert_block(const float* q, float alpha, float h, uint32_t k, uint32_t magic,
                                              uint32_t* v) {
    if constexpr (CT == CT_BF16 || CT == CT_F16) {
        // two values per v_cvt_pk_{bf16,f16}_f32 (round to nearest even) of the rounded fp32 products
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            f32x2 p = {materialize(q[j] * alpha), materialize(q[j + 1] * alpha)};
            uint32_t pk;
            if constexpr (CT == CT_BF16) pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
            else pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
            v[j] = pk & 0xFFFFu;
            v[j + 1] = pk >> 16;
        }
    } else if constexpr (CT == CT_F8E4M3) {
        // two values per v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even) of the fp32 products,
        // clamped to +-448 first (med3), which makes the cast saturating
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const float a = __builtin_amdgcn_fmed3f(q[j] * h, -448.0f, 448.0f);
            const float b = __builtin_amdgcn_fmed3f(q[j + 1] * h, -448.0f, 448.0f);
            const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
            v[j] = pk & 0xFFu;
            v[j + 1] = (pk >> 8) & 0xFFu;
        }
    } else if constexpr (CT == CT_I8) {
        if (k == 1) {
            // the row's largest |q| is at most 127: the INT8 value is the coordinate itself
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (uint32_t)__float_as_int(q[j]) & 0xFFu;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = Conv<CT>::f(q[j], alpha, h, k, magic);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = Conv<CT>::f(q[j], alpha, h, k, magic);
    }
}

// One block of a row shared by the whole wave (layout 0: the row is wave-uniform).
template <int CT>
__device__ __forceinline__ void store_block(const MatDesc& M, uint32_t row, uint32_t col0, const float* q, float alpha,
                                   float h, uint32_t k, uint32_t magic) {
    using T = typename Conv<CT>::T;
    T* out = static_cast<T*>(M.out) + (size_t)row * M.cols;
    uint32_t v[8];
    convert_block<CT>(q, alpha, h, k, magic, v);
    if ((M.cols * (uint32_t)sizeof(T)) % 4 == 0) {
        // one unconditional buffer store per row: the resource spans this row, so dwords past its
        // end are dropped by the bounds check (whole dwords, as the row length is a multiple of 4)
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            out, 0, (int)__builtin_amdgcn_readfirstlane((int)(M.cols * sizeof(T))), 0x00020000);
        const uint32_t off = col0 < M.cols ? col0 * (uint32_t)sizeof(T) : 0x80000000u;
        if constexpr (sizeof(T) == 2) {
            const uint4 d = make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, d), ro, off, 0, 0);
        } else {
            const uint2 d = make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24, v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, d), ro, off, 0, 0);
        }
    } else if (col0 + 8 <= M.cols && (M.cols & 7) == 0) {
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint4*>(out + col0) =
                make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
        } else {
            *reinterpret_cast<uint2*>(out + col0) =
                make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24, v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
        }
    } else if (col0 < M.cols) {
        for (int j = 0; j < 8; ++j)
            if (col0 + j < M.cols) out[col0 + j] = (T)v[j];
    }
}

// One block at a row of the lane's own (layout 1: the rows differ across the wave), through a
// per-lane address; columns past the matrix are dropped.
template <int CT>
__device__ __forceinline__ void store_block_lane(const MatDesc& M, uint32_t row, uint32_t col0, const float* q,
                                                 float alpha, float h, uint32_t k, uint32_t magic) {
    using T = typename Conv<CT>::T;
    uint32_t v[8];
    convert_block<CT>(q, alpha, h, k, magic, v);
    T* out = static_cast<T*>(M.out) + (size_t)row * M.cols;
    if (col0 + 8 <= M.cols && (M.cols & 7) == 0) {
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint4*>(out + col0) =
                make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
        } else {
            *reinterpret_cast<uint2*>(out + col0) =
                make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24, v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
        }
    } else if (col0 < M.cols) {
        for (int j = 0; j < 8; ++j)
            if (col0 + j < M.cols) out[col0 + j] = (T)v[j];
    }
}

// ----------------------------------------------------------------------------- lossy kernel

// Sum over the 64 lanes of a wave with DPP moves (no LDS traffic): quad swaps, half-row and row
// mirrors give every lane its 16-lane row's sum; row broadcasts 15 and 31 then carry rows 0-2
// into row 3, so lane 63 holds the total.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
    return v + __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v = dpp_add<0xB1, 0xF>(v);      // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E, 0xF>(v);      // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141, 0xF>(v);     // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);     // row_mirror
    v = dpp_add<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
    return v;
}

// Stores the blocks of block step rr. Layout 0: tile row rr, block column l of lane l. Layout 1
// (ROWS): tile row l mod tile_rows, block column (32 / tile_rows) rr + l / tile_rows, the lane's
// own row scale.
template <int CT, bool ROWS>
__device__ __forceinline__ void store_row(const MatDesc& M, const Tile& t, const PairRows& P, int rr, const float* q,
                                          float h) {
    if constexpr (ROWS) {
        const bool r16 = M.tile_rows == 16;
        const uint32_t row = P.row0 + ((uint32_t)t.l & (r16 ? 15u : 31u));
        if (!t.valid || row >= M.rows) return;
        const uint32_t blk = r16 ? 2u * (uint32_t)rr + ((uint32_t)t.l >> 4) : (uint32_t)rr;
        const float alpha = h * P.sc_l;
        store_block_lane<CT>(M, row, P.tc * 256 + 8 * blk, q, alpha, h, P.k_l, P.magic_l);
        if constexpr (CT == CT_F8E4M3 || CT == CT_I8) {
            if (P.tc == 0 && rr == 0 && (uint32_t)t.l < M.tile_rows)
                M.scale_out[row] = CT == CT_F8E4M3 ? P.sc_l : alpha * (float)P.k_l;
        }
    } else if constexpr (gemv_rows(CT) > 0) {
        // fused matrix-vector product: the row's BF16 weights bf16(q alpha_r), the values the
        // decode stores (so the products are those of the GEMM path, each exact in fp32), times
        // every activation row, summed over the wave (both tiles of the pair cover the same row);
        // lane 63 stores the pair's partial sum, and the finishing kernel adds a row's partials in
        // pair order, so the result does not depend on the schedule
        constexpr int MT = gemv_rows(CT);
        const uint32_t row = P.row0 + rr;
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, P.sc_l), rr));
        if (row >= M.rows) return;
        const float alpha = h * sc;
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            f32x2 p = {materialize(q[j] * alpha), materialize(q[j + 1] * alpha)};
            const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
            w[j] = __uint_as_float(pk << 16);
            w[j + 1] = __uint_as_float(pk & 0xFFFF0000u);
        }
        float s[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc += P.xv[m][i] * w[i];
            s[m] = wave_sum_to_lane63(acc);
        }
        if ((threadIdx.x & 63) == 63) {
            // partials [pair column][m][row]; lane 63 holds the pair's odd tile, tc = 2 pc + 1
            float* part = static_cast<float*>(M.out) + (size_t)(P.tc >> 1) * M.gemv_m * M.rows + row;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < M.gemv_m) part[(size_t)m * M.rows] = s[m];
        }
    } else {
        const uint32_t row = P.row0 + rr;
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, P.sc_l), rr));
        if (row >= M.rows) return;
        const float alpha = h * sc;
        uint32_t k = 1, magic = 0;
        if constexpr (CT == CT_I8) {
            k = (uint32_t)__builtin_amdgcn_readlane((int)P.k_l, rr);
            magic = (uint32_t)__builtin_amdgcn_readlane((int)P.magic_l, rr);
        }
        const uint32_t col0 = t.valid ? P.tc * 256 + 8 * t.l : 0xFFFFFFF0u;     // no tile: out of range
        store_block<CT>(M, row, col0, q, alpha, h, k, magic);
        if constexpr (CT == CT_F8E4M3 || CT == CT_I8) {
            if (P.tc == 0 && t.l == 0) M.scale_out[row] = CT == CT_F8E4M3 ? sc : alpha * (float)k;
        }
    }
}

// Decode C tile pairs side by side (C independent rANS chains per lane, interleaved by the
// compiler to hide LDS latency).
template <int CT, int N, int C, bool ROWS>
__device__ __forceinline__ void lossy_run(const MatDesc& M, const Tables& T, Tile* t, const uint64_t* pair,
                                          uint64_t pend) {
    const float h = M.step * 0.5f;
    const uint2* coset = reinterpret_cast<const uint2*>(M.tables + ((size_t)M.n_tables << N));   // table 0
    const uint32_t f0 = coset[0].x, f1 = coset[1].x;
    const int lo0 = (int32_t)coset[0].y >> 16;
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    PairRows P[C];
#pragma unroll
    for (int c = 0; c < C; ++c) begin_pair<CT, ROWS>(M, rs, pair[c], pair[c] < pend, t[c], P[c]);
    // A row's values are stored after the next row's ring top-up: the top-up waits for its chunk
    // loads with the vector-memory counter, which also counts stores, so a store issued just
    // before it would be waited for too; issued after it, the store has a whole row to drain.
    float qp[C][8];
    for (int rr = 0; rr < M.tile_rows; ++rr) {
        int b[C];
        uint32_t base[C];
        const uint2* ent_b[C];
        float q[C][8];
#pragma unroll
        for (int c = 0; c < C; ++c) top_up(t[c], rs);
        if (rr > 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) store_row<CT, ROWS>(M, t[c], P[c], rr - 1, qp[c], h);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) b[c] = lo0 + (int)coset_step<N>(t[c], f0, f1);
        refill_all<C>(t);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            // tables 1 + 2j + b for this lane's coset; j selects a compile-time offset
            base[c] = (uint32_t)b[c] << N;
            ent_b[c] = T.ent + b[c] * 256;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (kTopUps == 3 && (j == 2 || j == 5)) {
#pragma unroll
                for (int c = 0; c < C; ++c) top_up(t[c], rs);
            }
            // all chains' step j in one basic block, so the scheduler can interleave the chains;
            // the rare escapes branch once for all chains, and only where either coset's table j
            // can decode the escape symbol (a uniform test)
            uint2 e[C];
            const uint2* ent_j[C];
#pragma unroll
            for (int c = 0; c < C; ++c) ent_j[c] = ent_b[c] + 2 * j * 256;
            rans_steps<N, C>(t, (2 * j) << N, base, ent_j, e);
            refill_all<C>(t);
#pragma unroll
            for (int c = 0; c < C; ++c) q[c][j] = coord_of_entry<CT>(e[c].y);
            if ((M.esc_tables >> (2 * j)) & 3u) {
                bool esc[C];
                uint64_t any = 0;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    esc[c] = (int32_t)e[c].x < 0;
                    any |= __ballot(esc[c]);
                }
                if (any) {
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const uint32_t w = take_words(t[c], esc[c]);
                        // the doubled coordinate is an int16 on every path (table values
                        // wrap the same way when the tables are built)
                        if (esc[c]) q[c][j] = coord_of<CT>((int32_t)(int16_t)(2 * (int32_t)(int16_t)w + b[c]));
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) qp[c][j] = q[c][j];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) store_row<CT, ROWS>(M, t[c], P[c], M.tile_rows - 1, qp[c], h);
#pragma unroll
    for (int c = 0; c < C; ++c) end_tile(t[c]);
}

// Pairs [p0, p1) of one matrix: wave w decodes pairs p0 + w and p0 + w + 16 together, then
// p0 + w + 32 and p0 + w + 48, ...: two independent chains per lane keep the SIMDs busy while
// the other chain waits on LDS.
template <int CT, int N, bool ROWS = false>
__device__ __forceinline__ void lossy_pairs(const MatDesc& M, const Tables& T, Tile* t, uint64_t p0, uint64_t p1) {
    // the wave's index is uniform across its lanes: keep it (and so the pair, tile row and row
    // addresses) in SGPRs
    const uint64_t w0 = (uint64_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    for (uint64_t p = p0 + w0; p < p1; p += kChains * kWaves) {
        uint64_t pr[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) pr[c] = p + (uint64_t)c * kWaves;
        lossy_run<CT, N, kChains, ROWS>(M, T, t, pr, p1);
    }
}

template <int N, bool ROWS>
__device__ __forceinline__ void lossy_dispatch(const MatDesc& M, const Tables& T, Tile* t, uint64_t p0, uint64_t p1) {
    switch (M.container) {
        case CT_BF16: lossy_pairs<CT_BF16, N, ROWS>(M, T, t, p0, p1); break;
        case CT_F16: lossy_pairs<CT_F16, N, ROWS>(M, T, t, p0, p1); break;
        case CT_F8E4M3: lossy_pairs<CT_F8E4M3, N, ROWS>(M, T, t, p0, p1); break;
        case CT_I8: lossy_pairs<CT_I8, N, ROWS>(M, T, t, p0, p1); break;
        default: lossy_pairs<CT_Q16, N, ROWS>(M, T, t, p0, p1); break;
    }
}

// ----------------------------------------------------------------------------- lossless kernel
template <int P>
__device__ __forceinline__ void store_lossless_row(const MatDesc& M, const Tile& t, uint32_t row, uint32_t col0,
                                                   const uint32_t* v) {
    using E = typename std::conditional<P == 1, uint8_t, typename std::conditional<P == 2, uint16_t, uint32_t>::type>::type;
    if (row < M.rows && t.valid && col0 < M.cols) {
        E* out = static_cast<E*>(M.out) + (size_t)row * M.cols;
        if (col0 + 8 <= M.cols && (M.cols & 7) == 0) {
            if constexpr (P == 2) {
                *reinterpret_cast<uint4*>(out + col0) =
                    make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
            } else if constexpr (P == 1) {
                *reinterpret_cast<uint2*>(out + col0) = make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24,
                                                                   v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
            } else {
                *reinterpret_cast<uint4*>(out + col0) = make_uint4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<uint4*>(out + col0 + 4) = make_uint4(v[4], v[5], v[6], v[7]);
            }
        } else {
            for (int j = 0; j < 8; ++j)
                if (col0 + j < M.cols) out[col0 + j] = (E)v[j];
        }
    }
}

// A row's elements are stored after the next row's first ring top-up (as in the lossy kernel):
// the top-up waits for its chunk with the in-order vector-memory counter, which would also wait
// for a store issued just before it.
template <int P, int N>
__device__ __forceinline__ void lossless_pairs(const MatDesc& M, const Tables& T, Tile& t, uint64_t p0, uint64_t p1) {
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    const uint64_t w0 = (uint64_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    for (uint64_t pair = p0 + w0; pair < p1; pair += kWaves) {
        const uint32_t tr = (uint32_t)(pair / M.pairs_c);
        const uint32_t tc = 2 * (uint32_t)(pair % M.pairs_c) + (t.sh ? 1u : 0u);
        t.valid = tc < M.tiles_c;
        begin_tile(M, rs, (uint64_t)tr * M.tiles_c + tc, t);
        const uint32_t row0 = tr * M.tile_rows, col0 = tc * 256 + 8 * t.l;
        uint32_t prev[8];
        for (int rr = 0; rr < M.tile_rows; ++rr) {
            uint32_t v[8];
            // an element is at most P steps x 32 words, and a top-up leaves more than
            // kRingWords - kChunkWords unread: enough for the whole row when P <= 2
            constexpr int kElemsPerTopUp = (kRingWords - kChunkWords) / (32 * P) >= 8 ? 8 : 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (e % kElemsPerTopUp == 0) top_up(t, rs);
                if (e == 0 && rr > 0) store_lossless_row<P>(M, t, row0 + rr - 1, col0, prev);
                uint32_t acc = 0;
#pragma unroll
                for (int pl = 0; pl < P; ++pl) {
                    uint32_t v;
                    const uint32_t s = rans_step<N>(t, pl << N, 0u, T.ent + pl * 256, v);
                    refill(t);
                    acc = acc << 8 | s;
                }
                v[e] = acc;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) prev[e] = v[e];
        }
        store_lossless_row<P>(M, t, row0 + M.tile_rows - 1, col0, prev);
        end_tile(t);
    }
}

__device__ __forceinline__ void lossless_dispatch(const MatDesc& M, const Tables& T, Tile* t, uint64_t p0, uint64_t p1) {
    switch (M.n_tables * 16 + M.prob_bits) {
        case 16 + 10: lossless_pairs<1, 10>(M, T, t[0], p0, p1); break;
        case 16 + 11: lossless_pairs<1, 11>(M, T, t[0], p0, p1); break;
        case 16 + 12: lossless_pairs<1, 12>(M, T, t[0], p0, p1); break;
        case 32 + 10: lossless_pairs<2, 10>(M, T, t[0], p0, p1); break;
        case 32 + 11: lossless_pairs<2, 11>(M, T, t[0], p0, p1); break;
        case 32 + 12: lossless_pairs<2, 12>(M, T, t[0], p0, p1); break;
        case 64 + 10: lossless_pairs<4, 10>(M, T, t[0], p0, p1); break;
        case 64 + 11: lossless_pairs<4, 11>(M, T, t[0], p0, p1); break;
        default: lossless_pairs<4, 12>(M, T, t[0], p0, p1); break;
    }
}

// ----------------------------------------------------------------------------- exponent-coded BF16
// One rANS step per element decodes its exponent byte; the sign and mantissa bytes of the lane's
// 8 elements of a row come from the raw plane [Rp][Cp] with one 8-byte load, issued a row ahead.
// bf16 = (r & 0x80) << 8 | e << 7 | (r & 0x7F) for raw byte r and exponent e.
__device__ __forceinline__ uint32_t join_pair(uint32_t raw_word, uint32_t sel, uint32_t e0, uint32_t e1) {
    const uint32_t r = __builtin_amdgcn_perm(0u, raw_word, sel);   // two raw bytes at bits 0 and 16
    return (r & 0x007F007Fu) | ((r << 8) & 0x80008000u) | (e0 << 7) | (e1 << 23);
}

__device__ __forceinline__ void store_bf16_row(const MatDesc& M, const Tile& t, uint32_t row, uint32_t col0,
                                               const uint4& o) {
    if (row < M.rows && t.valid && col0 < M.cols) {
        uint16_t* out = static_cast<uint16_t*>(M.out) + (size_t)row * M.cols;
        if (col0 + 8 <= M.cols && (M.cols & 7) == 0) {
            *reinterpret_cast<uint4*>(out + col0) = o;
        } else {
            const uint32_t w[4] = {o.x, o.y, o.z, o.w};
            for (int j = 0; j < 8; ++j)
                if (col0 + j < M.cols) out[col0 + j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// Order of the memory operations in a row, so that every wait of the in-order vector-memory
// counter is for operations issued a row earlier: wait for this row's raw bytes (their load was
// the last one issued in the previous row), top up the ring (its chunk load was issued before
// that), store the previous row's values, issue the next row's raw load, decode.
template <int N>
__device__ __forceinline__ void split_pairs(const MatDesc& M, const Tables& T, Tile& t, uint64_t p0, uint64_t p1) {
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    const uint64_t w0 = (uint64_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint64_t stride = (uint64_t)M.tiles_c * 256u;     // raw plane row length Cp
    for (uint64_t pair = p0 + w0; pair < p1; pair += kWaves) {
        const uint32_t tr = (uint32_t)(pair / M.pairs_c);
        const uint32_t tc = 2 * (uint32_t)(pair % M.pairs_c) + (t.sh ? 1u : 0u);
        t.valid = tc < M.tiles_c;
        // a half without a tile reads the bytes of the tile row's first tile (in range, unused)
        const uint8_t* raw = M.raw + (uint64_t)tr * M.tile_rows * stride + (t.valid ? tc * 256u : 0u) + 8u * t.l;
        uint2 next = *reinterpret_cast<const uint2*>(raw);   // before the tile's first chunk loads
        begin_tile(M, rs, (uint64_t)tr * M.tiles_c + tc, t);
        const uint32_t row0 = tr * M.tile_rows, col0 = tc * 256 + 8 * t.l;
        uint4 prev = make_uint4(0u, 0u, 0u, 0u);
        for (int rr = 0; rr < M.tile_rows; ++rr) {
            const uint2 cur = next;
            asm volatile("" ::"v"(cur.x), "v"(cur.y));
            top_up(t, rs);
            if (rr > 0) store_bf16_row(M, t, row0 + rr - 1, col0, prev);
            if (rr + 1 < M.tile_rows) next = *reinterpret_cast<const uint2*>(raw + (uint64_t)(rr + 1) * stride);
            uint32_t e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t v;
                e[k] = rans_step<N>(t, 0u, 0u, T.ent, v);
                refill(t);
            }
            prev = make_uint4(join_pair(cur.x, 0x0C010C00u, e[0], e[1]), join_pair(cur.x, 0x0C030C02u, e[2], e[3]),
                              join_pair(cur.y, 0x0C010C00u, e[4], e[5]), join_pair(cur.y, 0x0C030C02u, e[6], e[7]));
        }
        store_bf16_row(M, t, row0 + M.tile_rows - 1, col0, prev);
        end_tile(t);
    }
}

// ----------------------------------------------------------------------------- grouped kernel
// Persistent blocks over a launch's matrix-major tile pairs, lossy and lossless matrices alike.
// Work is balanced by cost, not by pair count: a pair costs its relative decode time
// (pair_cost), matrix i spans cost units [cost_start[i], cost_start[i + 1]), and block k owns
// the pairs whose first unit falls in [k C, (k + 1) C). A block walks its range one matrix
// segment at a time and restages the decode tables when it crosses into the next matrix.
// GEMV = 0: the general grouped decode; GEMV = CT_GEMV1/2/4: the fused matrix-vector product of
// lossy matrices (a kernel of its own, so that its registers do not weigh on the decode kernel).
// ROWS: lossy matrices in the row layout only (a kernel of its own too: sharing one kernel with the
// layout-0 loop cost that loop 3% on gfx950).
template <int GEMV, bool ROWS = false>
__device__ __forceinline__ void group_body(const GroupArgs& g) {
    extern __shared__ __align__(16) uint8_t smem[];
    // the lookups address the LUTs absolutely: the dynamic LDS must start at address 0
    if ((uint32_t)(size_t)(lds_u8*)smem != 0u) {
        if (threadIdx.x == 0)
            for (int i = 0; i < g.count; ++i) atomicOr(g.m[i].err, kErrLayout);
        return;
    }
    const uint64_t a = (uint64_t)blockIdx.x * g.block_cost;
    const uint64_t b = std::min<uint64_t>(a + g.block_cost, g.cost_start[g.count]);
    for (int mi = 0; mi < g.count; ++mi) {
        const uint64_t cs = g.cost_start[mi], ce = g.cost_start[mi + 1];
        if (ce <= a || cs >= b) continue;
        const MatDesc M = g.m[mi];
        const uint64_t w = M.pair_cost;
        const uint64_t p0 = (std::max(a, cs) - cs + w - 1) / w;
        const uint64_t p1 = (std::min(b, ce) - cs + w - 1) / w;
        if (p0 >= p1) continue;
        const bool lossy = M.mode == 0;
        __syncthreads();                            // every wave is done with the previous tables
        Tables T;
        if constexpr (ROWS) T = stage_lossy_tables_dma(M, smem);   // once per launch, mostly
        else T = stage_tables(M, smem, lossy);
        Tile t[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) init_lane(t[c], smem + lds_table_bytes(M.n_tables, M.prob_bits, lossy), c);
        if constexpr (GEMV > 0) {
            switch (M.prob_bits) {
                case 10: lossy_pairs<GEMV, 10>(M, T, t, p0, p1); break;
                case 11: lossy_pairs<GEMV, 11>(M, T, t, p0, p1); break;
                default: lossy_pairs<GEMV, 12>(M, T, t, p0, p1); break;
            }
        } else if (lossy || ROWS) {
            switch (M.prob_bits) {
                case 10: lossy_dispatch<10, ROWS>(M, T, t, p0, p1); break;
                case 11: lossy_dispatch<11, ROWS>(M, T, t, p0, p1); break;
                default: lossy_dispatch<12, ROWS>(M, T, t, p0, p1); break;
            }
        } else if constexpr (ROWS) {
        } else if (M.mode == 2) {
            switch (M.prob_bits) {
                case 10: split_pairs<10>(M, T, t[0], p0, p1); break;
                case 11: split_pairs<11>(M, T, t[0], p0, p1); break;
                default: split_pairs<12>(M, T, t[0], p0, p1); break;
            }
        } else {
            lossless_dispatch(M, T, t, p0, p1);
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            if (t[c].err) atomicOr(M.err, t[c].err);
    }
}

__global__ __launch_bounds__(64 * kWaves) void decode_group(GroupArgs g) { group_body<0>(g); }

__global__ __launch_bounds__(64 * kWaves) void decode_group_rows(GroupArgs g) { group_body<0, true>(g); }

template <int CT>
__global__ __launch_bounds__(64 * kWaves) void decode_gemv(GroupArgs g) { group_body<CT>(g); }

// Y [M][N] bf16 = the sum, in pair-column order, of the partials [pcs][M][N] (+ bias [N] bf16),
// rounded to nearest even; pcs = 0 (an empty product) gives the bias or zeros.
__global__ __launch_bounds__(256) void gemv_finish(const float* part, int64_t pcs, const uint16_t* bias, uint16_t* y,
                                                   int64_t M, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    float v = 0.0f;
    for (int64_t p = 0; p < pcs; ++p) v += part[p * M * N + i];
    if (bias) v += __uint_as_float((uint32_t)bias[i % N] << 16);
    y[i] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.0f}, bf16x2)) & 0xFFFFu);
}


}  // namespace

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

namespace {

// One launch of `kernel` over the listed matrices, cost-balanced across the CUs.
hipError_t launch_group_with(void (*kernel)(GroupArgs), const MatDesc* const* mats, int count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    GroupArgs g{};
    g.count = count;
    uint64_t total = 0;
    size_t lds = 0;
    for (int i = 0; i < count; ++i) {
        const MatDesc& m = *mats[i];
        g.m[i] = m;
        g.cost_start[i] = total;
        const uint64_t pairs = (uint64_t)((m.rows + m.tile_rows - 1) / m.tile_rows) * m.pairs_c;
        total += pairs * m.pair_cost;
        if (pairs)
            lds = std::max(lds, lds_table_bytes(m.n_tables, m.prob_bits, m.mode == 0) +
                                    (size_t)kWaves * kChains * 2 * kRingBytes);
    }
    g.cost_start[count] = total;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (uint64_t)device_cus();
    g.block_cost = (total + blocks - 1) / blocks;
    const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
    hipError_t e = allow_lds(reinterpret_cast<const void*>(kernel));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3((unsigned)used), dim3(64 * kWaves), lds, stream, g);
    return hipGetLastError();
}

}  // namespace

// Lossy matrices in the row layout go to their own kernel (a second launch when a group mixes
// layouts).
hipError_t launch_group(const MatDesc* mats, int count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    if (count > kMaxGroup) return hipErrorInvalidValue;
    const MatDesc* plain[kMaxGroup];
    const MatDesc* rows[kMaxGroup];
    int np = 0, nr = 0;
    for (int i = 0; i < count; ++i) {
        if (mats[i].mode == 0 && mats[i].layout != 0) rows[nr++] = &mats[i];
        else plain[np++] = &mats[i];
    }
    hipError_t e = launch_group_with(decode_group, plain, np, stream);
    if (e == hipSuccess) e = launch_group_with(decode_group_rows, rows, nr, stream);
    return e;
}

hipError_t launch_gemv(const MatDesc& m, hipStream_t stream) {
    // the matrix-vector kernel reads layout-0 streams (layout 1 goes to the MFMA kernel)
    if (m.mode != 0 || m.layout != 0 || m.gemv_m == 0 || m.gemv_m > gemv_rows(m.container)) return hipErrorInvalidValue;
    GroupArgs g{};
    g.count = 1;
    g.m[0] = m;
    const uint64_t pairs = (uint64_t)((m.rows + m.tile_rows - 1) / m.tile_rows) * m.pairs_c;
    const uint64_t total = pairs * m.pair_cost;
    g.cost_start[0] = 0;
    g.cost_start[1] = total;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (uint64_t)device_cus();
    g.block_cost = (total + blocks - 1) / blocks;
    const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
    const size_t lds = lds_table_bytes(m.n_tables, m.prob_bits, true) + (size_t)kWaves * kChains * 2 * kRingBytes;
    const void* k;
    switch (m.container) {
        case CT_GEMV1: k = reinterpret_cast<const void*>(decode_gemv<CT_GEMV1>); break;
        case CT_GEMV2: k = reinterpret_cast<const void*>(decode_gemv<CT_GEMV2>); break;
        default: k = reinterpret_cast<const void*>(decode_gemv<CT_GEMV4>); break;
    }
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    switch (m.container) {
        case CT_GEMV1: hipLaunchKernelGGL(decode_gemv<CT_GEMV1>, dim3((unsigned)used), dim3(64 * kWaves), lds, stream, g); break;
        case CT_GEMV2: hipLaunchKernelGGL(decode_gemv<CT_GEMV2>, dim3((unsigned)used), dim3(64 * kWaves), lds, stream, g); break;
        default: hipLaunchKernelGGL(decode_gemv<CT_GEMV4>, dim3((unsigned)used), dim3(64 * kWaves), lds, stream, g); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_finish(const float* part, int64_t pcs, const uint16_t* bias, uint16_t* y, int64_t M,
                              int64_t N, hipStream_t stream) {
    if (M * N <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_finish, dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, stream, part, pcs, bias, y,
                       M, N);
    return hipGetLastError();
}

}  // namespace ep
