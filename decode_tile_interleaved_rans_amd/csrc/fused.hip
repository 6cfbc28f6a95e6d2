// gfx950 kernel of the decode fused into the compressed linear layer's matrix product.
//
// The method decodes its tiles on the GPU fused with the numerical reconstruction of the weights
// ("EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates",
// Abstract), and its compressed linear layer consumes the compressed weight in the forward pass
// ("EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Replace one
// linear layer before a whole model"). Here the reconstructed weights of a tile pair go straight
// into the B operand of the BF16 MFMA through LDS and are never written to memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "decode_core.h"
#include "fused.h"
#include "kernels.h"

namespace ep {
namespace {

// ----------------------------------------------------------------------------- fused decode + MFMA
// Decoding fused into the layer's matrix product for up to 16 activation rows: every weight is
// decoded once, straight into the B operand of v_mfma_f32_16x16x32_bf16, and never written to
// memory. A wave decodes one tile pair (16 weight rows x 512 columns) as the decode kernel does,
// keeping each decoded row as 8 packed BF16 values per lane (lane l: columns 8l .. 8l + 7 of the
// pair; 16 rows = 64 registers). The pair is then transposed through the wave's 4 KiB LDS buffer in
// four rounds: MFMA lane l (q = l / 16, n = l % 16) needs, at K step s, the 8 weights of row n in
// the pair's 8-column block 16 q + s, which the decoding lane 16 q + s holds; round u moves the
// blocks of the K steps 4u .. 4u + 3. Entry (g, r) (g = 4 q + s % 4, r = weight row) sits at slot
// 16 r + (g ^ r): the 16 lanes of a write instruction (fixed r) and of a read instruction (fixed g)
// both cover 16 distinct 16-byte bank groups. Lane l supplies the activations X[m][k] of the same
// block (16 q + s) for m = 16 mt + n, so equal k meet in the MFMA, and receives the pair's partial
// sums Y[16 mt + 4 q + i][16 tr + n], i < 4, written per pair (fp32) and summed over the tile row's
// pairs by fused_finish in column order, so the result does not depend on scheduling.
constexpr int kFusedBuf = 4096;            // LDS transposition buffer per wave

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 p = {materialize(a), materialize(b)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

template <int N, int MT>
__device__ __forceinline__ void fused_pair(const MatDesc& M, const Tables& T, Tile& t, uint64_t pair, bool live,
                                           uint8_t* tbuf, __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx) {
    const float h = M.step * 0.5f;
    const uint2* coset = reinterpret_cast<const uint2*>(M.tables + ((size_t)M.n_tables << N));   // table 0
    const uint32_t f0 = coset[0].x, f1 = coset[1].x;
    const int lo0 = (int32_t)coset[0].y >> 16;
    PairRows P;
    begin_pair<CT_BF16>(M, rs, pair, live, t, P);
    uint32_t rowv[16][4];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        top_up(t, rs);
        const int b = lo0 + (int)coset_step<N>(t, f0, f1);
        refill(t);
        const uint32_t base = (uint32_t)b << N;
        const uint2* ent_b = T.ent + b * 256;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint2 e;
            const uint2* ent_j = ent_b + 2 * j * 256;
            rans_steps<N, 1>(&t, (2 * j) << N, &base, &ent_j, &e);
            refill_all<1>(&t);
            q[j] = hi16_to_f32(e.y);
            if ((M.esc_tables >> (2 * j)) & 3u) {
                const bool esc = (int32_t)e.x < 0;
                if (__ballot(esc)) {
                    const uint32_t w = take_words(t, esc);
                    if (esc) q[j] = (float)(int32_t)(int16_t)(2 * (int32_t)(int16_t)w + b);
                }
            }
        }
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, P.sc_l), rr));
        const float alpha = h * sc;                 // rows past the matrix have scale 0
        const uint32_t keep = t.valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) rowv[rr][i] = pack_bf16(q[2 * i] * alpha, q[2 * i + 1] * alpha) & keep;
        __builtin_amdgcn_sched_barrier(0);          // rows stay in order: one row's values live at a time
    }
    end_tile(t);

    const int lane = threadIdx.x & 63, qg = lane >> 4, n = lane & 15;
    const uint32_t tr = (uint32_t)(pair / M.pairs_c), pc = (uint32_t)(pair % M.pairs_c);
    const uint32_t K = M.cols;
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    lds_u32* buf = (lds_u32*)tbuf;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        __builtin_amdgcn_sched_barrier(0);          // one round's activation loads in flight at a time
        if ((n >> 2) == u) {                        // the lanes holding this round's blocks
            const int g = 4 * qg + (n & 3);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                lds_u32* d = buf + 4 * (16 * r + (g ^ r));
                d[0] = rowv[r][0];
                d[1] = rowv[r][1];
                d[2] = rowv[r][2];
                d[3] = rowv[r][3];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = 4 * qg + j;
            const lds_u32* sbuf = buf + 4 * (16 * n + (g ^ n));
            const uint4 bw = make_uint4(sbuf[0], sbuf[1], sbuf[2], sbuf[3]);
            const uint32_t kc = pc * 512u + 8u * (uint32_t)(16 * qg + 4 * u + j);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // columns past K read as zero (K % 8 == 0: a block is wholly inside or outside)
                const uint32_t off = ((uint32_t)(16 * mt + n) * K + kc) * 2u | ((uint32_t)((int32_t)(K - 1u - kc) >> 31) & 0x80000000u);
                const uint4 ax = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax),
                                                                  __builtin_bit_cast(bf16x8_t, bw), acc[mt], 0, 0, 0);
            }
        }
    }
    // partials [pair][mt][q][n][i] (fp32): 1 KiB per M tile, one 16-byte store per lane
    if (live) {
        float* part = static_cast<float*>(M.out) + pair * (uint64_t)(MT * 256);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<f32x4_t*>(part + ((mt * 4 + qg) * 16 + n) * 4) = acc[mt];
    }
    (void)tr;
}

template <int N, int MT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_mfma(GroupArgs g) {
    extern __shared__ __align__(16) uint8_t smem[];
    const MatDesc& M = g.m[0];
    if ((uint32_t)(size_t)(lds_u8*)smem != 0u) {
        if (threadIdx.x == 0) atomicOr(M.err, kErrLayout);
        return;
    }
    const uint64_t a = (uint64_t)blockIdx.x * g.block_cost;
    const uint64_t b = std::min<uint64_t>(a + g.block_cost, g.cost_start[1]);
    const uint64_t w = M.pair_cost;
    const uint64_t p0 = (a + w - 1) / w, p1 = (b + w - 1) / w;
    if (p0 >= p1) return;
    const Tables T = stage_lossy_tables_dma(M, smem);
    const size_t tb = lds_table_bytes(M.n_tables, M.prob_bits, true);
    Tile t;
    init_lane(t, smem + tb, 0);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    uint8_t* tbuf = smem + tb + (size_t)WAVES * 2 * kRingBytes + (size_t)wave * kFusedBuf;
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(M.gemv_x), 0, (int)((size_t)M.gemv_m * M.cols * 2), 0x00020000);
    for (uint64_t p = p0 + (uint64_t)wave; p < p1; p += WAVES) fused_pair<N, MT>(M, T, t, p, true, tbuf, rs, rx);
    if (t.err) atomicOr(M.err, t.err);
}

// FP8 variant: each decoded row becomes 8 E4M3 codes per lane (fp32(q h) clamped to +-448 and
// rounded to nearest even, the FP8 container of the decode kernel; the row scale s_r is applied
// in fused_finish), 16 rows = 32 registers. The activations arrive as per-row E4M3 codes (the
// quantizer of the FP8 forward). v_mfma_f32_16x16x128_f8f6f4: lane l (q = l / 16, n = l % 16)
// supplies, at K step s (128 columns), the 32 codes of the pair's 8-column blocks 16 q + 4 s + j,
// j < 4, for weight row n (B) and activation row 16 mt + n (A), in the same order. The pair's
// 8 KiB of codes cross the wave's 4 KiB buffer in two rounds (K steps 2u, 2u + 1): entry (g, r)
// (g = 8 q + block % 8, r = weight row) sits at 8-byte slot 32 r + (g ^ 4 (r % 8)), which keeps a
// reader's four blocks contiguous.
template <int N, int MT>
__device__ __forceinline__ void fused_pair_f8(const MatDesc& M, const Tables& T, Tile& t, uint64_t pair, uint8_t* tbuf,
                                              __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx) {
    const float h = M.step * 0.5f;
    const uint2* coset = reinterpret_cast<const uint2*>(M.tables + ((size_t)M.n_tables << N));   // table 0
    const uint32_t f0 = coset[0].x, f1 = coset[1].x;
    const int lo0 = (int32_t)coset[0].y >> 16;
    PairRows P;
    begin_pair<CT_F8E4M3>(M, rs, pair, true, t, P);
    uint32_t rowv[16][2];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        top_up(t, rs);
        const int b = lo0 + (int)coset_step<N>(t, f0, f1);
        refill(t);
        const uint32_t base = (uint32_t)b << N;
        const uint2* ent_b = T.ent + b * 256;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint2 e;
            const uint2* ent_j = ent_b + 2 * j * 256;
            rans_steps<N, 1>(&t, (2 * j) << N, &base, &ent_j, &e);
            refill_all<1>(&t);
            q[j] = hi16_to_f32(e.y);
            if ((M.esc_tables >> (2 * j)) & 3u) {
                const bool esc = (int32_t)e.x < 0;
                if (__ballot(esc)) {
                    const uint32_t w = take_words(t, esc);
                    if (esc) q[j] = (float)(int32_t)(int16_t)(2 * (int32_t)(int16_t)w + b);
                }
            }
        }
        const uint32_t keep = t.valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float a0 = __builtin_amdgcn_fmed3f(q[4 * i] * h, -448.0f, 448.0f);
            const float a1 = __builtin_amdgcn_fmed3f(q[4 * i + 1] * h, -448.0f, 448.0f);
            const float a2 = __builtin_amdgcn_fmed3f(q[4 * i + 2] * h, -448.0f, 448.0f);
            const float a3 = __builtin_amdgcn_fmed3f(q[4 * i + 3] * h, -448.0f, 448.0f);
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
            rowv[rr][i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true) & keep;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    end_tile(t);

    const int lane = threadIdx.x & 63, qg = lane >> 4, n = lane & 15;
    const uint32_t pc = (uint32_t)(pair % M.pairs_c);
    const uint32_t K = M.cols;
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    lds_u32* buf = (lds_u32*)tbuf;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        if ((n >> 3) == u) {                        // the lanes holding this round's blocks
            const int g = 8 * qg + (n & 7);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                lds_u32* d = buf + 2 * (32 * r + (g ^ (4 * (r & 7))));
                d[0] = rowv[r][0];
                d[1] = rowv[r][1];
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int s = 2 * u + hh;
            const lds_u32* sb = buf + 2 * (32 * n + ((8 * qg + 4 * hh) ^ (4 * (n & 7))));
            typedef int i32x8_t __attribute__((ext_vector_type(8)));
            const i32x8_t b8 = {(int)sb[0], (int)sb[1], (int)sb[2], (int)sb[3], (int)sb[4], (int)sb[5], (int)sb[6], (int)sb[7]};
            const uint32_t kc = pc * 512u + 8u * (uint32_t)(16 * qg + 4 * s);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // 16-code halves past K read as zero (K % 16 == 0)
                const uint32_t row = (uint32_t)(16 * mt + n) * K;
                const uint32_t o0 = (row + kc) | ((uint32_t)((int32_t)(K - 1u - kc) >> 31) & 0x80000000u);
                const uint32_t o1 = (row + kc + 16u) | ((uint32_t)((int32_t)(K - 17u - kc) >> 31) & 0x80000000u);
                const uint4 x0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, o0, 0, 0));
                const uint4 x1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, o1, 0, 0));
                const i32x8_t a8 = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[mt], 0, 0, 0, 0, 0, 0);
            }
        }
    }
    float* part = static_cast<float*>(M.out) + pair * (uint64_t)(MT * 256);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4_t*>(part + ((mt * 4 + qg) * 16 + n) * 4) = acc[mt];
}

template <int N, int MT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void decode_mfma_f8(GroupArgs g) {
    extern __shared__ __align__(16) uint8_t smem[];
    const MatDesc& M = g.m[0];
    if ((uint32_t)(size_t)(lds_u8*)smem != 0u) {
        if (threadIdx.x == 0) atomicOr(M.err, kErrLayout);
        return;
    }
    const uint64_t a = (uint64_t)blockIdx.x * g.block_cost;
    const uint64_t b = std::min<uint64_t>(a + g.block_cost, g.cost_start[1]);
    const uint64_t w = M.pair_cost;
    const uint64_t p0 = (a + w - 1) / w, p1 = (b + w - 1) / w;
    if (p0 >= p1) return;
    const Tables T = stage_lossy_tables_dma(M, smem);
    const size_t tb = lds_table_bytes(M.n_tables, M.prob_bits, true);
    Tile t;
    init_lane(t, smem + tb, 0);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    uint8_t* tbuf = smem + tb + (size_t)WAVES * 2 * kRingBytes + (size_t)wave * kFusedBuf;
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(M.gemv_x), 0, (int)((size_t)M.gemv_m * M.cols), 0x00020000);
    for (uint64_t p = p0 + (uint64_t)wave; p < p1; p += WAVES) fused_pair_f8<N, MT>(M, T, t, p, tbuf, rs, rx);
    if (t.err) atomicOr(M.err, t.err);
}

// ----------------------------------------------------------------------------- row layout
// Streams in the row layout (every rANS state of a tile stays on one tile row: lane l codes row
// l mod 16 at block column 2 s + l / 16 in block step s) need no transposition at all: at block
// step s of a tile pair, lane L holds the 8 weights of row n = L mod 16 in the 8 columns
// c0(L) + 16 s, c0(L) = 512 pc + 256 (L / 32) + 8 ((L / 16) mod 2) (tile L / 32 of pair pc), i.e.
// exactly its part of the B operand of a 16 x 16 x 32 MFMA whose K group L / 16 is those 8
// columns. The lane converts them in registers (BF16 of q alpha_r with its own row's alpha_r, or
// the E4M3 code of q h) and the MFMA consumes them at once, with the activations of the same 8
// columns of row 16 mt + n as the A operand, loaded before the step's decode so that their latency
// hides behind it. LDS holds only the decoder's tables and word rings, so the kernel runs 16 waves
// per CU as the decode kernel does. The accumulators have the layout of the transposing kernel's,
// so the partials and the finishing sums are the same. (Loading the activations of 2 or 4 steps
// at once, so that whole 128-byte lines are requested together, measured no faster.)
typedef long i64_t;

template <int N, int MT, bool F8>
__device__ __forceinline__ void rows_pair(const MatDesc& M, const Tables& T, Tile& t, uint64_t pair,
                                          __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx) {
    const float h = M.step * 0.5f;
    const uint2* coset = reinterpret_cast<const uint2*>(M.tables + ((size_t)M.n_tables << N));   // table 0
    const uint32_t f0 = coset[0].x, f1 = coset[1].x;
    const int lo0 = (int32_t)coset[0].y >> 16;
    PairRows P;
    begin_pair<F8 ? CT_F8E4M3 : CT_BF16, true>(M, rs, pair, true, t, P);
    const float alpha = h * P.sc_l;                 // the lane's row (scale 0 past the matrix)
    const int lane = threadIdx.x & 63, qg = lane >> 4, n = lane & 15;
    const uint32_t K = M.cols;
    const uint32_t c0 = (uint32_t)(pair % M.pairs_c) * 512u + (uint32_t)(qg >> 1) * 256u + 8u * (uint32_t)(qg & 1);
    const uint32_t keep = t.valid ? 0xFFFFFFFFu : 0u;
    constexpr uint32_t kEs = F8 ? 1u : 2u;          // activation bytes per element
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < 16; ++s) {
        const uint32_t kc = c0 + 16u * (uint32_t)s;
        // columns past K read as zero (K % 8 == 0: a block is wholly inside or outside), and so do
        // activation rows past M (past the end of the resource)
        const uint32_t oob = (uint32_t)((int32_t)(K - 1u - kc) >> 31) & 0x80000000u;
        uint4 ax[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint32_t off = (((uint32_t)(16 * mt + n) * K + kc) * kEs) | oob;
            if constexpr (F8) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0));
                ax[mt] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                ax[mt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            }
        }
        top_up(t, rs);
        const int b = lo0 + (int)coset_step<N>(t, f0, f1);
        refill(t);
        const uint32_t base = (uint32_t)b << N;
        const uint2* ent_b = T.ent + b * 256;
        float q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint2 e;
            const uint2* ent_j = ent_b + 2 * j * 256;
            rans_steps<N, 1>(&t, (2 * j) << N, &base, &ent_j, &e);
            refill_all<1>(&t);
            q[j] = hi16_to_f32(e.y);
            if ((M.esc_tables >> (2 * j)) & 3u) {
                const bool esc = (int32_t)e.x < 0;
                if (__ballot(esc)) {
                    const uint32_t w = take_words(t, esc);
                    if (esc) q[j] = (float)(int32_t)(int16_t)(2 * (int32_t)(int16_t)w + b);
                }
            }
        }
        if constexpr (F8) {
            uint32_t bw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float a0 = __builtin_amdgcn_fmed3f(q[4 * i] * h, -448.0f, 448.0f);
                const float a1 = __builtin_amdgcn_fmed3f(q[4 * i + 1] * h, -448.0f, 448.0f);
                const float a2 = __builtin_amdgcn_fmed3f(q[4 * i + 2] * h, -448.0f, 448.0f);
                const float a3 = __builtin_amdgcn_fmed3f(q[4 * i + 3] * h, -448.0f, 448.0f);
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
                bw[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true) & keep;
            }
            const i64_t bop = __builtin_bit_cast(i64_t, make_uint2(bw[0], bw[1]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                    __builtin_bit_cast(i64_t, make_uint2(ax[mt].x, ax[mt].y)), bop, acc[mt], 0, 0, 0);
        } else {
            uint4 bw;
            bw.x = pack_bf16(q[0] * alpha, q[1] * alpha) & keep;
            bw.y = pack_bf16(q[2] * alpha, q[3] * alpha) & keep;
            bw.z = pack_bf16(q[4] * alpha, q[5] * alpha) & keep;
            bw.w = pack_bf16(q[6] * alpha, q[7] * alpha) & keep;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[mt]),
                                                                  __builtin_bit_cast(bf16x8_t, bw), acc[mt], 0, 0, 0);
        }
    }
    end_tile(t);
    // partials [pair][mt][q][n][i] (fp32): 1 KiB per M tile, one 16-byte store per lane
    float* part = static_cast<float*>(M.out) + pair * (uint64_t)(MT * 256);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4_t*>(part + ((mt * 4 + qg) * 16 + n) * 4) = acc[mt];
}

template <int N, int MT, bool F8>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_rows(GroupArgs g) {
    extern __shared__ __align__(16) uint8_t smem[];
    const MatDesc& M = g.m[0];
    if ((uint32_t)(size_t)(lds_u8*)smem != 0u) {
        if (threadIdx.x == 0) atomicOr(M.err, kErrLayout);
        return;
    }
    const uint64_t a = (uint64_t)blockIdx.x * g.block_cost;
    const uint64_t b = std::min<uint64_t>(a + g.block_cost, g.cost_start[1]);
    const uint64_t w = M.pair_cost;
    const uint64_t p0 = (a + w - 1) / w, p1 = (b + w - 1) / w;
    if (p0 >= p1) return;
    const Tables T = stage_lossy_tables_dma(M, smem);
    Tile t;
    init_lane(t, smem + lds_table_bytes(M.n_tables, M.prob_bits, true), 0);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(M.gemv_x), 0, (int)((size_t)M.gemv_m * M.cols * (F8 ? 1 : 2)), 0x00020000);
    // pairs in column-major order: the 16 waves of a block take the same 512 columns of 16
    // consecutive tile rows, so their activation loads are the same lines at about the same time
    // and the L1 serves them once (in row-major order each wave had its own columns, and with four
    // M tiles their lines no longer fit the L1)
    const uint32_t tiles_r = (M.rows + 15u) / 16u;
    for (uint64_t p = p0 + (uint64_t)wave; p < p1; p += kWaves) {
        const uint32_t pc = (uint32_t)p / tiles_r, tr = (uint32_t)p % tiles_r;
        rows_pair<N, MT, F8>(M, T, t, (uint64_t)tr * M.pairs_c + pc, rs, rx);
    }
    if (t.err) atomicOr(M.err, t.err);
}

// 0 + p[0] + p[1] + ... + p[n - 1] (stride MT x 256) in that order, with eight loads in flight at
// a time (a loop of dependent additions would wait for each load in turn).
template <int MT>
__device__ __forceinline__ float sum_partials(const float* p, int n) {
    float v = 0.0f;
    for (int pc0 = 0; pc0 < n; pc0 += 8) {
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = pc0 + j < n ? p[(uint64_t)(pc0 + j) * (MT * 256)] : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (pc0 + j < n) v += t[j];
    }
    return v;
}

// Y [M][N] bf16 = (sum over the tile row's pairs of the partials) x s_x[m] x s_w[n] (+ bias).
template <int MT>
__global__ __launch_bounds__(256) void fused_finish_f8(const float* part, const float* sx, const float* sw,
                                                        const uint16_t* bias, uint16_t* y, int Mrows, int Nrows,
                                                        int pairs_c) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Mrows * Nrows) return;
    const int m = (int)(e / Nrows), col = (int)(e % Nrows);
    const int tr = col >> 4, n = col & 15;
    const int mt = m >> 4, qg = (m >> 2) & 3, i = m & 3;
    const float* p = part + (uint64_t)tr * pairs_c * (MT * 256) + ((mt * 4 + qg) * 16 + n) * 4 + i;
    float v = sum_partials<MT>(p, pairs_c);
    v = v * sw[col] * sx[m];
    if (bias) v += __uint_as_float((uint32_t)bias[col] << 16);
    y[e] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.0f}, bf16x2)) & 0xFFFFu);
}

// Y [M][N] bf16 = sum over the tile row's pairs of the partials (+ bias), in pair order.
template <int MT>
__global__ __launch_bounds__(256) void fused_finish(const float* part, const uint16_t* bias, uint16_t* y, int Mrows,
                                                     int Nrows, int pairs_c) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)Mrows * Nrows) return;
    const int m = (int)(e / Nrows), col = (int)(e % Nrows);
    const int tr = col >> 4, n = col & 15;
    const int mt = m >> 4, qg = (m >> 2) & 3, i = m & 3;
    const float* p = part + (uint64_t)tr * pairs_c * (MT * 256) + ((mt * 4 + qg) * 16 + n) * 4 + i;
    float v = sum_partials<MT>(p, pairs_c);
    if (bias) v += __uint_as_float((uint32_t)bias[col] << 16);
    y[e] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.0f}, bf16x2)) & 0xFFFFu);
}


template <int N, int MT>
hipError_t launch_mfma_n(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    constexpr int W = N == 12 ? 8 : 12;
    const MatDesc& m = g.m[0];
    const size_t lds = lds_table_bytes(m.n_tables, m.prob_bits, true) + (size_t)W * 2 * kRingBytes + (size_t)W * kFusedBuf;
    const void* k = reinterpret_cast<const void*>(decode_mfma<N, MT, W>);
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_mfma<N, MT, W>), dim3((unsigned)blocks), dim3(64 * W), lds, stream, g);
    return hipGetLastError();
}

template <int N, int MT>
hipError_t launch_mfma_f8_n(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    constexpr int W = N == 12 ? 8 : 12;
    const MatDesc& m = g.m[0];
    const size_t lds = lds_table_bytes(m.n_tables, m.prob_bits, true) + (size_t)W * 2 * kRingBytes + (size_t)W * kFusedBuf;
    const void* k = reinterpret_cast<const void*>(decode_mfma_f8<N, MT, W>);
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_mfma_f8<N, MT, W>), dim3((unsigned)blocks), dim3(64 * W), lds, stream, g);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mfma_f8_mt(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    switch (g.m[0].prob_bits) {
        case 10: return launch_mfma_f8_n<10, MT>(g, blocks, stream);
        case 11: return launch_mfma_f8_n<11, MT>(g, blocks, stream);
        default: return launch_mfma_f8_n<12, MT>(g, blocks, stream);
    }
}

template <int MT>
hipError_t launch_mfma_mt(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    switch (g.m[0].prob_bits) {
        case 10: return launch_mfma_n<10, MT>(g, blocks, stream);
        case 11: return launch_mfma_n<11, MT>(g, blocks, stream);
        default: return launch_mfma_n<12, MT>(g, blocks, stream);
    }
}

// decode_mfma_rows over several row-layout matrices in one launch (layers that take the same
// activations, e.g. the gate and up projections of a gated FFN): the matrices' tile pairs are laid
// out matrix by matrix and weighted by their decode cost, each block owns an equal share and
// restages the decode tables when its share crosses into the next matrix, and every matrix writes
// its own partial sums, so each layer's result is the single-layer kernel's. A layer of fewer tile
// pairs than the CU's wave slots, or one whose last round of pairs is mostly empty, shares its
// rounds with the others instead of ending on a pair's latency. Same probability precision N and
// input width for all matrices.
template <int N, int MT, bool F8>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_rows_many(GroupArgs g) {
    extern __shared__ __align__(16) uint8_t smem[];
    if ((uint32_t)(size_t)(lds_u8*)smem != 0u) {
        if (threadIdx.x == 0)
            for (int i = 0; i < g.count; ++i) atomicOr(g.m[i].err, kErrLayout);
        return;
    }
    const uint64_t a = (uint64_t)blockIdx.x * g.block_cost;
    const uint64_t b = std::min<uint64_t>(a + g.block_cost, g.cost_start[g.count]);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    for (int mi = 0; mi < g.count; ++mi) {
        const uint64_t cs = g.cost_start[mi], ce = g.cost_start[mi + 1];
        if (ce <= a || cs >= b) continue;
        const MatDesc& M = g.m[mi];
        const uint64_t w = M.pair_cost;
        const uint64_t p0 = (std::max(a, cs) - cs + w - 1) / w, p1 = (std::min(b, ce) - cs + w - 1) / w;
        if (p0 >= p1) continue;
        __syncthreads();                            // every wave is done with the previous tables
        const Tables T = stage_lossy_tables_dma(M, smem);
        Tile t;
        init_lane(t, smem + lds_table_bytes(M.n_tables, M.prob_bits, true), 0);
        const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(M.gemv_x), 0, (int)((size_t)M.gemv_m * M.cols * (F8 ? 1 : 2)), 0x00020000);
        const uint32_t tiles_r = (M.rows + 15u) / 16u;          // column-major pair order, as above
        for (uint64_t p = p0 + (uint64_t)wave; p < p1; p += kWaves) {
            const uint32_t pc = (uint32_t)p / tiles_r, tr = (uint32_t)p % tiles_r;
            rows_pair<N, MT, F8>(M, T, t, (uint64_t)tr * M.pairs_c + pc, rs, rx);
        }
        if (t.err) atomicOr(M.err, t.err);
    }
}

template <int N, int MT, bool F8>
hipError_t launch_rows_n(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    const MatDesc& m = g.m[0];
    const size_t lds = lds_table_bytes(m.n_tables, m.prob_bits, true) + (size_t)kWaves * 2 * kRingBytes;
    const void* k = reinterpret_cast<const void*>(decode_mfma_rows<N, MT, F8>);
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_mfma_rows<N, MT, F8>), dim3((unsigned)blocks), dim3(64 * kWaves), lds, stream, g);
    return hipGetLastError();
}

template <int MT, bool F8>
hipError_t launch_rows_mt(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    switch (g.m[0].prob_bits) {
        case 10: return launch_rows_n<10, MT, F8>(g, blocks, stream);
        case 11: return launch_rows_n<11, MT, F8>(g, blocks, stream);
        default: return launch_rows_n<12, MT, F8>(g, blocks, stream);
    }
}

// 16-row M tiles the kernel keeps per wave: 1 for the transposing kernel, up to 4 in the row layout.
int fused_mt(const MatDesc& m, int64_t M) { return m.layout == 0 || M <= 16 ? 1 : M <= 32 ? 2 : 4; }

template <bool F8>
hipError_t launch_rows(const GroupArgs& g, int mt, uint64_t blocks, hipStream_t stream) {
    switch (mt) {
        case 1: return launch_rows_mt<1, F8>(g, blocks, stream);
        case 2: return launch_rows_mt<2, F8>(g, blocks, stream);
        default: return launch_rows_mt<4, F8>(g, blocks, stream);
    }
}

template <int N, int MT, bool F8>
hipError_t launch_rows_many_n(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    const MatDesc& m = g.m[0];
    const size_t lds = lds_table_bytes(m.n_tables, m.prob_bits, true) + (size_t)kWaves * 2 * kRingBytes;
    const void* k = reinterpret_cast<const void*>(decode_mfma_rows_many<N, MT, F8>);
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_mfma_rows_many<N, MT, F8>), dim3((unsigned)blocks), dim3(64 * kWaves), lds, stream, g);
    return hipGetLastError();
}

template <int MT, bool F8>
hipError_t launch_rows_many_mt(const GroupArgs& g, uint64_t blocks, hipStream_t stream) {
    switch (g.m[0].prob_bits) {
        case 10: return launch_rows_many_n<10, MT, F8>(g, blocks, stream);
        case 11: return launch_rows_many_n<11, MT, F8>(g, blocks, stream);
        default: return launch_rows_many_n<12, MT, F8>(g, blocks, stream);
    }
}

hipError_t launch_finish(const float* part, const float* xs, const float* sw, const uint16_t* bias, uint16_t* y,
                         int M, int rows, int pairs_c, int mt, hipStream_t stream) {
    const unsigned fb = (unsigned)(((int64_t)M * rows + 255) / 256);
    if (xs) {
        switch (mt) {
            case 1: hipLaunchKernelGGL(fused_finish_f8<1>, dim3(fb), dim3(256), 0, stream, part, xs, sw, bias, y, M, rows, pairs_c); break;
            case 2: hipLaunchKernelGGL(fused_finish_f8<2>, dim3(fb), dim3(256), 0, stream, part, xs, sw, bias, y, M, rows, pairs_c); break;
            default: hipLaunchKernelGGL(fused_finish_f8<4>, dim3(fb), dim3(256), 0, stream, part, xs, sw, bias, y, M, rows, pairs_c); break;
        }
    } else {
        switch (mt) {
            case 1: hipLaunchKernelGGL(fused_finish<1>, dim3(fb), dim3(256), 0, stream, part, bias, y, M, rows, pairs_c); break;
            case 2: hipLaunchKernelGGL(fused_finish<2>, dim3(fb), dim3(256), 0, stream, part, bias, y, M, rows, pairs_c); break;
            default: hipLaunchKernelGGL(fused_finish<4>, dim3(fb), dim3(256), 0, stream, part, bias, y, M, rows, pairs_c); break;
        }
    }
    return hipGetLastError();
}

}  // namespace

bool fused_fits(const MatDesc& m, int64_t M) {
    // X is addressed through one buffer resource with 32-bit byte offsets
    const int max_rows = m.layout ? kFusedMaxRowsRowLayout : kFusedMaxRows;
    return m.mode == 0 && m.tile_rows == 16 && M >= 1 && M <= max_rows && (m.cols & 7) == 0 &&
           (uint64_t)kFusedMaxRowsRowLayout * m.cols * 2 < (1ull << 31);
}

size_t fused_partial_bytes(const MatDesc& m, int64_t M) {
    const uint64_t pairs = (uint64_t)((m.rows + m.tile_rows - 1) / m.tile_rows) * m.pairs_c;
    return (size_t)pairs * (size_t)fused_mt(m, M) * 256 * sizeof(float);   // a 16 x 16 fp32 tile per M tile
}

hipError_t launch_fused(const MatDesc& m, const uint16_t* x, int64_t M, float* part, const uint16_t* bias,
                        uint16_t* y, hipStream_t stream) {
    if (!fused_fits(m, M)) return hipErrorInvalidValue;
    GroupArgs g{};
    g.count = 1;
    g.m[0] = m;
    g.m[0].gemv_x = x;
    g.m[0].gemv_m = (uint8_t)M;
    g.m[0].out = part;
    const uint64_t pairs = (uint64_t)((m.rows + m.tile_rows - 1) / m.tile_rows) * m.pairs_c;
    const uint64_t total = pairs * m.pair_cost;
    g.cost_start[0] = 0;
    g.cost_start[1] = total;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (uint64_t)device_cus();
    g.block_cost = (total + blocks - 1) / blocks;
    const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
    const int mt = fused_mt(m, M);
    hipError_t e = m.layout ? launch_rows<false>(g, mt, used, stream) : launch_mfma_mt<1>(g, used, stream);
    if (e != hipSuccess) return e;
    return launch_finish(part, nullptr, nullptr, bias, y, (int)M, (int)m.rows, (int)m.pairs_c, mt, stream);
}


hipError_t launch_fused_f8(const MatDesc& m, const uint8_t* xq, const float* xs, int64_t M, float* part,
                           const uint16_t* bias, uint16_t* y, hipStream_t stream) {
    if (!fused_fits(m, M) || (m.cols & 15)) return hipErrorInvalidValue;
    GroupArgs g{};
    g.count = 1;
    g.m[0] = m;
    g.m[0].gemv_x = reinterpret_cast<const uint16_t*>(xq);
    g.m[0].gemv_m = (uint8_t)M;
    g.m[0].out = part;
    const uint64_t pairs = (uint64_t)((m.rows + m.tile_rows - 1) / m.tile_rows) * m.pairs_c;
    const uint64_t total = pairs * m.pair_cost;
    g.cost_start[0] = 0;
    g.cost_start[1] = total;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (uint64_t)device_cus();
    g.block_cost = (total + blocks - 1) / blocks;
    const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
    const int mt = fused_mt(m, M);
    hipError_t e = m.layout ? launch_rows<true>(g, mt, used, stream) : launch_mfma_f8_mt<1>(g, used, stream);
    if (e != hipSuccess) return e;
    return launch_finish(part, xs, m.row_scale, bias, y, (int)M, (int)m.rows, (int)m.pairs_c, mt, stream);
}

bool fused_many_fits(const MatDesc* ms, int count, int64_t M) {
    if (count < 1 || count > kMaxGroup) return false;
    for (int i = 0; i < count; ++i)
        if (!fused_fits(ms[i], M) || ms[i].layout != 1 || ms[i].prob_bits != ms[0].prob_bits ||
            ms[i].cols != ms[0].cols)
            return false;
    return true;
}

namespace {
// launch_fused_many and launch_fused_many_f8: x the BF16 activations, or the E4M3 codes with their
// row scales xs (F8)
template <bool F8>
hipError_t fused_many(const MatDesc* ms, int count, const void* x, const float* xs, int64_t M, float* const* parts,
                      const uint16_t* const* bias, uint16_t* const* y, hipStream_t stream) {
    if (!fused_many_fits(ms, count, M) || (F8 && (ms[0].cols & 15))) return hipErrorInvalidValue;
    GroupArgs g{};
    g.count = count;
    uint64_t total = 0;
    for (int i = 0; i < count; ++i) {
        g.m[i] = ms[i];
        g.m[i].gemv_x = static_cast<const uint16_t*>(x);
        g.m[i].gemv_m = (uint8_t)M;
        g.m[i].out = parts[i];
        g.cost_start[i] = total;
        total += (uint64_t)((ms[i].rows + ms[i].tile_rows - 1) / ms[i].tile_rows) * ms[i].pairs_c * ms[i].pair_cost;
    }
    g.cost_start[count] = total;
    const int mt = fused_mt(ms[0], M);
    if (total > 0) {
        const uint64_t blocks = (uint64_t)device_cus();
        g.block_cost = (total + blocks - 1) / blocks;
        const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
        hipError_t e;
        switch (mt) {
            case 1: e = launch_rows_many_mt<1, F8>(g, used, stream); break;
            case 2: e = launch_rows_many_mt<2, F8>(g, used, stream); break;
            default: e = launch_rows_many_mt<4, F8>(g, used, stream); break;
        }
        if (e != hipSuccess) return e;
    }
    for (int i = 0; i < count; ++i) {
        if ((uint64_t)ms[i].rows * ms[i].cols == 0) continue;
        hipError_t e = launch_finish(parts[i], F8 ? xs : nullptr, F8 ? ms[i].row_scale : nullptr, bias[i], y[i], (int)M,
                                     (int)ms[i].rows, (int)ms[i].pairs_c, mt, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace

hipError_t launch_fused_many(const MatDesc* ms, int count, const uint16_t* x, int64_t M, float* const* parts,
                             const uint16_t* const* bias, uint16_t* const* y, hipStream_t stream) {
    return fused_many<false>(ms, count, x, nullptr, M, parts, bias, y, stream);
}

hipError_t launch_fused_many_f8(const MatDesc* ms, int count, const uint8_t* xq, const float* xs, int64_t M,
                                float* const* parts, const uint16_t* const* bias, uint16_t* const* y,
                                hipStream_t stream) {
    return fused_many<true>(ms, count, xq, xs, M, parts, bias, y, stream);
}
}  // namespace ep
