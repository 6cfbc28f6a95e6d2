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
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "kernels.h"

namespace ep {
namespace {

constexpr uint32_t kLow = 1u << 16;
constexpr int kWaves = 16;                 // waves per block
constexpr int kRingWords = 1024;           // per tile
constexpr int kTopUps = kRingWords >= 1024 ? 1 : 3;   // ring top-ups per block row (see top_up)
constexpr int kRingBytes = 2 * kRingWords;
constexpr int kChains = 1;                 // tile pairs decoded together by a wave (see lossy_pairs)
constexpr int kChunkDw = 128;              // one chunk: 32 lanes x 4 dwords = 256 words
constexpr int kChunkWords = 2 * kChunkDw;
constexpr int kErrWords = 1;               // words ran out or were left over
constexpr int kErrState = 2;               // a final state differs from 2^16
constexpr int kErrLayout = 4;              // the kernel's LDS does not start at address 0

// ----------------------------------------------------------------------------- containers
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne(float v) {
    uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;      // finite inputs only
}
// The fp32 product is rounded first and then converted: without the register barrier the
// backend folds "multiply then narrow" into one mixed-precision FMA that rounds only once,
// which differs from the two-step rounding in rare ties.
__device__ __forceinline__ float materialize(float v) {
    asm volatile("" : "+v"(v));
    return v;
}
// The signed 16-bit value in the high half of v as fp32, in one conversion (SDWA word select with
// sign extension).
__device__ __forceinline__ float hi16_to_f32(uint32_t v) {
    float r;
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ uint32_t f16_rne(float v) {
    _Float16 h = (_Float16)materialize(v);               // v_cvt_f16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// ----------------------------------------------------------------------------- matrix setup
typedef const __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

struct Tables {
    const uint8_t* lut;
    const uint2* ent;
};

__device__ __forceinline__ Tables stage_tables(const MatDesc& M, uint8_t* smem, bool lossy) {
    const int n = M.prob_bits;
    const int skip = lossy ? 1 : 0;                 // the coset table stays out of LDS
    const int nt = M.n_tables - skip;
    const size_t lut_bytes = (size_t)nt << n, ent_bytes = (size_t)nt * 2048;
    const uint4* lut_src = reinterpret_cast<const uint4*>(M.tables + ((size_t)skip << n));
    const uint4* ent_src = reinterpret_cast<const uint4*>(M.tables + ((size_t)M.n_tables << n) + (size_t)skip * 2048);
    uint4* dst = reinterpret_cast<uint4*>(smem);
    for (size_t i = threadIdx.x; i < lut_bytes / 16; i += blockDim.x) dst[i] = lut_src[i];
    for (size_t i = threadIdx.x; i < ent_bytes / 16; i += blockDim.x) dst[lut_bytes / 16 + i] = ent_src[i];
    __syncthreads();
    Tables T;
    T.lut = smem;
    T.ent = reinterpret_cast<const uint2*>(smem + lut_bytes);
    return T;
}

// ----------------------------------------------------------------------------- one half-wave tile
struct Tile {
    uint32_t x;            // rANS state of this lane
    uint32_t pos;          // words consumed
    uint32_t fill;         // words placed in the ring (multiple of 256)
    uint32_t nwords;       // words of the tile (pad word included)
    uint32_t ndw;          // the same in dwords
    uint32_t gdw;          // byte offset of the tile's words in the payload (buffer loads)
    lds_u16* ring;         // this half's LDS ring
    uint32_t pf[4];        // next chunk, loaded ahead
    uint32_t below;        // lanes below this one within the half
    uint32_t sh;           // 0 for the low half, 32 for the high half
    int l;                 // lane within the half
    bool valid;
    int err;
};

// Chunk loads go through a buffer resource over the matrix payload; lanes whose dword lies past
// the tile (or that have no tile) use an out-of-range offset, which the buffer unit answers with
// 0 without touching memory.
__device__ __forceinline__ void load_chunk(const Tile& t, __amdgpu_buffer_rsrc_t rs, uint32_t chunk, uint32_t* dst) {
    const uint32_t d = chunk * kChunkDw + t.l;
    const uint32_t off = t.gdw + 4u * d;
    // only the tile's own words are fetched: other lanes take an out-of-range offset (reads 0);
    // arithmetic rather than a select, which the backend would turn into branches around loads
    const uint32_t lim = t.valid ? t.ndw : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t oob = (uint32_t)((int32_t)(d + 32u * i - lim) >> 31) ^ 0xFFFFFFFFu;   // d + 32 i >= lim
        dst[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (off + 128u * i) | (oob & 0x80000000u), 0, 0);
    }
}
__device__ __forceinline__ void store_chunk(Tile& t, uint32_t chunk, const uint32_t* src) {
    lds_u32* ring = (lds_u32*)t.ring;
    const uint32_t base = (chunk * kChunkDw) & (kRingWords / 2 - 1);   // kRingWords / 2 dwords
#pragma unroll
    for (int i = 0; i < 4; ++i) ring[base + t.l + 32 * i] = src[i];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t payload_rsrc(const MatDesc& M) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(M.payload), 0, (int)M.payload_bytes, 0x00020000);
}

__device__ __forceinline__ void begin_tile(const MatDesc& M, __amdgpu_buffer_rsrc_t rs, uint64_t tile, Tile& t) {
    if (t.valid) {
        const uint32_t a = M.index[tile], b = M.index[tile + 1];
        t.x = M.payload[a + t.l];
        t.gdw = 4u * (a + 32);
        t.ndw = b - a - 32;
    } else {
        t.x = kLow;
        t.gdw = 0;
        t.ndw = 0;
    }
    t.nwords = 2 * t.ndw;
    t.pos = 0;
    constexpr int kFirst = kRingWords / kChunkWords;
    uint32_t first[4 * kFirst];
#pragma unroll
    for (int k = 0; k < kFirst; ++k) load_chunk(t, rs, k, first + 4 * k);
#pragma unroll
    for (int k = 0; k < kFirst; ++k) store_chunk(t, k, first + 4 * k);
    t.fill = kRingWords;
    load_chunk(t, rs, kFirst, t.pf);
    __builtin_amdgcn_wave_barrier();
}

// After a top-up the ring holds more than kRingWords - kChunkWords unread words (768 with the
// 1024-word ring: more than a block row's worst case of 9 steps x 64 words; 256 with a 512-word
// ring, which then needs kTopUps = 3 top-ups per row), or the rest of the tile.
__device__ __forceinline__ void top_up(Tile& t, __amdgpu_buffer_rsrc_t rs) {
    while (t.fill < t.nwords && t.fill - t.pos <= kRingWords - kChunkWords) {
        store_chunk(t, t.fill / kChunkWords, t.pf);
        t.fill += kChunkWords;
        if (t.fill < t.nwords) load_chunk(t, rs, t.fill / kChunkWords, t.pf);
    }
    __builtin_amdgcn_wave_barrier();
}

// Word for each lane in `need`, compacted in ascending lane order per half. Branch-free: every
// lane reads the ring (always in range) and the caller keeps the word only where it was needed.
__device__ __forceinline__ uint32_t take_words(Tile& t, bool need) {
    const uint64_t m = __ballot(need);
    const uint32_t mine = (uint32_t)(m >> t.sh);
    const uint32_t idx = t.pos + __popc(mine & t.below);
    const uint32_t w = t.ring[idx & (kRingWords - 1)];
    t.pos += __popc(mine);
    return w;
}

__device__ __forceinline__ void refill(Tile& t) {
    const bool need = t.x < kLow;
    const uint32_t w = take_words(t, need);
    t.x = need ? (t.x << 16) | w : t.x;
}

// refill() for C chains, written phase by phase so that the chains' LDS reads are in flight
// together.
template <int C>
__device__ __forceinline__ void refill_all(Tile* t) {
    bool need[C];
    uint32_t idx[C], w[C];
#pragma unroll
    for (int c = 0; c < C; ++c) need[c] = t[c].x < kLow;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint32_t mine = (uint32_t)(__ballot(need[c]) >> t[c].sh);
        idx[c] = t[c].pos + __popc(mine & t[c].below);
        t[c].pos += __popc(mine);
    }
    // volatile: read by every lane (always in range), so the compiler keeps the selects below
    // instead of branching around the reads
#pragma unroll
    for (int c = 0; c < C; ++c) w[c] = *(volatile lds_u16*)(t[c].ring + (idx[c] & (kRingWords - 1)));
#pragma unroll
    for (int c = 0; c < C; ++c) t[c].x = need[c] ? (t[c].x << 16) | w[c] : t[c].x;
}

// One rANS decode step. The lookup address is the slot or'ed into `base` (the LDS offset of the
// lane's LUT group, a multiple of 2^N), `lut` adds the step's table (an absolute LDS byte address:
// the LUTs start at LDS address 0, which the kernel checks, so this is an immediate offset), and
// `ent` points at the entries of the same table; the entry's cumulative frequency carries `base`,
// so slot - c is the address minus that field. Returns the symbol; `v` receives the entry's
// second word (value in the high half). f <= 2^12 and x >> N < 2^22 fit the 24-bit multiplier.
template <int N>
__device__ __forceinline__ uint32_t rans_step(Tile& t, uint32_t lut, uint32_t base, const uint2* ent, uint32_t& v) {
    uint32_t a;                                         // (x & (2^N - 1)) | base in one instruction
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(a) : "v"(t.x), "s"((1u << N) - 1u), "v"(base));
    const uint32_t s = ((lds_u8*)(size_t)lut)[a];      // LDS byte address lut + a
    const uint2 e = ent[s];
    t.x = __umul24(e.x, t.x >> N) + (a - (e.y & 0xFFFFu));
    v = e.y;
    return s;
}

// rans_step() for C chains at the same step, phase by phase (see refill_all).
// Returns each chain's entry: .x = frequency (bit 31: escape symbol), .y = value << 16 | c + base.
template <int N, int C>
__device__ __forceinline__ void rans_steps(Tile* t, uint32_t lut, const uint32_t* base, const uint2* const* ent,
                                           uint2* e) {
    uint32_t a[C], s[C];
#pragma unroll
    for (int c = 0; c < C; ++c) asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(a[c]) : "v"(t[c].x), "s"((1u << N) - 1u), "v"(base[c]));
#pragma unroll
    for (int c = 0; c < C; ++c) s[c] = ((lds_u8*)(size_t)lut)[a[c]];
#pragma unroll
    for (int c = 0; c < C; ++c) e[c] = ent[c][s[c]];
#pragma unroll
    for (int c = 0; c < C; ++c) t[c].x = __umul24(e[c].x, t[c].x >> N) + (a[c] - (e[c].y & 0xFFFFu));
}

// The coset table has at most two symbols (0 and 1, cumulative 0 and f0), decoded arithmetically.
template <int N>
__device__ __forceinline__ uint32_t coset_step(Tile& t, uint32_t f0, uint32_t f1) {
    const uint32_t slot = t.x & ((1u << N) - 1u);
    const bool one = slot >= f0;
    const uint32_t f = one ? f1 : f0;
    const uint32_t c = one ? f0 : 0u;
    t.x = __umul24(f, t.x >> N) + slot - c;
    return one ? 1u : 0u;
}

__device__ __forceinline__ void end_tile(Tile& t) {
    if (!t.valid) return;
    if (t.x != kLow) t.err |= kErrState;
    const bool exact = t.pos == t.nwords;
    const bool loaded = t.fill >= t.nwords;
    const bool pad = t.pos + 1 == t.nwords && t.ring[t.pos & (kRingWords - 1)] == 0;
    if (!loaded || (!exact && !pad)) t.err |= kErrWords;
}

// Lane constants; each (wave, chain, half) owns one ring.
__device__ __forceinline__ void init_lane(Tile& t, uint8_t* ring_base, int chain) {
    const int lane = threadIdx.x & 63;
    t.l = lane & 31;
    t.sh = (uint32_t)(lane & 32);
    t.below = (1u << t.l) - 1u;
    const int ring = ((threadIdx.x >> 6) * kChains + chain) * 2 + (lane >> 5);
    t.ring = (lds_u16*)(ring_base + ring * kRingBytes);
    t.err = 0;
    t.valid = false;
}

// ----------------------------------------------------------------------------- stores
// Decoded coordinates are carried as fp32 values (exact: |q| < 2^17).
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
        const int32_t q = (int32_t)qf;
        const uint32_t a = (uint32_t)(q < 0 ? -q : q);
        const int32_t v = (int32_t)__umulhi(2u * a + k, magic);
        return (uint32_t)(uint8_t)(int8_t)(q < 0 ? -v : v);
    }
};
template <>
struct Conv<CT_Q16> {
    using T = uint16_t;
    __device__ static uint32_t f(float q, float, float, uint32_t, uint32_t) { return (uint32_t)(uint16_t)(int16_t)(int32_t)q; }
};

template <int CT>
__device__ __forceinline__ void store_block(const MatDesc& M, uint32_t row, uint32_t col0, const float* q, float alpha,
                                   float h, uint32_t k, uint32_t magic) {
    using T = typename Conv<CT>::T;
    T* out = static_cast<T*>(M.out) + (size_t)row * M.cols;
    uint32_t v[8];
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
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = Conv<CT>::f(q[j], alpha, h, k, magic);
    }
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

// ----------------------------------------------------------------------------- lossy kernel
// Rows of one tile pair: tile coordinates and the per-row scales, one row per lane, read back
// per row with readlane. INT8: the row's divisor k and its reciprocal multiplier, computed once
// per pair by each lane for its row (a vector division per pair instead of a scalar one per row).
struct PairRows {
    uint32_t tc, row0;
    float sc_l;
    uint32_t k_l, magic_l;
    float xv[4][8];        // fused matrix-vector product: the lane's 8 activation columns per row m
};

constexpr int gemv_rows(int CT) { return CT >= CT_GEMV1 ? CT - 100 : 0; }

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

template <int CT>
__device__ __forceinline__ void begin_pair(const MatDesc& M, __amdgpu_buffer_rsrc_t rs, uint64_t pair, bool live,
                                           Tile& t, PairRows& P) {
    const uint32_t tr = (uint32_t)(pair / M.pairs_c);
    P.tc = 2 * (uint32_t)(pair % M.pairs_c) + (t.sh ? 1u : 0u);
    t.valid = live && P.tc < M.tiles_c;
    begin_tile(M, rs, (uint64_t)tr * M.tiles_c + P.tc, t);
    P.row0 = tr * M.tile_rows;
    const uint32_t my_row = P.row0 + t.l;
    const bool mine = t.l < M.tile_rows && my_row < M.rows;
    P.sc_l = mine ? M.row_scale[my_row] : 0.0f;
    P.k_l = 1;
    P.magic_l = 0;
    if constexpr (CT == CT_I8) {
        const uint32_t qm = mine ? M.row_qmax[my_row] : 0u;
        P.k_l = qm > 127u ? (qm + 126u) / 127u : 1u;
        P.magic_l = 0xFFFFFFFFu / (2u * P.k_l) + 1u;
    }
    if constexpr (gemv_rows(CT) > 0) {
        // the lane's 8 columns of each activation row; zeros past the matrix or the tile pair
        const uint32_t col0 = P.tc * 256 + 8 * t.l;
#pragma unroll
        for (int m = 0; m < gemv_rows(CT); ++m) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (t.valid && col0 < M.cols && m < M.gemv_m)
                v = *reinterpret_cast<const uint4*>(M.gemv_x + (size_t)m * M.cols + col0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P.xv[m][2 * i] = __uint_as_float(w[i] << 16);
                P.xv[m][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                asm volatile("" ::"v"(P.xv[m][2 * i]), "v"(P.xv[m][2 * i + 1]));
            }
        }
    }
    // Wait for these loads here, once per pair: first used inside the row loop, their wait would
    // land inside it, on every row, and (the vector-memory counter being in order) would also
    // wait for the ring chunk just prefetched.
    asm volatile("" ::"v"(P.sc_l), "v"(P.k_l), "v"(P.magic_l), "v"(t.x));
}

template <int CT>
__device__ __forceinline__ void store_row(const MatDesc& M, const Tile& t, const PairRows& P, int rr, const float* q,
                                          float h) {
    if constexpr (gemv_rows(CT) > 0) {
        // fused matrix-vector product: the row's dot products with every activation row, summed
        // over the wave (both tiles of the pair cover the same rows) and added to Y by lane 63
        constexpr int MT = gemv_rows(CT);
        const uint32_t row = P.row0 + rr;
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, P.sc_l), rr));
        if (row >= M.rows) return;
        const float alpha = h * sc;
        float s[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc += P.xv[m][i] * q[i];
            s[m] = wave_sum_to_lane63(acc * alpha);
        }
        if ((threadIdx.x & 63) == 63) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < M.gemv_m) atomicAdd(static_cast<float*>(M.out) + (size_t)m * M.rows + row, s[m]);
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
template <int CT, int N, int C>
__device__ __forceinline__ void lossy_run(const MatDesc& M, const Tables& T, Tile* t, const uint64_t* pair,
                                          uint64_t pend) {
    const float h = M.step * 0.5f;
    const uint2* coset = reinterpret_cast<const uint2*>(M.tables + ((size_t)M.n_tables << N));   // table 0
    const uint32_t f0 = coset[0].x, f1 = coset[1].x;
    const int lo0 = (int32_t)coset[0].y >> 16;
    const __amdgpu_buffer_rsrc_t rs = payload_rsrc(M);
    PairRows P[C];
#pragma unroll
    for (int c = 0; c < C; ++c) begin_pair<CT>(M, rs, pair[c], pair[c] < pend, t[c], P[c]);
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
            for (int c = 0; c < C; ++c) store_row<CT>(M, t[c], P[c], rr - 1, qp[c], h);
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
            for (int c = 0; c < C; ++c) q[c][j] = hi16_to_f32(e[c].y);
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
                        if (esc[c]) q[c][j] = (float)(int32_t)(int16_t)(2 * (int32_t)(int16_t)w + b[c]);
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
    for (int c = 0; c < C; ++c) store_row<CT>(M, t[c], P[c], M.tile_rows - 1, qp[c], h);
#pragma unroll
    for (int c = 0; c < C; ++c) end_tile(t[c]);
}

// Pairs [p0, p1) of one matrix: wave w decodes pairs p0 + w and p0 + w + 16 together, then
// p0 + w + 32 and p0 + w + 48, ...: two independent chains per lane keep the SIMDs busy while
// the other chain waits on LDS.
template <int CT, int N>
__device__ __forceinline__ void lossy_pairs(const MatDesc& M, const Tables& T, Tile* t, uint64_t p0, uint64_t p1) {
    // the wave's index is uniform across its lanes: keep it (and so the pair, tile row and row
    // addresses) in SGPRs
    const uint64_t w0 = (uint64_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    for (uint64_t p = p0 + w0; p < p1; p += kChains * kWaves) {
        uint64_t pr[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) pr[c] = p + (uint64_t)c * kWaves;
        lossy_run<CT, N, kChains>(M, T, t, pr, p1);
    }
}

template <int N>
__device__ __forceinline__ void lossy_dispatch(const MatDesc& M, const Tables& T, Tile* t, uint64_t p0, uint64_t p1) {
    switch (M.container) {
        case CT_BF16: lossy_pairs<CT_BF16, N>(M, T, t, p0, p1); break;
        case CT_F16: lossy_pairs<CT_F16, N>(M, T, t, p0, p1); break;
        case CT_F8E4M3: lossy_pairs<CT_F8E4M3, N>(M, T, t, p0, p1); break;
        case CT_I8: lossy_pairs<CT_I8, N>(M, T, t, p0, p1); break;
        default: lossy_pairs<CT_Q16, N>(M, T, t, p0, p1); break;
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
template <int GEMV>
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
        const Tables T = stage_tables(M, smem, lossy);
        Tile t[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) init_lane(t[c], smem + lds_table_bytes(M.n_tables, M.prob_bits, lossy), c);
        if constexpr (GEMV > 0) {
            switch (M.prob_bits) {
                case 10: lossy_pairs<GEMV, 10>(M, T, t, p0, p1); break;
                case 11: lossy_pairs<GEMV, 11>(M, T, t, p0, p1); break;
                default: lossy_pairs<GEMV, 12>(M, T, t, p0, p1); break;
            }
        } else if (lossy) {
            switch (M.prob_bits) {
                case 10: lossy_dispatch<10>(M, T, t, p0, p1); break;
                case 11: lossy_dispatch<11>(M, T, t, p0, p1); break;
                default: lossy_dispatch<12>(M, T, t, p0, p1); break;
            }
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

template <int CT>
__global__ __launch_bounds__(64 * kWaves) void decode_gemv(GroupArgs g) { group_body<CT>(g); }

__global__ __launch_bounds__(256) void gemv_zero(float* y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = 0.0f;
}

__global__ __launch_bounds__(256) void gemv_finish(const float* yacc, const uint16_t* bias, uint16_t* y, int64_t M,
                                                   int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    float v = yacc[i];
    if (bias) v += __uint_as_float((uint32_t)bias[i % N] << 16);
    y[i] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.0f}, bf16x2)) & 0xFFFFu);
}


// Allow a kernel the full 160 KiB of LDS, once per device.
hipError_t allow_lds(const void* kernel) {
    static std::mutex mu;
    static std::set<std::pair<int, const void*>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(mu);
    if (done.count({dev, kernel})) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess) done.insert({dev, kernel});
    return e;
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

hipError_t launch_group(const MatDesc* mats, int count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    if (count > kMaxGroup) return hipErrorInvalidValue;
    GroupArgs g{};
    g.count = count;
    uint64_t total = 0;
    size_t lds = 0;
    for (int i = 0; i < count; ++i) {
        g.m[i] = mats[i];
        g.cost_start[i] = total;
        const uint64_t pairs = (uint64_t)((mats[i].rows + mats[i].tile_rows - 1) / mats[i].tile_rows) * mats[i].pairs_c;
        total += pairs * mats[i].pair_cost;
        if (pairs)
            lds = std::max(lds, lds_table_bytes(mats[i].n_tables, mats[i].prob_bits, mats[i].mode == 0) +
                                    (size_t)kWaves * kChains * 2 * kRingBytes);
    }
    g.cost_start[count] = total;
    if (total == 0) return hipSuccess;
    const uint64_t blocks = (uint64_t)device_cus();
    g.block_cost = (total + blocks - 1) / blocks;
    const uint64_t used = (total + g.block_cost - 1) / g.block_cost;
    const void* k = reinterpret_cast<const void*>(decode_group);
    hipError_t e = allow_lds(k);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_group, dim3((unsigned)used), dim3(64 * kWaves), lds, stream, g);
    return hipGetLastError();
}

hipError_t launch_gemv(const MatDesc& m, hipStream_t stream) {
    if (m.mode != 0 || m.gemv_m == 0 || m.gemv_m > gemv_rows(m.container)) return hipErrorInvalidValue;
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

hipError_t launch_gemv_zero(float* yacc, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, yacc, n);
    return hipGetLastError();
}

hipError_t launch_gemv_finish(const float* yacc, const uint16_t* bias, uint16_t* y, int64_t M, int64_t N,
                              hipStream_t stream) {
    if (M * N <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_finish, dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, stream, yacc, bias, y, M, N);
    return hipGetLastError();
}

}  // namespace ep
