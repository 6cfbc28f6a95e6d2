// Device-side building blocks of the tile-rANS decode kernels (decode.hip) and of the decode fused
// into the matrix product (fused.hip): the LDS tables, the half-wave tile with its LDS word ring,
// one rANS step, the coset step, and the per-pair row metadata. Kernel-private (anonymous
// namespace): each kernel source gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <set>
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

// stage_tables for a lossy matrix by direct global -> LDS loads (buffer_load ... lds): each wave
// instruction moves 1 KiB (64 lanes x 16 bytes) with no registers staging it, and a wave issues
// all of its loads before it waits, where stage_tables' copy waits for each 16-byte load in turn
// (four to six global round trips). For kernels that stage once per launch, mostly: the fused
// kernels (row layout at M = 1: 77.0 -> 76.1 us) and the row-layout decode, whose launches are
// mostly one layer's weight slice each. In the layout-0 decode, which restages per matrix inside
// its pair loop, the resource and loop state pushed the scalar registers into spills (1160 more
// v_readlane, DiT-like step 837 -> 872 us per launch). prob_bits >= 10: both arrays whole KiB.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t src, uint8_t* dst, uint32_t bytes) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t nw = blockDim.x >> 6;
    for (uint32_t g = wave; g < bytes / 1024; g += nw)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + 1024 * g), 16, src + 1024 * g + 16 * lane, 0, 0, 0);
}

__device__ __forceinline__ Tables stage_lossy_tables_dma(const MatDesc& M, uint8_t* smem) {
    const int n = M.prob_bits, nt = M.n_tables - 1;        // the coset table stays out of LDS
    const uint32_t lut_bytes = (uint32_t)nt << n, ent_bytes = (uint32_t)nt * 2048u;
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(M.tables), 0, (int)table_blob_bytes(M.n_tables, n), 0x00020000);
    dma_to_lds(rt, 1u << n, smem, lut_bytes);
    dma_to_lds(rt, ((uint32_t)M.n_tables << n) + 2048u, smem + lut_bytes, ent_bytes);
    __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0): this wave's loads have landed
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

// Rows of one tile pair: tile coordinates and the per-row scales, one row per lane: in layout 0
// lane l holds tile row l's, read back per row with readlane; in layout 1 the row the lane codes
// (tile row l mod tile_rows), used by the lane itself. INT8: the row's divisor k and its
// reciprocal multiplier, computed once per pair by each lane for its row (a vector division per
// pair instead of a scalar one per row).
struct PairRows {
    uint32_t tc, row0;
    float sc_l;
    uint32_t k_l, magic_l;
    float xv[4][8];        // fused matrix-vector product: the lane's 8 activation columns per row m
};

constexpr int gemv_rows(int CT) { return CT >= CT_GEMV1 ? CT - 100 : 0; }

template <int CT, bool ROWS = false>
__device__ __forceinline__ void begin_pair(const MatDesc& M, __amdgpu_buffer_rsrc_t rs, uint64_t pair, bool live,
                                           Tile& t, PairRows& P) {
    const uint32_t tr = (uint32_t)(pair / M.pairs_c);
    P.tc = 2 * (uint32_t)(pair % M.pairs_c) + (t.sh ? 1u : 0u);
    t.valid = live && P.tc < M.tiles_c;
    begin_tile(M, rs, (uint64_t)tr * M.tiles_c + P.tc, t);
    P.row0 = tr * M.tile_rows;
    const uint32_t my_l = ROWS ? (uint32_t)t.l & (M.tile_rows - 1u) : (uint32_t)t.l;   // tile_rows: 16 or 32
    const uint32_t my_row = P.row0 + my_l;
    const bool mine = my_l < M.tile_rows && my_row < M.rows;
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
}  // namespace ep
