// gfx950 decode kernels of the tile-rANS weight codec.
//
// "The final coordinates are entropy-coded in independently decodable tiles, enabling fast,
// fused symbol decoding and numerical weight reconstruction on the GPU", with BF16, FP16, FP8 and
// INT8 containers ("EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
// Bitrates", Abstract). Lossless byte-plane tiles follow the lossless tile-ANS contract named in
// "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", "Choose a compression
// contract".
//
// Work mapping. A tile is tile_rows x 256 weights coded by 32 interleaved rANS states; lane l of
// a tile owns the 8-column block l of every tile row. One wave64 decodes two horizontally
// adjacent tiles of the same tile row: lanes 0-31 the even tile, lanes 32-63 the odd one, so
// every decoded block row becomes one contiguous store of 1 KiB (BF16) per wave, and both halves
// share the row's scale. Blocks of 16 waves stage the symbol tables of the matrix in LDS once
// and walk tile pairs persistently.
//
// Per decoding step every lane looks up its slot in the LDS table, updates its state, and lanes
// whose state fell below 2^16 take the next word of their tile; a wave ballot plus a popcount of
// the lower lanes gives each refilling lane its word index, so each half reads one compact run
// of words. Lanes that decoded the escape symbol then read their raw value the same way.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <set>

#include "kernels.h"

namespace ep {
namespace {

constexpr uint32_t kLow = 1u << 16;
constexpr int kWavesPerBlock = 16;
constexpr int kErrWords = 1;    // a tile ran out of words / did not end on its last word
constexpr int kErrState = 2;    // a final state differs from 2^16

// ----------------------------------------------------------------------------- containers
__device__ inline uint32_t bf16_rne(float v) {
    uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;      // finite inputs only
}
// The fp32 product is rounded first and then converted: without the register barrier the
// backend folds "multiply then narrow" into one mixed-precision FMA that rounds only once,
// which differs from the two-step rounding in rare ties.
__device__ inline float materialize(float v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ inline uint32_t f16_rne(float v) {
    _Float16 h = (_Float16)materialize(v);               // v_cvt_f16_f32: round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// OCP E4M3FN, round to nearest even, saturating at +-448.
__device__ inline uint32_t e4m3_rne_sat(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7FFFFFFFu;
    uint32_t r;
    if (u >= 0x43E00000u) {                              // >= 448 (448..464 rounds to 448 too)
        r = 0x7Eu;
    } else if (u < 0x3C800000u) {                        // below 2^-6: subnormal grid of 2^-9
        float m = __builtin_rintf(__uint_as_float(u) * 512.0f);
        r = (uint32_t)m;                                 // 8 -> 0x08, the smallest normal
    } else {
        u += 0x7FFFFu + ((u >> 20) & 1u);                // round the mantissa to 3 bits
        uint32_t e = (u >> 23) - 127u + 7u;
        r = (e << 3) | ((u >> 20) & 7u);
        if (r > 0x7Eu) r = 0x7Eu;
    }
    return r | sign;
}

// ----------------------------------------------------------------------------- LDS tables
// lut[t][slot] = symbol; sym[t][s] = (f | c << 13) | (int64)value << 32, where value is the
// doubled coordinate 2 (lo + s) + b for lossy coordinate tables, the coset b for table 0 and the
// byte s for lossless planes.
struct Lds {
    const uint8_t* lut;
    const uint64_t* sym;
};

__device__ inline void stage_tables(const DecodeParams& p, uint8_t* smem, Lds* L) {
    const size_t lut_bytes = (size_t)p.n_tables << p.prob_bits;
    const size_t total = lut_bytes + (size_t)p.n_tables * 256 * 8;
    const uint4* src = reinterpret_cast<const uint4*>(p.tables);
    uint4* dst = reinterpret_cast<uint4*>(smem);
    for (size_t i = threadIdx.x; i < total / 16; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
    L->lut = smem;
    L->sym = reinterpret_cast<const uint64_t*>(smem + lut_bytes);
}

struct Lane {
    uint32_t x;          // rANS state
    uint32_t pos;        // next word of this half's tile
    uint32_t nwords;     // words in this half's tile
    const uint16_t* words;
    bool valid;          // this half has a tile
    int half, l;         // half of the wave, lane within the half
    int err;
};

__device__ inline uint32_t half_mask(uint64_t m, int half) {
    return half ? (uint32_t)(m >> 32) : (uint32_t)m;
}

// Decode one symbol of table t; returns the table entry of the decoded symbol (with bit 63 of
// nothing special: the escape symbol is reported through *sym_out).
__device__ inline uint64_t rans_step(Lane& s, const Lds& L, int t, int n, uint32_t* sym_out) {
    const uint32_t slot = s.x & ((1u << n) - 1u);
    const uint32_t sy = L.lut[((uint32_t)t << n) + slot];
    const uint64_t e = L.sym[t * 256 + sy];
    const uint32_t fc = (uint32_t)e;
    s.x = (fc & 0x1FFFu) * (s.x >> n) + slot - (fc >> 13);
    *sym_out = sy;
    return e;
}

// Take the next word for every lane in `need`, compacted in ascending lane order per half.
__device__ inline uint32_t take_words(Lane& s, bool need) {
    const uint32_t m = half_mask(__ballot(need), s.half);
    const uint32_t below = m & ((1u << s.l) - 1u);
    uint32_t w = 0;
    if (need) {
        const uint32_t idx = s.pos + __popc(below);
        if (idx < s.nwords) w = s.words[idx];
        else s.err |= kErrWords;
    }
    s.pos += __popc(m);
    return w;
}

__device__ inline void refill(Lane& s) {
    const bool need = s.valid && s.x < kLow;
    const uint32_t w = take_words(s, need);
    if (need) s.x = (s.x << 16) | w;
}

__device__ inline void begin_tile(const DecodeParams& p, int64_t tile, Lane& s) {
    if (s.valid) {
        const uint32_t a = p.index[tile], b = p.index[tile + 1];
        const uint32_t* t = p.payload + a;
        s.x = t[s.l];
        s.words = reinterpret_cast<const uint16_t*>(t + 32);
        s.nwords = 2 * (b - a - 32);
    } else {
        s.x = kLow;
        s.words = nullptr;
        s.nwords = 0;
    }
    s.pos = 0;
}

__device__ inline void end_tile(Lane& s) {
    if (!s.valid) return;
    if (s.x != kLow) s.err |= kErrState;
    // all words consumed, except possibly the one zero pad word
    if (!(s.pos == s.nwords || (s.pos + 1 == s.nwords && s.words[s.pos] == 0))) s.err |= kErrWords;
}

// ----------------------------------------------------------------------------- stores
template <int CT>
struct Store;

template <>
struct Store<CT_BF16> {
    using T = uint16_t;
    __device__ static uint32_t conv(int32_t q, float alpha, float, uint32_t) { return bf16_rne((float)q * alpha); }
};
template <>
struct Store<CT_F16> {
    using T = uint16_t;
    __device__ static uint32_t conv(int32_t q, float alpha, float, uint32_t) { return f16_rne((float)q * alpha); }
};
template <>
struct Store<CT_F8E4M3> {
    using T = uint8_t;
    __device__ static uint32_t conv(int32_t q, float, float h, uint32_t) { return e4m3_rne_sat((float)q * h); }
};
template <>
struct Store<CT_I8> {
    using T = uint8_t;
    // round-half-away(q / k): floor((2|q| + k) / 2k) by a multiply with ceil(2^32 / 2k), exact
    // because (2|q| + k) * 2k < 2^32.
    __device__ static uint32_t conv(int32_t q, float, float, uint32_t kk) {
        const uint32_t k = kk & 0xFFFFu, a = (uint32_t)(q < 0 ? -q : q);
        const uint32_t D = 2u * k;
        const uint32_t m = 0xFFFFFFFFu / D + 1u;
        const uint32_t v = __umulhi(2u * a + k, m);
        return (uint32_t)(uint8_t)(int8_t)(q < 0 ? -(int32_t)v : (int32_t)v);
    }
};
template <>
struct Store<CT_Q16> {
    using T = uint16_t;
    __device__ static uint32_t conv(int32_t q, float, float, uint32_t) { return (uint32_t)(uint16_t)(int16_t)q; }
};

template <int CT>
__device__ inline void store_block(const DecodeParams& p, int64_t row, int64_t col0, const int32_t* q, float alpha,
                                   float h, uint32_t k) {
    using T = typename Store<CT>::T;
    T* out = static_cast<T*>(p.out) + row * p.cols;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = Store<CT>::conv(q[j], alpha, h, k);
    if (col0 + 8 <= p.cols && (p.cols & 7) == 0) {
        if constexpr (sizeof(T) == 2) {
            uint4 pk = make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
            *reinterpret_cast<uint4*>(out + col0) = pk;
        } else {
            uint2 pk = make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24, v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
            *reinterpret_cast<uint2*>(out + col0) = pk;
        }
    } else {
        for (int j = 0; j < 8; ++j)
            if (col0 + j < p.cols) out[col0 + j] = (T)v[j];
    }
}

// ----------------------------------------------------------------------------- lossy kernel
template <int CT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_lossy_kernel(DecodeParams p) {
    extern __shared__ __align__(16) uint8_t smem[];
    Lds L;
    stage_tables(p, smem, &L);
    const int n = p.prob_bits;
    const float h = p.step * 0.5f;
    Lane s;
    s.half = (threadIdx.x >> 5) & 1;
    s.l = threadIdx.x & 31;
    s.err = 0;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t wstride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t pair = wave0; pair < p.n_pairs; pair += wstride) {
        const int64_t tr = pair / p.pairs_c;
        const int64_t tc = 2 * (pair % p.pairs_c) + s.half;
        s.valid = tc < p.tiles_c;
        begin_tile(p, tr * p.tiles_c + tc, s);
        for (int rr = 0; rr < p.tile_rows; ++rr) {
            uint32_t sy;
            const uint64_t e0 = rans_step(s, L, 0, n, &sy);
            refill(s);
            const int b = (int)(e0 >> 32);
            int32_t q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t e = rans_step(s, L, 1 + 2 * j + b, n, &sy);
                q[j] = (int32_t)(e >> 32);
                refill(s);
                const bool esc = s.valid && sy == 255u;
                if (__ballot(esc)) {
                    const uint32_t w = take_words(s, esc);
                    if (esc) q[j] = 2 * (int32_t)(int16_t)w + b;
                }
            }
            const int64_t row = tr * p.tile_rows + rr;
            if (row < p.rows && s.valid) {
                const float sc = p.row_scale[row];
                const float alpha = h * sc;
                uint32_t k = 1;
                if constexpr (CT == CT_I8) {
                    const uint32_t qm = p.row_qmax[row];
                    k = qm > 127u ? (qm + 126u) / 127u : 1u;
                }
                const int64_t col0 = tc * 256 + 8 * s.l;
                if (col0 < p.cols) store_block<CT>(p, row, col0, q, alpha, h, k);
                if constexpr (CT == CT_F8E4M3 || CT == CT_I8) {
                    if (tc == 0 && s.l == 0) p.scale_out[row] = CT == CT_F8E4M3 ? sc : alpha * (float)k;
                }
            }
        }
        end_tile(s);
    }
    if (s.err) atomicOr(p.err, s.err);
}

// ----------------------------------------------------------------------------- lossless kernel
template <int P>
__global__ __launch_bounds__(64 * kWavesPerBlock) void decode_lossless_kernel(DecodeParams p) {
    extern __shared__ __align__(16) uint8_t smem[];
    Lds L;
    stage_tables(p, smem, &L);
    const int n = p.prob_bits;
    Lane s;
    s.half = (threadIdx.x >> 5) & 1;
    s.l = threadIdx.x & 31;
    s.err = 0;
    const int64_t wave0 = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t wstride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t pair = wave0; pair < p.n_pairs; pair += wstride) {
        const int64_t tr = pair / p.pairs_c;
        const int64_t tc = 2 * (pair % p.pairs_c) + s.half;
        s.valid = tc < p.tiles_c;
        begin_tile(p, tr * p.tiles_c + tc, s);
        for (int rr = 0; rr < p.tile_rows; ++rr) {
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t acc = 0;
#pragma unroll
                for (int pl = 0; pl < P; ++pl) {
                    uint32_t sy;
                    rans_step(s, L, pl, n, &sy);
                    refill(s);
                    acc = acc << 8 | sy;
                }
                v[e] = acc;
            }
            const int64_t row = tr * p.tile_rows + rr;
            const int64_t col0 = tc * 256 + 8 * s.l;
            if (row < p.rows && s.valid && col0 < p.cols) {
                if constexpr (P == 2) {
                    uint16_t* out = static_cast<uint16_t*>(p.out) + row * p.cols;
                    if (col0 + 8 <= p.cols && (p.cols & 7) == 0)
                        *reinterpret_cast<uint4*>(out + col0) =
                            make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
                    else
                        for (int j = 0; j < 8; ++j)
                            if (col0 + j < p.cols) out[col0 + j] = (uint16_t)v[j];
                } else if constexpr (P == 1) {
                    uint8_t* out = static_cast<uint8_t*>(p.out) + row * p.cols;
                    if (col0 + 8 <= p.cols && (p.cols & 7) == 0)
                        *reinterpret_cast<uint2*>(out + col0) =
                            make_uint2(v[0] | v[1] << 8 | v[2] << 16 | v[3] << 24, v[4] | v[5] << 8 | v[6] << 16 | v[7] << 24);
                    else
                        for (int j = 0; j < 8; ++j)
                            if (col0 + j < p.cols) out[col0 + j] = (uint8_t)v[j];
                } else {
                    uint32_t* out = static_cast<uint32_t*>(p.out) + row * p.cols;
                    if (col0 + 8 <= p.cols && (p.cols & 7) == 0) {
                        *reinterpret_cast<uint4*>(out + col0) = make_uint4(v[0], v[1], v[2], v[3]);
                        *reinterpret_cast<uint4*>(out + col0 + 4) = make_uint4(v[4], v[5], v[6], v[7]);
                    } else {
                        for (int j = 0; j < 8; ++j)
                            if (col0 + j < p.cols) out[col0 + j] = v[j];
                    }
                }
            }
        }
        end_tile(s);
    }
    if (s.err) atomicOr(p.err, s.err);
}

int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int v = 0;
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        cache[dev] = v > 0 ? v : 256;
    }
    return cache[dev];
}

// Allow a kernel the full 160 KiB of LDS once.
hipError_t allow_lds(const void* kernel) {
    static std::mutex mu;
    static std::set<const void*> done;
    std::lock_guard<std::mutex> g(mu);
    if (done.count(kernel)) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess) done.insert(kernel);
    return e;
}

template <class K>
hipError_t launch(K kernel, const DecodeParams& p, hipStream_t stream) {
    const size_t lds = table_blob_bytes(p.n_tables, p.prob_bits);
    hipError_t e = allow_lds(reinterpret_cast<const void*>(kernel));
    if (e != hipSuccess) return e;
    const int per_cu = std::max<int>(1, std::min<int>(2, (int)((160 * 1024) / lds)));
    int64_t blocks = (p.n_pairs + kWavesPerBlock - 1) / kWavesPerBlock;
    blocks = std::min<int64_t>(blocks, (int64_t)device_cus() * per_cu);
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int container, hipStream_t stream) {
    if (p.n_pairs == 0) return hipSuccess;
    if (p.mode == 0) {
        switch (container) {
            case CT_BF16: return launch(decode_lossy_kernel<CT_BF16>, p, stream);
            case CT_F16: return launch(decode_lossy_kernel<CT_F16>, p, stream);
            case CT_F8E4M3: return launch(decode_lossy_kernel<CT_F8E4M3>, p, stream);
            case CT_I8: return launch(decode_lossy_kernel<CT_I8>, p, stream);
            case CT_Q16: return launch(decode_lossy_kernel<CT_Q16>, p, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.n_tables) {
        case 1: return launch(decode_lossless_kernel<1>, p, stream);
        case 2: return launch(decode_lossless_kernel<2>, p, stream);
        case 4: return launch(decode_lossless_kernel<4>, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ep
