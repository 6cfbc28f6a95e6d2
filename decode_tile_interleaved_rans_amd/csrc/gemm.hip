// gfx950 BF16 GEMM for the compressed linear layer: Y[M][N] = X[M][K] W[N][K]^T (+ bias), fp32
// accumulation on the matrix cores (v_mfma_f32_32x32x16_bf16), BF16 output.
//
// Tiling. A block of 4 waves owns a 128 x 128 tile of Y and walks K in steps of 64: both operand
// tiles (128 rows x 64 K of X and of W, K contiguous, as the MFMA wants 8 consecutive K per lane)
// are staged in LDS with a 16-byte row pad against bank conflicts, double-buffered, the next K
// step being fetched into registers while the current one feeds the MFMAs. Each wave computes
// 64 x 64 as 2 x 2 MFMA tiles of 32 x 32, reusing every A and B fragment twice. Operand lane
// layout of the 32x32x16 BF16 MFMA (checked on the device): lane l supplies A[l % 32][8 (l / 32)
// + i] and B[8 (l / 32) + i][l % 32], i < 8, and receives C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32]
// for i < 16.
//
// The compressed linear forward (capi.cpp) decodes the weight slice by slice into a scratch
// buffer small enough to stay in the Infinity Cache and runs this GEMM on each slice: every
// weight is decoded once per forward, which the large-M (prefill) case needs, since decoding per
// output tile would repeat it M / 128 times.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm.h"

namespace ep {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int kPad = 8;                      // bf16 elements of padding per LDS row
constexpr int kLd = BK + kPad;               // LDS row stride in elements (144 bytes)
constexpr int kThreads = 256;

template <int ROWS>
struct Frag {
    uint4 v[ROWS / 32];                      // ROWS x 64 bf16 = ROWS * 8 chunks of 16 bytes over 256 threads
};

// Fetch a ROWS x 64 operand tile (rows r0.., K k0..) into registers: thread t takes 16-byte
// chunks t, t + 256, ... (row = chunk / 8, K chunk = chunk % 8); rows past `rows` and chunks
// past K read as zero.
template <int ROWS>
__device__ __forceinline__ void fetch(const uint16_t* src, int ld, int r0, int rows, int k0, int K, Frag<ROWS>& f) {
#pragma unroll
    for (int j = 0; j < ROWS / 32; ++j) {
        const int c = threadIdx.x + kThreads * j;
        const int r = r0 + (c >> 3), k = k0 + 8 * (c & 7);
        // K % 8 == 0, so a chunk is either wholly inside K or wholly past it
        f.v[j] = (r < rows && k < K) ? *reinterpret_cast<const uint4*>(src + (size_t)r * ld + k) : make_uint4(0, 0, 0, 0);
    }
}

template <int ROWS>
__device__ __forceinline__ void stash(const Frag<ROWS>& f, uint16_t* lds) {
#pragma unroll
    for (int j = 0; j < ROWS / 32; ++j) {
        const int c = threadIdx.x + kThreads * j;
        *reinterpret_cast<uint4*>(lds + (c >> 3) * kLd + 8 * (c & 7)) = f.v[j];
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// BM x BN output tile per block of 4 waves (2 x 2), each wave (BM / 2) x (BN / 2) as
// (BM / 64) x (BN / 64) MFMA tiles of 32 x 32.
template <int BM, int BN, bool BIAS>
__global__ __launch_bounds__(kThreads) void gemm_nt(GemmArgs g) {
    constexpr int TI = BM / 64, TJ = BN / 64;
    __shared__ __align__(16) uint16_t As[2][BM * kLd];
    __shared__ __align__(16) uint16_t Bs[2][BN * kLd];
    // XCD-aware order: consecutive block ids go to different XCDs, so give each XCD a compact
    // band of N tiles (W slices then stay in that XCD's L2)
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int nblk = tiles_m * tiles_n;
    int b = blockIdx.x;
    if (nblk % 8 == 0) b = (b % 8) * (nblk / 8) + b / 8;
    const int tm = b % tiles_m, tn = b / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    Frag<BM> fa;
    Frag<BN> fb;
    fetch<BM>(g.X, g.ldx, m0, g.M, 0, g.K, fa);
    fetch<BN>(g.W, g.ldw, n0, g.N, 0, g.K, fb);
    stash<BM>(fa, As[0]);
    stash<BN>(fb, Bs[0]);
    __syncthreads();
    const int nk = (g.K + BK - 1) / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            fetch<BM>(g.X, g.ldx, m0, g.M, (kt + 1) * BK, g.K, fa);
            fetch<BN>(g.W, g.ldw, n0, g.N, (kt + 1) * BK, g.K, fb);
        }
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8 a[TI], bb[TJ];
            const int kk = ks + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < TI; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm + 32 * i + (lane & 31)) * kLd + kk]);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bb[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn + 32 * j + (lane & 31)) * kLd + kk]);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            stash<BM>(fa, As[cur ^ 1]);
            stash<BN>(fb, Bs[cur ^ 1]);
        }
        __syncthreads();
    }

    // epilogue: C[8 (r / 4) + 4 (lane / 32) + r % 4][lane % 32] of each 32 x 32 tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn + 32 * j + (lane & 31);
            if (col >= g.N) continue;
            float bv = 0.0f;
            if constexpr (BIAS) bv = __uint_as_float((uint32_t)g.bias[col] << 16);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const uint32_t pk = pack_bf16x2(acc[i][j][r] + bv, acc[i][j][r + 1] + bv);
                if (row < g.M) g.Y[(size_t)row * g.ldy + col] = (uint16_t)(pk & 0xFFFFu);
                if (row + 1 < g.M) g.Y[(size_t)(row + 1) * g.ldy + col] = (uint16_t)(pk >> 16);
            }
        }
}

// Skinny GEMM for M <= 64 (a few tokens): W is streamed once from HBM straight into MFMA
// registers, no LDS staging. A block owns 16 output columns; its 8 waves split K (wave w takes
// the 64-wide K chunks w, w + 8, ..., four chunks per iteration with all loads issued first),
// each computing MT 16 x 16 tiles of Y with the 16x16x32 BF16 MFMA (lane l supplies
// A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16], i < 8, and receives
// C[4 (l / 16) + i][l % 16], i < 4); the partial sums meet in LDS. Operands come through buffer
// resources bounded to the block's rows, so rows past N or M and K past the end read as zero.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 4;
constexpr uint32_t kOob = 0x80000000u;      // an offset past every resource: the load returns 0

template <int MT, bool BIAS>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny(GemmArgs g) {
    __shared__ float red[kSkinnyWaves][MT][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, kq = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nrows = g.N - n0 < 16 ? g.N - n0 : 16;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(g.W + (size_t)n0 * g.ldw), 0, (int)((size_t)nrows * g.ldw * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(g.X), 0, (int)((size_t)g.M * g.ldx * 2), 0x00020000);
    const uint32_t woff = (uint32_t)r * g.ldw * 2;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{};
    const int nkc = (g.K + 63) / 64;
    for (int kb = wave; kb < nkc; kb += kSkinnyWaves * kSkinnyUnroll) {
        uint4 bw[kSkinnyUnroll][2], ax[kSkinnyUnroll][MT][2];
#pragma unroll
        for (int u = 0; u < kSkinnyUnroll; ++u) {
            const int kc = kb + u * kSkinnyWaves;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = kc * 64 + 32 * h + 8 * kq;
                const bool in = kc < nkc && k < g.K;
                bw[u][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, in ? woff + 2u * k : kOob, 0, 0));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t xo = (uint32_t)(mt * 16 + r) * g.ldx * 2 + 2u * k;
                    ax[u][mt][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xo : kOob, 0, 0));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kSkinnyUnroll; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ax[u][mt][h]),
                                                                      __builtin_bit_cast(bf16x8, bw[u][h]), acc[mt], 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][mt][(4 * kq + i) * 16 + r] = acc[mt][i];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * 256; e += 64 * kSkinnyWaves) {
        const int mt = e >> 8, row = (e >> 4) & 15, col = e & 15;
        const int m = mt * 16 + row, nn = n0 + col;
        if (m >= g.M || nn >= g.N) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kSkinnyWaves; ++w) v += red[w][mt][e & 255];
        if constexpr (BIAS) v += __uint_as_float((uint32_t)g.bias[nn] << 16);
        g.Y[(size_t)m * g.ldy + nn] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

int gemm_device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
        cache[dev] = v > 0 ? v : 256;
    }
    return cache[dev];
}

template <int BM, int BN>
hipError_t launch_tiled(const GemmArgs& g, hipStream_t stream) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (g.bias)
        hipLaunchKernelGGL((gemm_nt<BM, BN, true>), dim3(tiles), dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_nt<BM, BN, false>), dim3(tiles), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_skinny(const GemmArgs& g, hipStream_t stream) {
    const int blocks = (g.N + 15) / 16;
    if (g.bias)
        hipLaunchKernelGGL((gemm_skinny<MT, true>), dim3(blocks), dim3(64 * kSkinnyWaves), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_skinny<MT, false>), dim3(blocks), dim3(64 * kSkinnyWaves), 0, stream, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    // tile choice: the skinny kernel for a few rows of X; 128 x 128 tiles when they give every CU
    // at least two blocks, else 64 x 64 tiles
    if (g.M <= 16) return launch_skinny<1>(g, stream);
    if (g.M <= 32) return launch_skinny<2>(g, stream);
    if (g.M <= 64) return launch_skinny<4>(g, stream);
    const long tiles128 = (long)((g.M + 127) / 128) * ((g.N + 127) / 128);
    if (tiles128 >= 2L * gemm_device_cus()) return launch_tiled<128, 128>(g, stream);
    return launch_tiled<64, 64>(g, stream);
}

}  // namespace ep
