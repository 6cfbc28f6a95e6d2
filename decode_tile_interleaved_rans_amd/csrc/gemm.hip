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

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kPad = 8;                      // bf16 elements of padding per LDS row
constexpr int kLd = BK + kPad;               // LDS row stride in elements (144 bytes)
constexpr int kThreads = 256;

struct Frag {
    uint4 v[4];                              // 4 x 16 bytes of one operand tile per thread
};

// Fetch a 128 x 64 operand tile (rows r0.., K k0..) into registers: thread t takes 16-byte
// chunks t, t + 256, t + 512, t + 768 (row = chunk / 8, K chunk = chunk % 8); rows past `rows`
// and chunks past K read as zero.
__device__ __forceinline__ void fetch(const uint16_t* src, int ld, int r0, int rows, int k0, int K, Frag& f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = threadIdx.x + kThreads * j;
        const int r = r0 + (c >> 3), k = k0 + 8 * (c & 7);
        // K % 8 == 0, so a chunk is either wholly inside K or wholly past it
        f.v[j] = (r < rows && k < K) ? *reinterpret_cast<const uint4*>(src + (size_t)r * ld + k) : make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void stash(const Frag& f, uint16_t* lds) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = threadIdx.x + kThreads * j;
        *reinterpret_cast<uint4*>(lds + (c >> 3) * kLd + 8 * (c & 7)) = f.v[j];
    }
}

template <bool BIAS>
__global__ __launch_bounds__(kThreads) void gemm_nt(GemmArgs g) {
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
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    Frag fa, fb;
    fetch(g.X, g.ldx, m0, g.M, 0, g.K, fa);
    fetch(g.W, g.ldw, n0, g.N, 0, g.K, fb);
    stash(fa, As[0]);
    stash(fb, Bs[0]);
    __syncthreads();
    const int nk = (g.K + BK - 1) / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            fetch(g.X, g.ldx, m0, g.M, (kt + 1) * BK, g.K, fa);
            fetch(g.W, g.ldw, n0, g.N, (kt + 1) * BK, g.K, fb);
        }
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8 a[2], bb[2];
            const int kk = ks + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm + 32 * i + (lane & 31)) * kLd + kk]);
                bb[i] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn + 32 * i + (lane & 31)) * kLd + kk]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            stash(fa, As[cur ^ 1]);
            stash(fb, Bs[cur ^ 1]);
        }
        __syncthreads();
    }

    // epilogue: C[8 (r / 4) + 4 (lane / 32) + r % 4][lane % 32] of each 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 32 * j + (lane & 31);
            if (col >= g.N) continue;
            float bv = 0.0f;
            if constexpr (BIAS) bv = __uint_as_float((uint32_t)g.bias[col] << 16);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                f32x2 v = {acc[i][j][r] + bv, acc[i][j][r + 1] + bv};
                const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
                if (row < g.M) g.Y[(size_t)row * g.ldy + col] = (uint16_t)(pk & 0xFFFFu);
                if (row + 1 < g.M) g.Y[(size_t)(row + 1) * g.ldy + col] = (uint16_t)(pk >> 16);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (g.bias)
        hipLaunchKernelGGL(gemm_nt<true>, dim3(tiles), dim3(kThreads), 0, stream, g);
    else
        hipLaunchKernelGGL(gemm_nt<false>, dim3(tiles), dim3(kThreads), 0, stream, g);
    return hipGetLastError();
}

}  // namespace ep
