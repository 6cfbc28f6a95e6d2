// gfx950 BF16 GEMM for the compressed linear layer: Y[M][N] = X[M][K] W[N][K]^T (+ bias), fp32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16 and v_mfma_f32_32x32x16_bf16), BF16
// output.
//
// Tiled kernels. A block of WGM x WGN waves owns a BM x BN tile of Y and walks K in steps of 64:
// both operand tiles (rows x 64 K of X and of W, K contiguous, as the MFMA wants 8 consecutive K
// per lane) are staged in LDS, double-buffered; global loads go through buffer resources (rows
// past the matrix and K past the end read as zero). Each wave computes its (BM / WGM) x
// (BN / WGN) part as MFMA tiles. 256 x 256 tiles with 8 waves of 128 x 64 (gemm_dma, 16 x 16 MFMA
// tiles: 4% faster than 32 x 32 ones, and 8 waves 2% faster than 16 of 64 x 64, with the same bits
// out) load straight from global memory into LDS;
// 128 x 128 and 64 x 64 tiles with 4 waves (gemm_nt, 32 x 32 MFMA tiles) go through two register
// stages and a padded LDS layout. Tile choice (launch_gemm): 256 x 256 when every CU
// gets a block, 128 x 128 when every CU gets two, else 64 x 64; the skinny kernel streams W
// straight into registers for M <= 64. Block order: consecutive block ids land on
// different XCDs, so each XCD gets a contiguous range of tiles, walked in groups of 4 M tiles so
// that the blocks running together share X and W slices in that XCD's L2. Operand lane layouts
// (checked on the device): 32x32x16 BF16 MFMA, lane l supplies A[l % 32][8 (l / 32) + i] and
// B[8 (l / 32) + i][l % 32], i < 8, and receives C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32] for
// i < 16; 16x16x32 BF16 MFMA, lane l supplies A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16],
// i < 8, and receives C[4 (l / 16) + i][l % 16] for i < 4.
//
// The compressed linear forward (capi.cpp) decodes the weight slice by slice into a scratch
// buffer small enough to stay in the Infinity Cache and runs this GEMM on each slice: every
// weight is decoded once per forward, which the large-M (prefill) case needs, since decoding per
// output tile would repeat it M / 128 times.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm.h"
#include "kernels.h"

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
constexpr int kPrefetch = 2;                 // register stages of the tiled kernels (see gemm_nt)
constexpr int kGroupM = 4;                   // M tiles per group in the block order (see gemm_nt)

template <int ROWS, int NT>
struct Frag {
    uint4 v[ROWS * 8 / NT];                  // ROWS x 64 bf16 = ROWS * 8 chunks of 16 bytes over NT threads
};

// Operand rows [r0, r0 + ROWS) of a row-major bf16 matrix as a buffer resource: rows past `rows`
// lie past the resource's end and read as zero.
template <int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint16_t* src, int ld, int r0, int rows) {
    const int n = rows - r0 < ROWS ? rows - r0 : ROWS;
    // readfirstlane: the size is block-uniform; without it the backend may build it in VGPRs and
    // wrap every load in a loop over distinct resources
    const int bytes = __builtin_amdgcn_readfirstlane((int)((size_t)(n > 0 ? n : 0) * ld * 2));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src + (size_t)r0 * ld), 0, bytes, 0x00020000);
}

constexpr uint32_t kOob = 0x80000000u;      // an offset past every resource: the load returns 0

// Fetch a ROWS x 64 operand tile (K k0..) into registers: thread t of NT takes 16-byte chunks t,
// t + NT, ... (row = chunk / 8, K chunk = chunk % 8); rows past the resource and chunks past K
// read as zero (K % 8 == 0, so a chunk is either wholly inside K or wholly past it).
template <int ROWS, int NT>
__device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int ld, int k0, int K, Frag<ROWS, NT>& f) {
#pragma unroll
    for (int j = 0; j < ROWS * 8 / NT; ++j) {
        const int c = threadIdx.x + NT * j;
        const int r = c >> 3, k = k0 + 8 * (c & 7);
        // k >= K moves the offset past the resource; arithmetic rather than a select, which the
        // backend would turn into a branch around the load
        const uint32_t off = (uint32_t)(r * ld + k) * 2u | ((uint32_t)((K - 1 - k) >> 31) & kOob);
        f.v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
}

template <int ROWS, int NT>
__device__ __forceinline__ void stash(const Frag<ROWS, NT>& f, uint16_t* lds) {
#pragma unroll
    for (int j = 0; j < ROWS * 8 / NT; ++j) {
        const int c = threadIdx.x + NT * j;
        *reinterpret_cast<uint4*>(lds + (c >> 3) * kLd + 8 * (c & 7)) = f.v[j];
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// BM x BN output tile per block of WGM x WGN waves, each wave (BM / WGM) x (BN / WGN) as
// TI x TJ MFMA tiles of 32 x 32.
template <int BM, int BN, int WGM, int WGN, int PF, bool BIAS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_nt(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int TI = BM / WGM / 32, TJ = BN / WGN / 32;
    __shared__ __align__(16) uint16_t As[2][BM * kLd];
    __shared__ __align__(16) uint16_t Bs[2][BN * kLd];
    // XCD-aware order: consecutive block ids go to different XCDs, so give each XCD a compact
    // band of N tiles (W slices then stay in that XCD's L2)
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int nblk = tiles_m * tiles_n;
    int b = blockIdx.x;
    if (nblk % 8 == 0) b = (b % 8) * (nblk / 8) + b / 8;
    // then groups of kGroupM M tiles: the blocks that run together share both X and W slices
    constexpr int G = kGroupM;
    const int per_group = G * tiles_n, first_m = (b / per_group) * G;
    const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
    const int tm = first_m + (b % per_group) % gsize, tn = (b % per_group) / gsize;
    // block-uniform (kept in SGPRs, so the operand resources below are scalar)
    const int m0 = __builtin_amdgcn_readfirstlane(tm * BM), n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    const __amdgpu_buffer_rsrc_t rx = operand_rsrc<BM>(g.X, g.ldx, m0, g.M);
    const __amdgpu_buffer_rsrc_t rw = operand_rsrc<BN>(g.W, g.ldw, n0, g.N);
    // PF register stages: step kt + PF is fetched while step kt is multiplied out of LDS, and
    // step kt + 1 (fetched PF - 1 steps ago) is stored into the other LDS buffer behind it.
    // Fetches past K read zeros, so the loop needs no tail guards on them.
    Frag<BM, NT> fa[PF];
    Frag<BN, NT> fb[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        fetch<BM, NT>(rx, g.ldx, p * BK, g.K, fa[p]);
        fetch<BN, NT>(rw, g.ldw, p * BK, g.K, fb[p]);
    }
    stash<BM, NT>(fa[0], As[0]);
    stash<BN, NT>(fb[0], Bs[0]);
    __syncthreads();
    const int nk = (g.K + BK - 1) / BK;
    for (int kt0 = 0; kt0 < nk; kt0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int kt = kt0 + u;
            if (kt >= nk) break;
            const int cur = kt & 1;
            fetch<BM, NT>(rx, g.ldx, (kt + PF) * BK, g.K, fa[u]);
            fetch<BN, NT>(rw, g.ldw, (kt + PF) * BK, g.K, fb[u]);
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
                stash<BM, NT>(fa[(u + 1) % PF], As[cur ^ 1]);
                stash<BN, NT>(fb[(u + 1) % PF], Bs[cur ^ 1]);
            }
            __syncthreads();
        }
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

// Tiled kernel with direct global -> LDS loads (buffer_load ... lds): a wave's load instruction
// writes its 64 lanes' 16 bytes to 1 KiB of LDS in lane order, 8 operand rows of 128 bytes, so no
// registers stage the tiles. Rows are unpadded and their eight 16-byte K chunks swizzled: chunk c
// of row r sits at slot c ^ ((r / 2) % 8). A fragment read has 16 lanes on 16 consecutive rows at
// the same chunk in each LDS cycle; with 128-byte rows the 16-byte bank group of (r, slot) is
// 8 (r % 2) + slot of 16, so the slots of the even rows and of the odd rows must each be distinct,
// which (r / 2) % 8 gives (the plain r % 8 put rows r and r + 8 on one bank group: counters showed
// half of the LDS cycles lost to conflicts). Two LDS stages: the loads of step k + 1 run while
// step k multiplies.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int chunk_swizzle(int r) { return (r >> 1) & 7; }

template <int ROWS, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int ld, int k0, int K, uint8_t* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rr = lane >> 3;                                 // row within the 8-row group
#pragma unroll
    for (int j = 0; j < ROWS / 8 / NW; ++j) {
        const int g = wave + NW * j;                          // 8-row group of this instruction
        const int k = k0 + 8 * ((lane & 7) ^ chunk_swizzle(8 * g + rr));   // the chunk for this slot
        const uint32_t off = (uint32_t)((8 * g + rr) * ld + k) * 2u | ((uint32_t)((K - 1 - k) >> 31) & kOob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 1024 * g), 16, off, 0, 0, 0);
    }
}

// SPLIT: blockIdx.y is the split index; the block multiplies K columns [split * g.kc, + g.kc) and
// writes its fp32 partial tile to g.part[split][M][N] (gemm_split_sum adds the splits in order).
template <int BM, int BN, int WGM, int WGN, bool BIAS, bool SPLIT = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_dma(GemmArgs g) {
    constexpr int NW = WGM * WGN;
    constexpr int TI = BM / WGM / 16, TJ = BN / WGN / 16;     // 16 x 16 MFMA tiles per wave
    constexpr int kStage = (BM + BN) * 128;                   // bytes of one LDS stage
    __shared__ __align__(1024) uint8_t lds[2 * kStage];
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int nblk = tiles_m * tiles_n;
    int b = blockIdx.x;
    if (nblk % 8 == 0) b = (b % 8) * (nblk / 8) + b / 8;
    constexpr int G = kGroupM;
    const int per_group = G * tiles_n, first_m = (b / per_group) * G;
    const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
    const int tm = first_m + (b % per_group) % gsize, tn = (b % per_group) / gsize;
    const int m0 = __builtin_amdgcn_readfirstlane(tm * BM), n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);
    const __amdgpu_buffer_rsrc_t rx = operand_rsrc<BM>(g.X, g.ldx, m0, g.M);
    const __amdgpu_buffer_rsrc_t rw = operand_rsrc<BN>(g.W, g.ldw, n0, g.N);

    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{};

    // K range of this block: all of K, or the split's g.kc columns (a multiple of BK)
    const int kb = SPLIT ? (int)blockIdx.y * g.kc : 0;
    const int ke = SPLIT ? (kb + g.kc < g.K ? kb + g.kc : g.K) : g.K;
    dma_tile<BM, NW>(rx, g.ldx, kb, g.K, lds);
    dma_tile<BN, NW>(rw, g.ldw, kb, g.K, lds + BM * 128);
    __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0): this wave's tile loads landed
    __syncthreads();
    const int nk = (ke - kb + BK - 1) / BK;
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t* cur = lds + (kt & 1) * kStage;
        if (kt + 1 < nk) {
            uint8_t* nxt = lds + ((kt + 1) & 1) * kStage;
            dma_tile<BM, NW>(rx, g.ldx, kb + (kt + 1) * BK, g.K, nxt);
            dma_tile<BN, NW>(rw, g.ldw, kb + (kt + 1) * BK, g.K, nxt + BM * 128);
        }
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8 a[TI], bb[TJ];
            const int kc = ks / 8 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int r = wm + 16 * i + (lane & 15);
                a[i] = *reinterpret_cast<const bf16x8*>(cur + r * 128 + ((kc ^ chunk_swizzle(r)) << 4));
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int r = wn + 16 * j + (lane & 15);
                bb[j] = *reinterpret_cast<const bf16x8*>(cur + BM * 128 + r * 128 + ((kc ^ chunk_swizzle(r)) << 4));
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): the next stage's loads landed
        __syncthreads();                                     // ... for every wave; this stage is free
    }

    // C[4 (lane / 16) + r][lane % 16] of each 16 x 16 tile
    if constexpr (SPLIT) {
        float* part = g.part + (size_t)blockIdx.y * g.M * g.N;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int col = n0 + wn + 16 * j + (lane & 15);
                if (col >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                    if (row < g.M) part[(size_t)row * g.N + col] = acc[i][j][r];
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn + 16 * j + (lane & 15);
            if (col >= g.N) continue;
            float bv = 0.0f;
            if constexpr (BIAS) bv = __uint_as_float((uint32_t)g.bias[col] << 16);
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                const uint32_t pk = pack_bf16x2(acc[i][j][r] + bv, acc[i][j][r + 1] + bv);
                if (row < g.M) g.Y[(size_t)row * g.ldy + col] = (uint16_t)(pk & 0xFFFFu);
                if (row + 1 < g.M) g.Y[(size_t)(row + 1) * g.ldy + col] = (uint16_t)(pk >> 16);
            }
        }
}

// Y [M][N] = sum over the splits of part[split][M][N] in split order (+ bias), BF16.
__global__ __launch_bounds__(256) void gemm_split_sum(const float* part, int splits, const uint16_t* bias, uint16_t* Y,
                                                      int M, int N, int ldy) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)M * N) return;
    const int64_t plane = (int64_t)M * N;
    float v = part[e];
    for (int s = 1; s < splits; ++s) v += part[s * plane + e];
    const int col = (int)(e % N), row = (int)(e / N);
    if (bias) v += __uint_as_float((uint32_t)bias[col] << 16);
    Y[(size_t)row * ldy + col] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_dma(const GemmArgs& g, hipStream_t stream) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (g.bias)
        hipLaunchKernelGGL((gemm_dma<BM, BN, WGM, WGN, true>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_dma<BM, BN, WGM, WGN, false>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
    return hipGetLastError();
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

// ----------------------------------------------------------------------------- FP8 (E4M3) GEMM
// Same tiling as gemm_dma with one-byte elements: a K step is 128 E4M3 codes, i.e. the same
// 128-byte LDS rows and 16-byte swizzled chunks, multiplied by two 32x32x64 FP8 MFMAs
// (v_mfma_f32_32x32x64_f8f6f4, both operands in the E4M3 format). Lane l supplies A row l % 32
// and B column l % 32 with 32 codes each; lanes l and l + 32 cover complementary K halves. A lane
// takes the 16-byte chunks 4j + l / 32 and 4j + 2 + l / 32 of the row for MFMA j: A and B use
// the same rule, so every product pairs equal k whatever order the unit sums them in. The
// accumulator layout is that of every 32 x 32 MFMA (see above); the epilogue applies the row
// scale of X and the row scale of W.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc_u8(const uint8_t* src, int ld, int r0, int rows) {
    const int n = rows - r0 < ROWS ? rows - r0 : ROWS;
    const int bytes = __builtin_amdgcn_readfirstlane((int)((size_t)(n > 0 ? n : 0) * ld));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src + (size_t)r0 * ld), 0, bytes, 0x00020000);
}

template <int ROWS, int NW>
__device__ __forceinline__ void dma_tile_u8(__amdgpu_buffer_rsrc_t rs, int ld, int k0, int K, uint8_t* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rr = lane >> 3;
#pragma unroll
    for (int j = 0; j < ROWS / 8 / NW; ++j) {
        const int g = wave + NW * j;
        const int k = k0 + 16 * ((lane & 7) ^ chunk_swizzle(8 * g + rr));
        const uint32_t off = (uint32_t)((8 * g + rr) * ld + k) | ((uint32_t)((K - 1 - k) >> 31) & kOob);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + 1024 * g), 16, off, 0, 0, 0);
    }
}

__device__ __forceinline__ i32x8 frag_f8(const uint8_t* row, int r, int c0) {
    const uint4 lo = *reinterpret_cast<const uint4*>(row + ((c0 ^ chunk_swizzle(r)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (((c0 + 2) ^ chunk_swizzle(r)) << 4));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int BM, int BN, int WGM, int WGN, bool BIAS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f8(GemmF8Args g) {
    constexpr int NW = WGM * WGN;
    constexpr int TI = BM / WGM / 32, TJ = BN / WGN / 32;
    constexpr int BK8 = 128;
    constexpr int kStage = (BM + BN) * 128;
    __shared__ __align__(1024) uint8_t lds[2 * kStage];
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int nblk = tiles_m * tiles_n;
    int b = blockIdx.x;
    if (nblk % 8 == 0) b = (b % 8) * (nblk / 8) + b / 8;
    constexpr int G = kGroupM;
    const int per_group = G * tiles_n, first_m = (b / per_group) * G;
    const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
    const int tm = first_m + (b % per_group) % gsize, tn = (b % per_group) / gsize;
    const int m0 = __builtin_amdgcn_readfirstlane(tm * BM), n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);
    const __amdgpu_buffer_rsrc_t rx = operand_rsrc_u8<BM>(g.X, g.ldx, m0, g.M);
    const __amdgpu_buffer_rsrc_t rw = operand_rsrc_u8<BN>(g.W, g.ldw, n0, g.N);

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    dma_tile_u8<BM, NW>(rx, g.ldx, 0, g.K, lds);
    dma_tile_u8<BN, NW>(rw, g.ldw, 0, g.K, lds + BM * 128);
    __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
    __syncthreads();
    const int nk = (g.K + BK8 - 1) / BK8;
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t* cur = lds + (kt & 1) * kStage;
        if (kt + 1 < nk) {
            uint8_t* nxt = lds + ((kt + 1) & 1) * kStage;
            dma_tile_u8<BM, NW>(rx, g.ldx, (kt + 1) * BK8, g.K, nxt);
            dma_tile_u8<BN, NW>(rw, g.ldw, (kt + 1) * BK8, g.K, nxt + BM * 128);
        }
#pragma unroll
        for (int js = 0; js < 2; ++js) {
            i32x8 a[TI], bb[TJ];
            const int c0 = 4 * js + (lane >> 5);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int r = wm + 32 * i + (lane & 31);
                a[i] = frag_f8(cur + r * 128, r, c0);
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int r = wn + 32 * j + (lane & 31);
                bb[j] = frag_f8(cur + BM * 128 + r * 128, r, c0);
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn + 32 * j + (lane & 31);
            if (col >= g.N) continue;
            const float sw = g.sw[col];
            float bv = 0.0f;
            if constexpr (BIAS) bv = __uint_as_float((uint32_t)g.bias[col] << 16);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const float s0 = row < g.M ? g.sx[row] : 0.0f, s1 = row + 1 < g.M ? g.sx[row + 1] : 0.0f;
                const uint32_t pk = pack_bf16x2(acc[i][j][r] * sw * s0 + bv, acc[i][j][r + 1] * sw * s1 + bv);
                if (row < g.M) g.Y[(size_t)row * g.ldy + col] = (uint16_t)(pk & 0xFFFFu);
                if (row + 1 < g.M) g.Y[(size_t)(row + 1) * g.ldy + col] = (uint16_t)(pk >> 16);
            }
        }
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_f8(const GemmF8Args& g, hipStream_t stream) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (g.bias)
        hipLaunchKernelGGL((gemm_f8<BM, BN, WGM, WGN, true>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_f8<BM, BN, WGM, WGN, false>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
    return hipGetLastError();
}

// Per-row E4M3 quantization: one 256-thread block per row. CH > 0: each thread holds its CH
// chunks of 8 elements in registers (K <= 2048 CH), so the row is read once; CH = 0: two passes
// over the row (the second from L2). The absolute maximum is reduced within each wave, then
// across the four waves in LDS.
template <int CH>
__global__ __launch_bounds__(256) void quantize_rows_f8(const uint16_t* X, int K, int ldx, uint8_t* Q, int ldq, float* S) {
    __shared__ float wmax[4];
    const int m = blockIdx.x;
    const uint16_t* x = X + (size_t)m * ldx;
    constexpr int R = CH > 0 ? CH : 1;
    uint4 v[R];
    float amax = 0.0f;
    auto absmax8 = [](const uint4& c, float a) {
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) a = fmaxf(a, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
        return a;
    };
    if constexpr (CH > 0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int k = 8 * (threadIdx.x + 256 * c);
            v[c] = k < K ? *reinterpret_cast<const uint4*>(x + k) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) amax = absmax8(v[c], amax);
    } else {
        for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) amax = absmax8(*reinterpret_cast<const uint4*>(x + k), amax);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    uint8_t* q = Q + (size_t)m * ldq;
    if (amax == 0.0f) {                                        // a zero row: scale 0, codes 0 (+0)
        for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) *reinterpret_cast<uint2*>(q + k) = make_uint2(0u, 0u);
        if (threadIdx.x == 0) S[m] = 0.0f;
        return;
    }
    amax = fmaxf(amax, 0x1p-100f);
    const float inv = 448.0f / amax;
    if (threadIdx.x == 0) S[m] = amax / 448.0f;
    // v_cvt_pk_fp8_f32: two fp32 values to OCP E4M3 codes, rounded to nearest even; |x inv| <= 448
    // up to one rounding of the product, which rounds back to 448, so no code saturates
    auto codes8 = [inv](const uint4& c) {
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
        auto lo = [inv](uint32_t v) { return __uint_as_float(v << 16) * inv; };
        auto hi = [inv](uint32_t v) { return __uint_as_float(v & 0xFFFF0000u) * inv; };
        int r0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo(w[0]), hi(w[0]), 0, false);
        r0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo(w[1]), hi(w[1]), r0, true);
        int r1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo(w[2]), hi(w[2]), 0, false);
        r1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo(w[3]), hi(w[3]), r1, true);
        return make_uint2((uint32_t)r0, (uint32_t)r1);
    };
    if constexpr (CH > 0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int k = 8 * (threadIdx.x + 256 * c);
            if (k < K) *reinterpret_cast<uint2*>(q + k) = codes8(v[c]);
        }
    } else {
        for (int k = 8 * threadIdx.x; k < K; k += 8 * 256)
            *reinterpret_cast<uint2*>(q + k) = codes8(*reinterpret_cast<const uint4*>(x + k));
    }
}

// Skinny FP8 GEMM for M <= 64, as gemm_skinny: a block owns 16 output columns, 8 waves split K in
// 128-code chunks, W streams from HBM into registers, 16x16x128 FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4):
// lane l supplies row l % 16 of A and column l % 16 of B with the 32 codes 32 (l / 16) .. + 31 of
// the chunk (the same rule for both operands, so equal k meet) and receives C[4 (l / 16) + i][l % 16].
template <int MT, bool BIAS>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_f8(GemmF8Args g) {
    __shared__ float red[kSkinnyWaves][MT][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, kq = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nrows = g.N - n0 < 16 ? g.N - n0 : 16;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.W + (size_t)n0 * g.ldw), 0, (int)((size_t)nrows * g.ldw), 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.X), 0, (int)((size_t)g.M * g.ldx), 0x00020000);
    const uint32_t woff = (uint32_t)r * g.ldw;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{};
    const int nkc = (g.K + 127) / 128;
    for (int kb = wave; kb < nkc; kb += kSkinnyWaves * kSkinnyUnroll) {
        uint4 bw[kSkinnyUnroll][2], ax[kSkinnyUnroll][MT][2];
#pragma unroll
        for (int u = 0; u < kSkinnyUnroll; ++u) {
            const int kc = kb + u * kSkinnyWaves;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = kc * 128 + 32 * kq + 16 * h;
                const bool in = kc < nkc && k < g.K;
                bw[u][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, in ? woff + (uint32_t)k : kOob, 0, 0));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t xo = (uint32_t)(mt * 16 + r) * g.ldx + (uint32_t)k;
                    ax[u][mt][h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xo : kOob, 0, 0));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kSkinnyUnroll; ++u) {
            const i32x8 b8 = {(int)bw[u][0].x, (int)bw[u][0].y, (int)bw[u][0].z, (int)bw[u][0].w,
                              (int)bw[u][1].x, (int)bw[u][1].y, (int)bw[u][1].z, (int)bw[u][1].w};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const i32x8 a8 = {(int)ax[u][mt][0].x, (int)ax[u][mt][0].y, (int)ax[u][mt][0].z, (int)ax[u][mt][0].w,
                                  (int)ax[u][mt][1].x, (int)ax[u][mt][1].y, (int)ax[u][mt][1].z, (int)ax[u][mt][1].w};
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[mt], 0, 0, 0, 0, 0, 0);
            }
        }
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
        v = v * g.sw[nn] * g.sx[m];
        if constexpr (BIAS) v += __uint_as_float((uint32_t)g.bias[nn] << 16);
        g.Y[(size_t)m * g.ldy + nn] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

template <int MT>
hipError_t launch_skinny_f8(const GemmF8Args& g, hipStream_t stream) {
    const int blocks = (g.N + 15) / 16;
    if (g.bias)
        hipLaunchKernelGGL((gemm_skinny_f8<MT, true>), dim3(blocks), dim3(64 * kSkinnyWaves), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_skinny_f8<MT, false>), dim3(blocks), dim3(64 * kSkinnyWaves), 0, stream, g);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int PF>
hipError_t launch_tiled(const GemmArgs& g, hipStream_t stream) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    if (g.bias)
        hipLaunchKernelGGL((gemm_nt<BM, BN, WGM, WGN, PF, true>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_nt<BM, BN, WGM, WGN, PF, false>), dim3(tiles), dim3(64 * WGM * WGN), 0, stream, g);
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

hipError_t launch_gemm_f8(const GemmF8Args& g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const long tiles256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256);
    if (tiles256 >= device_cus()) return launch_f8<256, 256, 4, 4>(g, stream);
    const long tiles128 = (long)((g.M + 127) / 128) * ((g.N + 127) / 128);
    if (tiles128 >= 2L * device_cus()) return launch_f8<128, 128, 2, 2>(g, stream);
    if (g.M <= 16) return launch_skinny_f8<1>(g, stream);
    if (g.M <= 32) return launch_skinny_f8<2>(g, stream);
    if (g.M <= 64) return launch_skinny_f8<4>(g, stream);
    return launch_f8<64, 64, 2, 2>(g, stream);
}

hipError_t launch_quantize_rows_f8(const uint16_t* X, int M, int K, int ldx, uint8_t* Q, int ldq, float* s,
                                   hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    const int chunks = (K + 2047) / 2048;                  // 8-element chunks per thread
    if (chunks <= 1) hipLaunchKernelGGL(quantize_rows_f8<1>, dim3(M), dim3(256), 0, stream, X, K, ldx, Q, ldq, s);
    else if (chunks <= 2) hipLaunchKernelGGL(quantize_rows_f8<2>, dim3(M), dim3(256), 0, stream, X, K, ldx, Q, ldq, s);
    else if (chunks <= 4) hipLaunchKernelGGL(quantize_rows_f8<4>, dim3(M), dim3(256), 0, stream, X, K, ldx, Q, ldq, s);
    else if (chunks <= 8) hipLaunchKernelGGL(quantize_rows_f8<8>, dim3(M), dim3(256), 0, stream, X, K, ldx, Q, ldq, s);
    else hipLaunchKernelGGL(quantize_rows_f8<0>, dim3(M), dim3(256), 0, stream, X, K, ldx, Q, ldq, s);
    return hipGetLastError();
}

int split_columns(int K, int splits) { return (K / splits + BK - 1) / BK * BK; }

int gemm_splits(int M, int N, int K) {
    if (M <= 64) return 1;
    const long tiles256 = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (tiles256 >= device_cus()) return 1;
    long s = (device_cus() + tiles256 - 1) / tiles256;
    s = s < 8 ? s : 8;
    while (s > 1 && K / s < 4 * BK) --s;
    return (int)s;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    // tile choice: the skinny kernel for a few rows of X; 256 x 256 tiles when every CU gets one,
    // 128 x 128 tiles when every CU gets two, else 64 x 64 tiles
    if (g.M <= 16) return launch_skinny<1>(g, stream);
    if (g.M <= 32) return launch_skinny<2>(g, stream);
    if (g.M <= 64) return launch_skinny<4>(g, stream);
    const long tiles256 = (long)((g.M + 255) / 256) * ((g.N + 255) / 256);
    if (tiles256 >= device_cus()) return launch_dma<256, 256, 2, 4>(g, stream);
    // too few 256 x 256 tiles to fill the CUs: K split over the blocks (the caller's choice, with
    // room for the fp32 partial tiles), then the splits added in order
    if (g.splits > 1) {
        if (!g.part || g.part_bytes < (size_t)g.splits * g.M * g.N * sizeof(float)) return hipErrorInvalidValue;
        GemmArgs h = g;
        h.kc = split_columns(g.K, g.splits);
        const int used = (g.K + h.kc - 1) / h.kc;
        const dim3 grid((unsigned)tiles256, (unsigned)used);
        hipLaunchKernelGGL((gemm_dma<256, 256, 2, 4, false, true>), grid, dim3(64 * 8), 0, stream, h);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n = (int64_t)g.M * g.N;
        hipLaunchKernelGGL(gemm_split_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, g.part, used, g.bias,
                           g.Y, g.M, g.N, g.ldy);
        return hipGetLastError();
    }
    const long tiles128 = (long)((g.M + 127) / 128) * ((g.N + 127) / 128);
    if (tiles128 >= 2L * device_cus()) return launch_tiled<128, 128, 2, 2, kPrefetch>(g, stream);
    return launch_tiled<64, 64, 2, 2, kPrefetch>(g, stream);
}

}  // namespace ep
