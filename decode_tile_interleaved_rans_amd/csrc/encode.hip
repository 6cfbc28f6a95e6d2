// gfx950 encoder of the tile-rANS weight codec (lossy mode): the same stream as the host encoder,
// byte for byte, from a weight in device memory.
//
// The method's encoder steps ("EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
// Arbitrary Bitrates", Abstract: rows scaled to unit size, E8 lattice quantization, a conditional
// coordinate model, a step chosen from a size estimate on a sample, tile-wise entropy coding) run
// as kernels:
//   row_stats      one thread per row sums w^2 in fp64 in column order (the order fixes the
//                  rounding, so it matches the host), then s_r = fp32(sqrt(sum / C)), and the
//                  row's max |w / s_r| (an exact maximum)
//   quantize       nearest E8 point of 8-column blocks at a given step: the rate-search sample
//                  (strided blocks) or every block of the padded matrix; per-table value
//                  histograms (LDS bins for |x| < 128, global atomics beyond), doubled
//                  coordinates, cosets and each row's max |q|
//   windows        per table, the coded window (the whole value range when it has at most 255
//                  values, else the 255-wide window holding the most values, smallest start on
//                  ties) and its symbol counts
//   encode_tiles   one wave64 per two tiles: every lane runs its rANS state backwards over the
//                  tile's steps and stacks its escape and renormalization words at positions given
//                  by wave ballots (escapes, then refills, each in descending lane order)
//   assemble       each tile's 32 states and its words in reading order at the tile's offset
//   chunk_crc      CRC-32 of 512-byte payload chunks, combined on the host
// The host part keeps what is order-sensitive in floating point or tiny: the entropy estimate of
// each bisection step (same summation as the host encoder), the frequency normalization, the tile
// offsets and the header.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kTables = 17;
constexpr int kSpan2 = 2 * kValueSpan;      // histogram bins per table, value x at x + kValueSpan
constexpr int kNearBins = 256;              // LDS bins per table for -128 <= x < 128
constexpr uint32_t kRansL = 1u << 16;

// ----------------------------------------------------------------------------- element access
template <int DT>
__device__ __forceinline__ double widen_d(const void* w, int64_t i) {
    if constexpr (DT == EP_F32) {
        return (double)static_cast<const float*>(w)[i];
    } else if constexpr (DT == EP_BF16) {
        return (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(w)[i] << 16);
    } else {
        const uint32_t h = static_cast<const uint16_t*>(w)[i];
        const int sgn = h >> 15, e = (h >> 10) & 31, m = h & 1023;
        const double v = e == 0 ? ldexp((double)m, -24)
                         : e == 31 ? (m ? __longlong_as_double(0x7FF8000000000000ll) : __longlong_as_double(0x7FF0000000000000ll))
                                   : ldexp(1.0 + m / 1024.0, e - 15);
        return sgn ? -v : v;
    }
}

// ----------------------------------------------------------------------------- E8 (Conway & Sloane)
__device__ __forceinline__ void round_d8(const double* v, double* a) {
    long parity = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = rint(v[i]);                                  // round half to even
        parity += (long)a[i];
    }
    if ((parity & 1) == 0) return;
    int worst = 0;
    double werr = -1.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double e = fabs(v[i] - a[i]);
        if (e > werr) {
            werr = e;
            worst = i;
        }
    }
    a[worst] += v[worst] >= a[worst] ? 1.0 : -1.0;
}

// Doubled coordinates q and coset b of the E8 point nearest to y.
__device__ __forceinline__ int nearest_e8(const double* y, int32_t* q) {
    double even[8], odd[8], shifted[8];
    round_d8(y, even);
#pragma unroll
    for (int i = 0; i < 8; ++i) shifted[i] = y[i] - 0.5;
    round_d8(shifted, odd);
    double de = 0.0, dodd = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        odd[i] += 0.5;
        const double e0 = y[i] - even[i], e1 = y[i] - odd[i];
        de += e0 * e0;
        dodd += e1 * e1;
    }
    const int b = de <= dodd ? 0 : 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (int32_t)(2.0 * (b ? odd[i] : even[i]));
    return b;
}

template <int DT>
__device__ __forceinline__ void block_y(const void* w, const float* scale, int64_t R, int64_t C, int64_t r, int64_t k,
                                        double delta, double* y) {
    const double den = r < R ? (double)scale[r] * delta : 1.0;
    const bool live = r < R && scale[r] != 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t c = 8 * k + i;
        y[i] = (live && c < C) ? widen_d<DT>(w, r * C + c) / den : 0.0;
    }
}

// ----------------------------------------------------------------------------- row statistics
// One thread per row: the fp64 sum of squares in column order (16-byte loads when every row is
// 16-byte aligned, the same order either way) and max |w|. max_j |w_j| / s_r equals the largest of
// the quotients |w_j| / s_r, since a correctly rounded division by s_r > 0 is monotone, so one
// division per row gives the row's max |w / s_r|.
template <int DT>
__device__ __forceinline__ void accumulate(double v, double& acc, double& amax, bool& finite) {
    finite = finite && isfinite(v);
    acc += v * v;
    amax = fmax(amax, fabs(v));
}

template <int DT, bool VEC>
__global__ __launch_bounds__(64) void row_stats(const void* w, int64_t R, int64_t C, float* scale, int* bad,
                                                unsigned long long* umax) {
    const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (r >= R) return;
    double acc = 0.0, amax = 0.0;
    bool finite = true;
    if constexpr (VEC) {
        constexpr int E = DT == EP_F32 ? 4 : 8;                 // elements per 16 bytes
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(w) + (size_t)r * C * (16 / E));
        for (int64_t j = 0; j < C / E; ++j) {
            const uint4 v = p[j];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
            if constexpr (DT == EP_F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) accumulate<DT>((double)__uint_as_float(u[i]), acc, amax, finite);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint16_t h = (uint16_t)(u[i >> 1] >> (16 * (i & 1)));
                    accumulate<DT>(widen_d<DT>(&h, 0), acc, amax, finite);
                }
            }
        }
    } else {
        for (int64_t j = 0; j < C; ++j) accumulate<DT>(widen_d<DT>(w, r * C + j), acc, amax, finite);
    }
    const float s = C ? (float)sqrt(acc / (double)C) : 0.0f;
    scale[r] = s;
    if (!finite || !isfinite(s)) atomicOr(bad, 1);
    if (s != 0.0f && finite) atomicMax(umax, (unsigned long long)__double_as_longlong(amax / (double)s));
}

// ----------------------------------------------------------------------------- quantization
struct QuantArgs {
    const void* w;
    const float* scale;
    int64_t R, C, kb;             // kb = 8-column blocks per padded row
    int64_t kb_sample;            // 8-column blocks per unpadded row (the sample's block numbering)
    int64_t n_blocks;             // blocks to quantize
    // sample mode: block i is the strided block i * nb / n_blocks = i * qn + (i * rn) / n_blocks
    int64_t qn, rn;
    int sample;
    double delta;
    unsigned long long* hist;     // [17][kSpan2] counts
    int* vmin;                    // [17]
    int* vmax;                    // [17]
    int16_t* q;                   // [Rp][Cp] doubled coordinates (full mode)
    uint8_t* coset;               // [Rp][kb] (full mode)
    unsigned int* qmax;           // [R] max |q| over real columns (full mode)
    int* bad;                     // bit 1: a coordinate beyond the int16 escape range
};

template <int DT>
__global__ __launch_bounds__(256) void quantize(QuantArgs a) {
    __shared__ unsigned int near_bins[kTables][kNearBins];
    __shared__ int tmin[kTables], tmax[kTables];
    __shared__ unsigned int rmax[9];
    for (int i = threadIdx.x; i < kTables * kNearBins; i += 256) (&near_bins[0][0])[i] = 0;
    if (threadIdx.x < kTables) {
        tmin[threadIdx.x] = INT32_MAX;
        tmax[threadIdx.x] = INT32_MIN;
    }
    if (threadIdx.x < 9) rmax[threadIdx.x] = 0;
    __syncthreads();
    const int64_t first = (int64_t)blockIdx.x * 256;
    const int64_t i = first + threadIdx.x;
    const int64_t row0 = a.sample ? 0 : first / a.kb;
    if (i < a.n_blocks) {
        const int64_t idx = a.sample ? i * a.qn + (i * a.rn) / a.n_blocks : i;
        const int64_t kbi = a.sample ? a.kb_sample : a.kb;
        const int64_t r = idx / kbi, k = idx % kbi;
        double y[8];
        block_y<DT>(a.w, a.scale, a.R, a.C, r, k, a.delta, y);
        int32_t q[8];
        const int b = nearest_e8(y, q);
        auto add = [&](int t, int32_t x) {
            if (x >= -128 && x < 128) atomicAdd(&near_bins[t][x + 128], 1u);
            else atomicAdd(&a.hist[(int64_t)t * kSpan2 + x + kValueSpan], 1ull);
            atomicMin(&tmin[t], x);
            atomicMax(&tmax[t], x);
        };
        add(0, b);
        uint32_t m = 0;
        bool range_ok = true;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int32_t x = (q[j] - b) / 2;
            if (x <= -kValueSpan || x >= kValueSpan) range_ok = false;
            else add(1 + 2 * j + b, x);
            if (8 * k + j < a.C) m = max(m, (uint32_t)abs(q[j]));
        }
        if (!range_ok) atomicOr(a.bad, 2);
        if (!a.sample) {
            uint32_t p0 = (uint32_t)(uint16_t)q[0] | (uint32_t)(uint16_t)q[1] << 16;
            uint32_t p1 = (uint32_t)(uint16_t)q[2] | (uint32_t)(uint16_t)q[3] << 16;
            uint32_t p2 = (uint32_t)(uint16_t)q[4] | (uint32_t)(uint16_t)q[5] << 16;
            uint32_t p3 = (uint32_t)(uint16_t)q[6] | (uint32_t)(uint16_t)q[7] << 16;
            *reinterpret_cast<uint4*>(a.q + r * (8 * a.kb) + 8 * k) = make_uint4(p0, p1, p2, p3);
            a.coset[idx] = (uint8_t)b;
            if (r < a.R) atomicMax(&rmax[r - row0], m);      // 256 consecutive blocks span <= 9 rows
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTables * kNearBins; e += 256) {
        const unsigned int c = (&near_bins[0][0])[e];
        if (c) atomicAdd(&a.hist[(int64_t)(e / kNearBins) * kSpan2 + (e % kNearBins) - 128 + kValueSpan], (unsigned long long)c);
    }
    if (threadIdx.x < kTables && tmin[threadIdx.x] <= tmax[threadIdx.x]) {
        atomicMin(&a.vmin[threadIdx.x], tmin[threadIdx.x]);
        atomicMax(&a.vmax[threadIdx.x], tmax[threadIdx.x]);
    }
    if (!a.sample && threadIdx.x < 9) {
        const int64_t r = row0 + threadIdx.x;
        if (r < a.R && rmax[threadIdx.x]) atomicMax(&a.qmax[r], rmax[threadIdx.x]);
    }
}

// ----------------------------------------------------------------------------- windows
struct WindowOut {
    int32_t lo, width;
    unsigned long long total;
    unsigned long long cnt[256];
};

// One block per table. Windows of 255 values start at s in [vmin, vmax - 254]; thread t scans a
// contiguous run of starts, then the block keeps the largest count at the smallest start.
__global__ __launch_bounds__(1024) void windows(const unsigned long long* hist, const int* vmin, const int* vmax,
                                                WindowOut* out) {
    __shared__ unsigned long long best_c[1024];
    __shared__ int best_s[1024];
    __shared__ unsigned long long tot_part[1024];
    const int t = blockIdx.x;
    const unsigned long long* h = hist + (int64_t)t * kSpan2 + kValueSpan;   // h[x], x in [-span, span)
    const int lo_v = vmin[t], hi_v = vmax[t];
    WindowOut& o = out[t];
    unsigned long long tot = 0;
    if (lo_v <= hi_v)
        for (int x = lo_v + (int)threadIdx.x; x <= hi_v; x += 1024) tot += h[x];
    tot_part[threadIdx.x] = tot;
    __syncthreads();
    for (int sft = 512; sft > 0; sft >>= 1) {
        if ((int)threadIdx.x < sft) tot_part[threadIdx.x] += tot_part[threadIdx.x + sft];
        __syncthreads();
    }
    const unsigned long long total = tot_part[0];
    int lo = 0, width = 1;
    if (total != 0) {
        if (hi_v - lo_v + 1 <= 255) {
            lo = lo_v;
            width = hi_v - lo_v + 1;
        } else {
            const int n_starts = hi_v - 254 - lo_v + 1;
            const int per = (n_starts + 1023) / 1024;
            const int s0 = lo_v + (int)threadIdx.x * per, s1 = min(s0 + per, lo_v + n_starts);
            unsigned long long bc = 0;
            int bs = INT32_MAX;
            if (s0 < s1) {
                unsigned long long run = 0;
                for (int x = s0; x < s0 + 255; ++x) run += h[x];
                bc = run;
                bs = s0;
                for (int s = s0 + 1; s < s1; ++s) {
                    run += h[s + 254];
                    run -= h[s - 1];
                    if (run > bc) {
                        bc = run;
                        bs = s;
                    }
                }
            }
            best_c[threadIdx.x] = bc;
            best_s[threadIdx.x] = bs;
            __syncthreads();
            for (int sft = 512; sft > 0; sft >>= 1) {
                if ((int)threadIdx.x < sft) {
                    const unsigned long long c2 = best_c[threadIdx.x + sft];
                    const int s2 = best_s[threadIdx.x + sft];
                    if (c2 > best_c[threadIdx.x] || (c2 == best_c[threadIdx.x] && s2 < best_s[threadIdx.x])) {
                        best_c[threadIdx.x] = c2;
                        best_s[threadIdx.x] = s2;
                    }
                }
                __syncthreads();
            }
            lo = best_s[0];
            width = 255;
        }
    }
    if (threadIdx.x < 256) {
        const int s = threadIdx.x;
        o.cnt[s] = (total != 0 && s < width) ? h[lo + s] : 0ull;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long in = 0;
        for (int s = 0; s < width && total != 0; ++s) in += o.cnt[s];
        if (total != 0 && width <= 255) o.cnt[255] = total - in;   // escapes (width <= 255 leaves slot 255 free)
        o.lo = lo;
        o.width = width;
        o.total = total;
    }
}

// ----------------------------------------------------------------------------- tile rANS
struct TileArgs {
    const int16_t* q;             // [Rp][Cp]
    const uint8_t* coset;         // [Rp][kb]
    const uint32_t* fc;           // [17][256] f | c << 16
    const int32_t* lo;            // [17]
    const int32_t* width;         // [17]
    int64_t kb, tiles_c, n_tiles;
    int tile_rows, prob_bits, layout;
    uint16_t* stack;              // [n_tiles][cap] words in stack order
    int64_t cap;
    uint32_t* states;             // [n_tiles][32] final states
    uint32_t* words;              // [n_tiles] word count
    unsigned int* n_esc;
};

__global__ __launch_bounds__(256) void encode_tiles(TileArgs a) {
    __shared__ uint32_t fc[kTables * 256];
    for (int i = threadIdx.x; i < kTables * 256; i += 256) fc[i] = a.fc[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, half = lane >> 5, l = lane & 31;
    const int64_t tile = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + half;
    const bool live = tile < a.n_tiles;
    const int64_t tr = live ? tile / a.tiles_c : 0, tc = live ? tile % a.tiles_c : 0;
    const int n = a.prob_bits;
    const int lo0 = a.lo[0];
    uint32_t x = kRansL;
    uint32_t sp = 0;
    unsigned int esc_count = 0;
    uint16_t* st = a.stack + (live ? tile : 0) * a.cap;
    const uint32_t above = l == 31 ? 0u : ~0u << (l + 1);     // lanes above this one in the half
    for (int bs = a.tile_rows - 1; bs >= 0; --bs) {
        int rr, kk;                                           // the block this lane codes at step bs
        block_of(a.layout, a.tile_rows, l, bs, &rr, &kk);
        const int64_t r = tr * a.tile_rows + rr, k = tc * 32 + kk;
        int32_t qv[8];
        int b = 0;
        if (live) {
            const uint4 p = *reinterpret_cast<const uint4*>(a.q + r * (8 * a.kb) + 8 * k);
            const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qv[2 * j] = (int16_t)(w[j] & 0xFFFFu);
                qv[2 * j + 1] = (int16_t)(w[j] >> 16);
            }
            b = a.coset[r * a.kb + k];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[j] = 0;
        }
        for (int m = 8; m >= 0; --m) {
            int t;
            uint32_t s;
            uint32_t escw = 0;
            bool esc = false;
            if (m == 0) {
                t = 0;
                s = (uint32_t)(b - lo0);
            } else {
                const int j = m - 1;
                t = 1 + 2 * j + b;
                int32_t qj = 0;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    if (jj == j) qj = qv[jj];
                const int32_t xv = (qj - b) / 2;
                const int32_t lo = a.lo[t], wd = a.width[t];
                if (xv >= lo && xv < lo + wd) {
                    s = (uint32_t)(xv - lo);
                } else {
                    s = 255;
                    esc = true;
                    escw = (uint32_t)(uint16_t)(int16_t)xv;
                }
            }
            const uint32_t e = fc[t * 256 + s];
            const uint32_t f = e & 0xFFFFu, c = e >> 16;
            bool spill = false;
            uint32_t spw = 0;
            const uint64_t xmax = (uint64_t)f << (32 - n);        // ((L >> n) << 16) * f
            uint32_t v = x;
            if (live && (uint64_t)v >= xmax) {
                spw = v & 0xFFFFu;
                v >>= 16;
                spill = true;
            }
            // v < f 2^(32 - n) here, so the quotient shifted by n and the sum fit 32 bits
            if (live) x = ((v / f) << n) + v % f + c;
            esc = esc && live;
            // stack order at this step: escapes, then refills, each from the highest lane down
            const uint32_t me = (uint32_t)(__ballot(esc) >> (32 * half));
            const uint32_t ms = (uint32_t)(__ballot(spill) >> (32 * half));
            if (esc) st[sp + __popc(me & above)] = (uint16_t)escw;
            const uint32_t sp2 = sp + __popc(me);
            if (spill) st[sp2 + __popc(ms & above)] = (uint16_t)spw;
            sp = sp2 + __popc(ms);
            esc_count += esc ? 1u : 0u;
        }
    }
    if (live) {
        a.states[tile * 32 + l] = x;
        if (l == 0) a.words[tile] = sp;
        if (esc_count) atomicAdd(a.n_esc, esc_count);
    }
}

// Tile bytes at their offset: 32 states (lane 0 first), the words in reading order (the stack
// reversed), one zero word if their count is odd.
__global__ __launch_bounds__(256) void assemble(const uint32_t* states, const uint32_t* words, const uint16_t* stack,
                                                int64_t cap, const uint64_t* offsets, int64_t n_tiles, uint8_t* payload) {
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x & 63;
    uint8_t* dst = payload + offsets[tile];
    if (lane < 32) reinterpret_cast<uint32_t*>(dst)[lane] = states[tile * 32 + lane];
    const uint32_t nw = words[tile];
    const uint16_t* st = stack + tile * cap;
    uint16_t* wd = reinterpret_cast<uint16_t*>(dst + 128);
    for (uint32_t i = lane; i < nw; i += 64) wd[i] = st[nw - 1 - i];
    if ((nw & 1) && lane == 0) wd[nw] = 0;
}

// CRC-32 (IEEE, reflected 0xEDB88320) of each 512-byte chunk of the payload.
constexpr int64_t kCrcChunk = 512;

__global__ __launch_bounds__(256) void chunk_crc(const uint8_t* p, int64_t n, uint32_t* out) {
    __shared__ uint32_t tab[256];
    {
        uint32_t c = threadIdx.x;
        for (int k = 0; k < 8; ++k) c = c & 1 ? 0xEDB88320u ^ (c >> 1) : c >> 1;
        tab[threadIdx.x] = c;
    }
    __syncthreads();
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b0 = ch * kCrcChunk;
    if (b0 >= n) return;
    const int64_t b1 = min(n, b0 + kCrcChunk);
    uint32_t c = 0xFFFFFFFFu;
    for (int64_t i = b0; i < b1; i += 4) {                     // n is a multiple of 4
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
        c = tab[(c ^ w) & 0xFF] ^ (c >> 8);
        c = tab[(c ^ (w >> 8)) & 0xFF] ^ (c >> 8);
        c = tab[(c ^ (w >> 16)) & 0xFF] ^ (c >> 8);
        c = tab[(c ^ (w >> 24)) & 0xFF] ^ (c >> 8);
    }
    out[ch] = ~c;
}

// ----------------------------------------------------------------------------- host helpers
// CRC-32 concatenation: crc(A B) = (x^(8 |B|) mod P) * crc(A) + crc(B) over GF(2), with
// polynomials in the reflected bit order of the CRC (bit 31 = x^0).
uint32_t gf2_mulmod(uint32_t a, uint32_t b) {
    uint32_t prod = 0;
    for (uint32_t m = 1u << 31; m; m >>= 1) {
        if (a & m) prod ^= b;
        b = b & 1 ? (b >> 1) ^ 0xEDB88320u : b >> 1;           // b * x mod P
    }
    return prod;
}
uint32_t x_pow_8n(uint64_t nbytes) {                          // x^(8 n) mod P
    uint32_t r = 1u << 31, sq = 1u << 23;                      // x^0 and x^8 in reflected order
    for (; nbytes; nbytes >>= 1) {
        if (nbytes & 1) r = gf2_mulmod(r, sq);
        sq = gf2_mulmod(sq, sq);
    }
    return r;
}

struct DevBuf {
    void* p = nullptr;
    DevBuf() = default;
    DevBuf(const DevBuf&) = delete;
    DevBuf& operator=(const DevBuf&) = delete;
    ~DevBuf() { reset(); }
    void reset() {
        if (p) (void)hipFree(p);
        p = nullptr;
    }
    hipError_t alloc(size_t n) { return hipMalloc(&p, n ? n : 16); }
    template <class T>
    T* as() const { return static_cast<T*>(p); }
};

// Device scratch of the encoder, kept per device between calls and grown to the largest matrix
// encoded so far (allocation and release of a few hundred MB per call would cost more than the
// kernels); calls on one device take turns on it.
struct Scratch {
    DevBuf buf;
    size_t cap = 0;
    hipError_t need(size_t n) {
        if (n <= cap) return hipSuccess;
        buf.reset();
        cap = 0;
        hipError_t e = buf.alloc(n);
        if (e == hipSuccess) cap = n;
        return e;
    }
    void* p() const { return buf.p; }
    template <class T>
    T* as() const { return static_cast<T*>(buf.p); }
};

struct EncoderScratch {
    std::mutex mu;
    Scratch scale, flag, umax, hist, vmin, vmax, win, q, coset, qmax, fc, lo, wd, stack, states, words, nesc, off,
        payload, crc;
};

constexpr int kMaxDevices = 64;

EncoderScratch& encoder_scratch(int device) {
    static EncoderScratch per_device[kMaxDevices];
    return per_device[device];
}

#define EP_HIP(call)                                                         \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            *why = std::string(#call) + ": " + hipGetErrorString(e_);        \
            return e_ == hipErrorOutOfMemory ? EP_ENOMEM : EP_EHIP;          \
        }                                                                    \
    } while (0)

template <int DT>
ep_status encode_lossy_dt(const void* w, int64_t R, int64_t C, const ep_encode_opts& o, hipStream_t s,
                          Bytes* out, std::string* why, EncoderScratch& X) {
    const int tr = o.tile_rows, n = o.prob_bits;
    const int64_t Rp = (R + tr - 1) / tr * tr, Cp = (C + 255) / 256 * 256, kb = Cp / 8;
    Scratch &d_scale = X.scale, &d_flag = X.flag, &d_umax = X.umax, &d_hist = X.hist, &d_vmin = X.vmin,
            &d_vmax = X.vmax, &d_win = X.win, &d_q = X.q, &d_coset = X.coset, &d_qmax = X.qmax;
    EP_HIP(d_scale.need(sizeof(float) * std::max<int64_t>(R, 1)));
    EP_HIP(d_flag.need(sizeof(int)));
    EP_HIP(d_umax.need(sizeof(unsigned long long)));
    EP_HIP(hipMemsetAsync(d_flag.p(), 0, sizeof(int), s));
    EP_HIP(hipMemsetAsync(d_umax.p(), 0, sizeof(unsigned long long), s));
    std::vector<float> scale(R, 0.0f);
    unsigned long long umax_bits = 0;
    if (R > 0) {
        const size_t esize = DT == EP_F32 ? 4 : 2;
        const bool vec = ((size_t)C * esize) % 16 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
        if (vec)
            hipLaunchKernelGGL((row_stats<DT, true>), dim3((unsigned)((R + 63) / 64)), dim3(64), 0, s, w, R, C,
                               d_scale.as<float>(), d_flag.as<int>(), d_umax.as<unsigned long long>());
        else
            hipLaunchKernelGGL((row_stats<DT, false>), dim3((unsigned)((R + 63) / 64)), dim3(64), 0, s, w, R, C,
                               d_scale.as<float>(), d_flag.as<int>(), d_umax.as<unsigned long long>());
        EP_HIP(hipGetLastError());
        EP_HIP(hipMemcpyAsync(scale.data(), d_scale.p(), sizeof(float) * R, hipMemcpyDeviceToHost, s));
    }
    int flag = 0;
    EP_HIP(hipMemcpyAsync(&flag, d_flag.p(), sizeof(int), hipMemcpyDeviceToHost, s));
    EP_HIP(hipMemcpyAsync(&umax_bits, d_umax.p(), sizeof(umax_bits), hipMemcpyDeviceToHost, s));
    EP_HIP(hipStreamSynchronize(s));
    if (flag & 1) {
        *why = "lossy input holds a non-finite value (or a row whose sum of squares overflows)";
        return EP_ERANGE;
    }
    double U;
    std::memcpy(&U, &umax_bits, sizeof U);

    EP_HIP(d_hist.need(sizeof(unsigned long long) * kTables * kSpan2));
    EP_HIP(d_vmin.need(sizeof(int) * kTables));
    EP_HIP(d_vmax.need(sizeof(int) * kTables));
    EP_HIP(d_win.need(sizeof(WindowOut) * kTables));
    std::vector<WindowOut> win(kTables);
    QuantArgs qa{};
    qa.w = w;
    qa.scale = d_scale.as<float>();
    qa.R = R;
    qa.C = C;
    qa.kb = kb;
    qa.kb_sample = (C + 7) / 8;
    qa.hist = d_hist.as<unsigned long long>();
    qa.vmin = d_vmin.as<int>();
    qa.vmax = d_vmax.as<int>();
    qa.bad = d_flag.as<int>();
    // histograms of one quantization pass, windowed per table, copied to win
    auto run_pass = [&](double delta) -> ep_status {
        std::vector<int> init_min(kTables, INT32_MAX), init_max(kTables, INT32_MIN);
        EP_HIP(hipMemsetAsync(d_hist.p(), 0, sizeof(unsigned long long) * kTables * kSpan2, s));
        EP_HIP(hipMemcpyAsync(d_vmin.p(), init_min.data(), sizeof(int) * kTables, hipMemcpyHostToDevice, s));
        EP_HIP(hipMemcpyAsync(d_vmax.p(), init_max.data(), sizeof(int) * kTables, hipMemcpyHostToDevice, s));
        qa.delta = delta;
        if (qa.n_blocks > 0) {
            hipLaunchKernelGGL(quantize<DT>, dim3((unsigned)((qa.n_blocks + 255) / 256)), dim3(256), 0, s, qa);
            EP_HIP(hipGetLastError());
        }
        hipLaunchKernelGGL(windows, dim3(kTables), dim3(1024), 0, s, d_hist.as<unsigned long long>(), d_vmin.as<int>(),
                           d_vmax.as<int>(), d_win.as<WindowOut>());
        EP_HIP(hipGetLastError());
        EP_HIP(hipMemcpyAsync(win.data(), d_win.p(), sizeof(WindowOut) * kTables, hipMemcpyDeviceToHost, s));
        EP_HIP(hipStreamSynchronize(s));
        return EP_OK;
    };

    float step = 1.0f;
    if (R > 0 && C > 0) {
        const int64_t nb = R * ((C + 7) / 8);
        const int64_t sb = std::min<int64_t>(nb, kSampleBlocks);
        qa.sample = 1;
        qa.n_blocks = sb;
        qa.qn = nb / sb;
        qa.rn = nb % sb;
        ep_status st = EP_OK;
        uint64_t cnt[kTables][256], totals[kTables];
        step = choose_step(U, o.target_bpp, [&](double d) {
            if (st != EP_OK) return 0.0;
            st = run_pass(d);
            if (st != EP_OK) return 0.0;
            for (int t = 0; t < kTables; ++t) {
                for (int k2 = 0; k2 < 256; ++k2) cnt[t][k2] = win[t].cnt[k2];
                totals[t] = win[t].total;
            }
            return sample_estimate(cnt, totals, sb);
        });
        if (st != EP_OK) return st;
    }

    // full quantization of the padded matrix
    EP_HIP(d_q.need(sizeof(int16_t) * Rp * Cp));
    EP_HIP(d_coset.need(Rp * kb));
    EP_HIP(d_qmax.need(sizeof(unsigned int) * std::max<int64_t>(R, 1)));
    EP_HIP(hipMemsetAsync(d_qmax.p(), 0, sizeof(unsigned int) * std::max<int64_t>(R, 1), s));
    EP_HIP(hipMemsetAsync(d_flag.p(), 0, sizeof(int), s));
    qa.sample = 0;
    qa.n_blocks = Rp * kb;
    qa.qn = qa.rn = 0;
    qa.q = d_q.as<int16_t>();
    qa.coset = d_coset.as<uint8_t>();
    qa.qmax = d_qmax.as<unsigned int>();
    if (ep_status st = run_pass((double)step); st != EP_OK) return st;
    EP_HIP(hipMemcpy(&flag, d_flag.p(), sizeof(int), hipMemcpyDeviceToHost));
    if (flag & 2) {
        *why = "lattice coordinate beyond the int16 escape range";
        return EP_ERANGE;
    }
    std::vector<unsigned int> qmax32(R);
    if (R > 0) EP_HIP(hipMemcpy(qmax32.data(), d_qmax.p(), sizeof(unsigned int) * R, hipMemcpyDeviceToHost));
    std::vector<uint16_t> qmax(R);
    for (int64_t r = 0; r < R; ++r) qmax[r] = (uint16_t)qmax32[r];
    std::vector<Table> tables(kTables);
    std::vector<uint32_t> fc(kTables * 256);
    std::vector<int32_t> lo(kTables), width(kTables);
    for (int t = 0; t < kTables; ++t) {
        uint64_t cnt[256];
        for (int k2 = 0; k2 < 256; ++k2) cnt[k2] = win[t].cnt[k2];
        tables[t].lo = win[t].lo;
        tables[t].width = win[t].width;
        if (!normalize_frequencies(cnt, n, tables[t].freq)) {
            *why = "frequency normalization failed";
            return EP_ERANGE;
        }
        uint32_t acc = 0;
        for (int k2 = 0; k2 < 256; ++k2) {
            fc[t * 256 + k2] = tables[t].freq[k2] | acc << 16;
            acc += tables[t].freq[k2];
        }
        lo[t] = win[t].lo;
        width[t] = win[t].width;
    }

    // tiles
    const int64_t tiles_c = Cp / 256, n_tiles = (Rp / tr) * tiles_c;
    const int64_t cap = 64 * 9 * (int64_t)tr;                // words a tile can stack at most
    Scratch &d_fc = X.fc, &d_lo = X.lo, &d_wd = X.wd, &d_stack = X.stack, &d_states = X.states, &d_words = X.words,
            &d_nesc = X.nesc;
    EP_HIP(d_fc.need(sizeof(uint32_t) * kTables * 256));
    EP_HIP(d_lo.need(sizeof(int32_t) * kTables));
    EP_HIP(d_wd.need(sizeof(int32_t) * kTables));
    EP_HIP(d_stack.need(sizeof(uint16_t) * std::max<int64_t>(n_tiles, 1) * cap));
    EP_HIP(d_states.need(sizeof(uint32_t) * 32 * std::max<int64_t>(n_tiles, 1)));
    EP_HIP(d_words.need(sizeof(uint32_t) * std::max<int64_t>(n_tiles, 1)));
    EP_HIP(d_nesc.need(sizeof(unsigned int)));
    EP_HIP(hipMemcpyAsync(d_fc.p(), fc.data(), sizeof(uint32_t) * kTables * 256, hipMemcpyHostToDevice, s));
    EP_HIP(hipMemcpyAsync(d_lo.p(), lo.data(), sizeof(int32_t) * kTables, hipMemcpyHostToDevice, s));
    EP_HIP(hipMemcpyAsync(d_wd.p(), width.data(), sizeof(int32_t) * kTables, hipMemcpyHostToDevice, s));
    EP_HIP(hipMemsetAsync(d_nesc.p(), 0, sizeof(unsigned int), s));
    std::vector<uint32_t> words(n_tiles);
    unsigned int n_esc = 0;
    if (n_tiles > 0) {
        TileArgs ta{d_q.as<int16_t>(), d_coset.as<uint8_t>(), d_fc.as<uint32_t>(), d_lo.as<int32_t>(), d_wd.as<int32_t>(),
                    kb, tiles_c, n_tiles, tr, n, o.layout, d_stack.as<uint16_t>(), cap, d_states.as<uint32_t>(),
                    d_words.as<uint32_t>(), d_nesc.as<unsigned int>()};
        hipLaunchKernelGGL(encode_tiles, dim3((unsigned)((n_tiles + 7) / 8)), dim3(256), 0, s, ta);
        EP_HIP(hipGetLastError());
        EP_HIP(hipMemcpyAsync(words.data(), d_words.p(), sizeof(uint32_t) * n_tiles, hipMemcpyDeviceToHost, s));
        EP_HIP(hipMemcpyAsync(&n_esc, d_nesc.p(), sizeof(unsigned int), hipMemcpyDeviceToHost, s));
        EP_HIP(hipStreamSynchronize(s));
    }
    std::vector<uint32_t> offsets(n_tiles + 1, 0);
    std::vector<uint64_t> byte_off(std::max<int64_t>(n_tiles, 1), 0);
    uint64_t acc = 0;
    for (int64_t t = 0; t < n_tiles; ++t) {
        byte_off[t] = acc;
        acc += 128 + 2 * (uint64_t)words[t] + 2 * (uint64_t)(words[t] & 1);
        offsets[t + 1] = (uint32_t)(acc / 4);
    }
    uint32_t crc = 0;
    Scratch &d_off = X.off, &d_payload = X.payload, &d_crc = X.crc;
    if (n_tiles > 0) {
        EP_HIP(d_off.need(sizeof(uint64_t) * n_tiles));
        EP_HIP(d_payload.need(acc));
        const int64_t n_chunks = (int64_t)((acc + kCrcChunk - 1) / kCrcChunk);
        EP_HIP(d_crc.need(sizeof(uint32_t) * n_chunks));
        EP_HIP(hipMemcpyAsync(d_off.p(), byte_off.data(), sizeof(uint64_t) * n_tiles, hipMemcpyHostToDevice, s));
        hipLaunchKernelGGL(assemble, dim3((unsigned)((n_tiles + 3) / 4)), dim3(256), 0, s, d_states.as<uint32_t>(),
                           d_words.as<uint32_t>(), d_stack.as<uint16_t>(), cap, d_off.as<uint64_t>(), n_tiles,
                           d_payload.as<uint8_t>());
        EP_HIP(hipGetLastError());
        hipLaunchKernelGGL(chunk_crc, dim3((unsigned)((n_chunks + 255) / 256)), dim3(256), 0, s, d_payload.as<uint8_t>(),
                           (int64_t)acc, d_crc.as<uint32_t>());
        EP_HIP(hipGetLastError());
        std::vector<uint32_t> crcs(n_chunks);
        EP_HIP(hipMemcpyAsync(crcs.data(), d_crc.p(), sizeof(uint32_t) * n_chunks, hipMemcpyDeviceToHost, s));
        EP_HIP(hipStreamSynchronize(s));
        const uint32_t op_full = x_pow_8n(kCrcChunk);             // every chunk but the last is full
        crc = crcs[0];
        for (int64_t i = 1; i < n_chunks; ++i) {
            const uint64_t len = std::min<uint64_t>(kCrcChunk, acc - (uint64_t)i * kCrcChunk);
            crc = gf2_mulmod(len == (uint64_t)kCrcChunk ? op_full : x_pow_8n(len), crc) ^ crcs[i];
        }
    }
    const uint64_t o_pay = serialize_lossy(DT, R, C, tr, o.layout, n, tables, step, (float)o.target_bpp, scale, qmax, acc,
                                           std::move(offsets), n_esc, n_tiles > 0 ? crc : 0u, out);
    if (n_tiles > 0) {
        EP_HIP(hipMemcpyAsync(out->data() + o_pay, d_payload.p(), acc, hipMemcpyDeviceToHost, s));
        EP_HIP(hipStreamSynchronize(s));
    }
    return EP_OK;
}

}  // namespace

ep_status encode_lossy_device(const void* dev_w, int dt, int64_t rows, int64_t cols, const ep_encode_opts& o,
                              hipStream_t stream, Bytes* out, std::string* why) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) {
        *why = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return EP_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *why = "the device encoder supports device ordinals below 64";
        return EP_EUNSUPPORTED;
    }
    EncoderScratch& X = encoder_scratch(dev);
    std::lock_guard<std::mutex> lock(X.mu);
    switch (dt) {
        case EP_F32: return encode_lossy_dt<EP_F32>(dev_w, rows, cols, o, stream, out, why, X);
        case EP_BF16: return encode_lossy_dt<EP_BF16>(dev_w, rows, cols, o, stream, out, why, X);
        case EP_F16: return encode_lossy_dt<EP_F16>(dev_w, rows, cols, o, stream, out, why, X);
        default:
            *why = "lossy mode takes F32, BF16 or F16 input";
            return EP_EUNSUPPORTED;
    }
}

}  // namespace ep
