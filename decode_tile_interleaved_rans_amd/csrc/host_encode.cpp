// Host encoder of the tile-rANS weight codec: row normalization, nearest E8 point, coordinate
// model, sampled rate search and tile rANS coding, threaded over rows, samples and tiles.
//
// Method steps follow "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
// Bitrates", Abstract: each row is scaled to unit size and quantized to the E8 lattice, the lattice
// coordinates get a conditional symbol model, the quantization step is chosen from a size estimate
// on a sample (one full encode only), and the symbols are entropy-coded in tiles that decode on
// their own.
// The rules the page leaves open are fixed as follows (the decoder relies on all of them):
//   row scale      s_r = fp32(sqrt(sum_j w_rj^2 / C)), fp64 sum in column order; s_r = 0 rows
//                  quantize to 0
//   lattice        E8 = D8 u (D8 + 1/2) (Conway & Sloane's nearest-point rule; odd rounding sums
//                  move the largest-error coordinate, lowest index on ties, upwards at zero
//                  error; equal coset distances keep the integer coset); y = w / (s_r * step)
//   model          table 0 codes the coset bit b, table 1 + 2j + b codes coordinate j of the
//                  block as x = (q_j - b) / 2 inside a window of <= 255 values; other values
//                  are symbol 255 followed by x as a raw int16 word
//   frequencies    f = max(1, floor(c M / T)) for present symbols; a shortfall goes to the most
//                  frequent symbol, an excess is taken one unit at a time from the largest f > 1
//                  (lowest index on ties)
//   rate search    65536 strided sample blocks; entropy of the 17 sampled tables + 16 bits per
//                  escape; 48 log-bisection steps of the step between max(2^-12, 2(U+1)/32767)
//                  and 64, keeping the side at or under the target
//   rANS           32-bit states in [2^16, 2^32), 16-bit words, states start at 2^16; decoding
//                  takes refill words then escape words, each in ascending lane order
//   tiles          tile_rows x 256 columns; lane l owns the 8-column block l of each tile row;
//                  step 9r codes the coset bit of row r, steps 9r+1..9r+8 its 8 coordinates
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <exception>
#include <mutex>
#include <thread>

#include "ep_internal.h"

namespace ep {
namespace {


// ------------------------------------------------------------------------------ threading
// Items 0..n-1 over up to `threads` workers taking the next item from a shared counter. An
// exception in a worker stops the others at their next item and is rethrown here after the join;
// if a thread cannot be started, the workers already running (or this thread) do all the items.
template <class F>
void parallel_for(int64_t n, int threads, F&& fn) {
    if (n <= 0) return;
    int t = (int)std::min<int64_t>(n, std::max(1, threads));
    if (t == 1) {
        for (int64_t i = 0; i < n; ++i) fn(i, 0);
        return;
    }
    std::atomic<int64_t> next{0};
    std::atomic<bool> failed{false};
    std::exception_ptr error;
    std::mutex error_mu;
    auto work = [&](int k) {
        try {
            for (int64_t i = next.fetch_add(1); i < n && !failed.load(); i = next.fetch_add(1)) fn(i, k);
        } catch (...) {
            std::lock_guard<std::mutex> g(error_mu);
            if (!error) error = std::current_exception();
            failed = true;
        }
    };
    std::vector<std::thread> pool;
    pool.reserve(t);
    try {
        for (int k = 0; k < t; ++k) pool.emplace_back(work, k);
    } catch (...) {
        // no more threads: the running ones share the remaining items
    }
    if (pool.empty()) work(0);
    for (auto& th : pool) th.join();
    if (error) std::rethrow_exception(error);
}

// ------------------------------------------------------------------------------ element access
inline double widen(const void* w, int dt, int64_t i) {
    if (dt == EP_F32) return (double)static_cast<const float*>(w)[i];
    uint32_t h = static_cast<const uint16_t*>(w)[i];
    if (dt == EP_BF16) {
        uint32_t u = h << 16;
        float f;
        std::memcpy(&f, &u, 4);
        return (double)f;
    }
    int sgn = h >> 15, e = (h >> 10) & 31, m = h & 1023;   // binary16
    double v = e == 0 ? std::ldexp((double)m, -24)
               : e == 31 ? (m ? NAN : INFINITY)
                         : std::ldexp(1.0 + m / 1024.0, e - 15);
    return sgn ? -v : v;
}

// ------------------------------------------------------------------------------ E8
struct Block {
    int32_t q[8];   // doubled coordinates
    int b;          // coset
};

inline void round_d8(const double* v, double* a) {
    long parity = 0;
    for (int i = 0; i < 8; ++i) {
        a[i] = std::nearbyint(v[i]);
        parity += (long)a[i];
    }
    if ((parity & 1) == 0) return;
    int worst = 0;
    double werr = -1.0;
    for (int i = 0; i < 8; ++i) {
        double e = std::fabs(v[i] - a[i]);
        if (e > werr) {
            werr = e;
            worst = i;
        }
    }
    a[worst] += v[worst] >= a[worst] ? 1.0 : -1.0;
}

inline Block nearest_e8(const double* y) {
    double even[8], odd[8], shifted[8];
    round_d8(y, even);
    for (int i = 0; i < 8; ++i) shifted[i] = y[i] - 0.5;
    round_d8(shifted, odd);
    double de = 0.0, dodd = 0.0;
    for (int i = 0; i < 8; ++i) {
        odd[i] += 0.5;
        double e0 = y[i] - even[i], e1 = y[i] - odd[i];
        de += e0 * e0;
        dodd += e1 * e1;
    }
    Block out;
    out.b = de <= dodd ? 0 : 1;
    const double* p = out.b ? odd : even;
    for (int i = 0; i < 8; ++i) out.q[i] = (int32_t)(2.0 * p[i]);
    return out;
}

// ------------------------------------------------------------------------------ model
struct Hist {
    std::vector<uint64_t> n;   // [2 * kValueSpan], value x at x + kValueSpan
    uint64_t total = 0;
    int32_t vmin = INT32_MAX, vmax = INT32_MIN;
    Hist() : n(2 * kValueSpan, 0) {}
    void clear() {
        if (total) std::fill(n.begin() + (vmin + kValueSpan), n.begin() + (vmax + kValueSpan + 1), 0);
        total = 0;
        vmin = INT32_MAX;
        vmax = INT32_MIN;
    }
    void add(int32_t x, uint64_t c = 1) {
        n[x + kValueSpan] += c;
        total += c;
        vmin = std::min(vmin, x);
        vmax = std::max(vmax, x);
    }
    uint64_t at(int32_t x) const { return n[x + kValueSpan]; }
};

// window + per-symbol counts (escape at 255)
void window_counts(const Hist& h, int32_t* lo, int32_t* width, uint64_t cnt[256]) {
    std::fill(cnt, cnt + 256, 0);
    if (h.total == 0) {
        *lo = 0;
        *width = 1;
        return;
    }
    if (h.vmax - h.vmin + 1 <= 255) {
        *lo = h.vmin;
        *width = h.vmax - h.vmin + 1;
    } else {
        uint64_t run = 0;
        for (int32_t x = h.vmin; x < h.vmin + 255; ++x) run += h.at(x);
        uint64_t best = run;
        int32_t best_lo = h.vmin;
        for (int32_t start = h.vmin + 1; start + 254 <= h.vmax; ++start) {
            run += h.at(start + 254);
            run -= h.at(start - 1);
            if (run > best) {
                best = run;
                best_lo = start;
            }
        }
        *lo = best_lo;
        *width = 255;
    }
    uint64_t in = 0;
    for (int32_t s = 0; s < *width; ++s) {
        cnt[s] = h.at(*lo + s);
        in += cnt[s];
    }
    cnt[kEscape] = h.total - in;
}

bool normalize_freq(const uint64_t cnt[256], int n, uint32_t f[256]) {
    const uint32_t M = 1u << n;
    uint64_t total = 0;
    for (int s = 0; s < 256; ++s) total += cnt[s];
    std::fill(f, f + 256, 0u);
    if (total == 0) {
        f[0] = M;
        return true;
    }
    uint64_t sum = 0;
    int top = 0;
    for (int s = 0; s < 256; ++s) {
        if (cnt[s] > cnt[top]) top = s;
        if (!cnt[s]) continue;
        uint64_t v = cnt[s] * (uint64_t)M / total;
        f[s] = (uint32_t)std::max<uint64_t>(1, v);
        sum += f[s];
    }
    if (sum < M) {
        f[top] += (uint32_t)(M - sum);
        sum = M;
    }
    for (; sum > M; --sum) {
        int big = -1;
        for (int s = 0; s < 256; ++s)
            if (f[s] > 1 && (big < 0 || f[s] > f[big])) big = s;
        if (big < 0) return false;
        --f[big];
    }
    return true;
}

// ------------------------------------------------------------------------------ rANS tile
struct EncTable {
    uint32_t f[256], c[256];
};

void make_enc_table(const uint32_t* f, EncTable* t) {
    uint32_t acc = 0;
    for (int s = 0; s < 256; ++s) {
        t->f[s] = f[s];
        t->c[s] = acc;
        acc += f[s];
    }
}

// One tile: sym/tab/esc are [steps][32]. Appends the tile bytes to out.
void encode_tile(const EncTable* tabs, int n, int steps, const uint8_t* tab, const uint8_t* sym,
                 const uint16_t* esc, bool escapes, std::vector<uint16_t>& stack, std::vector<uint8_t>& out) {
    uint32_t x[kLanes];
    std::fill(x, x + kLanes, kRansLow);
    stack.clear();
    const uint64_t renorm_unit = (uint64_t)((kRansLow >> n) << 16);
    for (int t = steps - 1; t >= 0; --t) {
        const uint8_t* ts = tab + t * kLanes;
        const uint8_t* ss = sym + t * kLanes;
        uint16_t spill[kLanes];
        uint32_t spilled = 0;   // lane bit mask
        for (int l = 0; l < kLanes; ++l) {
            const EncTable& T = tabs[ts[l]];
            uint32_t f = T.f[ss[l]];
            uint64_t v = x[l];
            if (v >= renorm_unit * f) {
                spill[l] = (uint16_t)v;
                v >>= 16;
                spilled |= 1u << l;
            }
            x[l] = (uint32_t)((v / f << n) + v % f + T.c[ss[l]]);
        }
        if (escapes)
            for (int l = kLanes - 1; l >= 0; --l)
                if (ss[l] == kEscape) stack.push_back(esc[t * kLanes + l]);
        for (int l = kLanes - 1; l >= 0; --l)
            if (spilled >> l & 1u) stack.push_back(spill[l]);
    }
    size_t words = stack.size(), base = out.size();
    size_t bytes = 4 * kLanes + 2 * words + (words & 1) * 2;
    out.resize(base + bytes, 0);
    uint8_t* p = out.data() + base;
    for (int l = 0; l < kLanes; ++l)
        for (int k = 0; k < 4; ++k) p[4 * l + k] = (uint8_t)(x[l] >> (8 * k));
    p += 4 * kLanes;
    for (size_t i = 0; i < words; ++i) {
        uint16_t wv = stack[words - 1 - i];
        p[2 * i] = (uint8_t)wv;
        p[2 * i + 1] = (uint8_t)(wv >> 8);
    }
}

// ------------------------------------------------------------------------------ serializer
inline void w16(uint8_t* p, uint32_t v) {
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}
inline void w32(uint8_t* p, uint32_t v) {
    for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k));
}
inline void w64(uint8_t* p, uint64_t v) {
    for (int k = 0; k < 8; ++k) p[k] = (uint8_t)(v >> (8 * k));
}
inline uint64_t up16(uint64_t v) { return (v + 15) & ~uint64_t(15); }
inline uint32_t f32bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

struct TileSet {
    std::vector<uint8_t> payload;
    std::vector<uint32_t> offsets;   // [n_tiles + 1], 4-byte units
    uint64_t external_len = 0;       // payload bytes the caller writes itself (payload empty)
};

// Returns the payload's offset in the stream.
uint64_t serialize(int mode, int dt, int64_t R, int64_t C, int tile_rows, int layout, int n, const std::vector<Table>& tables,
               float step, float target, const std::vector<float>& scale, const std::vector<uint16_t>& qmax,
               const TileSet& ts, uint32_t n_esc, Bytes* out,
               const std::vector<uint8_t>* raw = nullptr, const uint32_t* payload_crc = nullptr) {
    const uint64_t meta_rows = mode == EP_MODE_LOSSY_E8 ? (uint64_t)R : 0;
    uint64_t tables_len = 0;
    for (const Table& t : tables) tables_len += 6 + 2 * (uint64_t)t.width;
    const uint32_t n_tiles = (uint32_t)(ts.offsets.size() - 1);
    const uint64_t o_scale = kHeaderBytes;
    const uint64_t o_qmax = up16(o_scale + 4 * meta_rows);
    const uint64_t o_tab = up16(o_qmax + 2 * meta_rows);
    const uint64_t o_idx = up16(o_tab + tables_len);
    const uint64_t o_raw = raw ? up16(o_idx + 4 * ((uint64_t)n_tiles + 1)) : 0;
    const uint64_t o_pay = raw ? up16(o_raw + raw->size()) : up16(o_idx + 4 * ((uint64_t)n_tiles + 1));
    const uint64_t total = o_pay + (ts.payload.empty() ? ts.external_len : ts.payload.size());
    out->allocate(total);
    uint8_t* s = out->data();
    std::memset(s, 0, o_pay);                       // header, metadata and padding; the payload follows
    std::memcpy(s + kMagic, "EPK1", 4);
    w16(s + kVersion, kFormatVersion);
    s[kMode] = (uint8_t)mode;
    s[kDtype] = (uint8_t)dt;
    w32(s + kRows, (uint32_t)R);
    w32(s + kCols, (uint32_t)C);
    w16(s + kTileRows, (uint32_t)tile_rows);
    s[kLayout] = (uint8_t)layout;
    w16(s + kTileColsField, kTileCols);
    w16(s + kLanesField, kLanes);
    s[kProbBits] = (uint8_t)n;
    s[kNumTables] = (uint8_t)tables.size();
    w32(s + kStep, f32bits(step));
    w32(s + kTarget, f32bits(target));
    w32(s + kNumTiles, n_tiles);
    w32(s + kNumEscapes, n_esc);
    w64(s + kOffScale, o_scale);
    w64(s + kOffQmax, o_qmax);
    w64(s + kOffTables, o_tab);
    w64(s + kOffIndex, o_idx);
    w64(s + kOffPayload, o_pay);
    w64(s + kTotalLen, total);
    w32(s + kPayloadCrc, payload_crc ? *payload_crc : crc32(ts.payload.data(), ts.payload.size()));
    if (raw) {
        w64(s + kOffRaw, o_raw);
        w32(s + kRawCrc, crc32(raw->data(), raw->size()));
        if (!raw->empty()) std::memcpy(s + o_raw, raw->data(), raw->size());
    }
    for (uint64_t r = 0; r < meta_rows; ++r) {
        w32(s + o_scale + 4 * r, f32bits(scale[r]));
        w16(s + o_qmax + 2 * r, qmax[r]);
    }
    uint8_t* p = s + o_tab;
    for (const Table& t : tables) {
        w16(p, (uint32_t)(uint16_t)(int16_t)t.lo);
        w16(p + 2, (uint32_t)t.width);
        w16(p + 4, mode == EP_MODE_LOSSY_E8 ? t.freq[kEscape] : 0);
        p += 6;
        for (int k = 0; k < t.width; ++k, p += 2) w16(p, t.freq[k]);
    }
    for (uint32_t i = 0; i <= n_tiles; ++i) w32(s + o_idx + 4 * (uint64_t)i, ts.offsets[i]);
    w32(s + kMetaCrc, meta_crc32(s, o_raw, raw ? raw->size() : 0, o_pay));
    if (!ts.payload.empty()) std::memcpy(s + o_pay, ts.payload.data(), ts.payload.size());
    return o_pay;
}

// Encode all tiles: fill(tile, tab, sym, esc) lays out one tile's symbols.
template <class Fill>
TileSet encode_tiles(int64_t n_tiles, int steps, int n, const std::vector<EncTable>& enc, bool escapes,
                     int threads, Fill fill) {
    TileSet ts;
    ts.offsets.assign(n_tiles + 1, 0);
    if (n_tiles == 0) return ts;
    const int workers = (int)std::min<int64_t>(std::max(1, threads), n_tiles);
    const int64_t per = (n_tiles + workers - 1) / workers;
    std::vector<std::vector<uint8_t>> part(workers);
    std::vector<uint64_t> tile_bytes(n_tiles);
    parallel_for(workers, workers, [&](int64_t k, int) {
        std::vector<uint8_t> tab(steps * kLanes), sym(steps * kLanes);
        std::vector<uint16_t> esc(steps * kLanes), stack;
        stack.reserve(64 * steps);
        for (int64_t t = k * per; t < std::min(n_tiles, (k + 1) * per); ++t) {
            fill(t, tab.data(), sym.data(), esc.data());
            size_t before = part[k].size();
            encode_tile(enc.data(), n, steps, tab.data(), sym.data(), esc.data(), escapes, stack, part[k]);
            tile_bytes[t] = part[k].size() - before;
        }
    });
    uint64_t acc = 0;
    for (int64_t t = 0; t < n_tiles; ++t) {
        acc += tile_bytes[t];
        ts.offsets[t + 1] = (uint32_t)(acc / 4);
    }
    ts.payload.reserve(acc);
    for (auto& p : part) ts.payload.insert(ts.payload.end(), p.begin(), p.end());
    return ts;
}

// ------------------------------------------------------------------------------ lossy
struct Quantizer {
    const void* w;
    int dt;
    int64_t R, C;
    const std::vector<float>& scale;

    // y of block (r, k) for a given step; zero outside the matrix and in zero rows
    void block_y(int64_t r, int64_t k, double delta, double* y) const {
        for (int i = 0; i < 8; ++i) {
            int64_t c = 8 * k + i;
            y[i] = (r < R && c < C && scale[r] != 0.0f) ? widen(w, dt, r * C + c) / ((double)scale[r] * delta) : 0.0;
        }
    }
};

// Payload estimate of a sample of sb blocks from its 17 windowed tables: the empirical entropy
// of every table plus 16 bits per escape, per weight.
double estimate_bits(const uint64_t (*cnt)[256], const uint64_t* totals, int64_t sb) {
    double bits = 0.0;
    for (int t = 0; t < kLossyTables; ++t) {
        const double tot = (double)totals[t];
        for (int s = 0; s < 256; ++s) {
            if (!cnt[t][s]) continue;
            const double c = (double)cnt[t][s];
            bits -= c * std::log2(c / tot);
        }
        bits += 16.0 * (double)cnt[t][kEscape];
    }
    return bits / (8.0 * (double)sb);
}

// Log-bisection of the step between max(2^-12, guard) and 64 on the estimate est(step), keeping
// the side at or under the target; guard = 2 (U + 1) / 32767 keeps every coordinate inside the
// int16 escape range (U = max |w / s_r|).
template <class Est>
float search_step(double U, double target, Est&& est) {
    const double guard = 2.0 * (U + 1.0) / 32767.0;
    double lo = std::max(std::ldexp(1.0, -12), guard), hi = 64.0, pick;
    if (est(lo) <= target) {
        pick = lo;
    } else if (est(hi) > target) {
        pick = hi;
    } else {
        for (int it = 0; it < kSearchIters; ++it) {
            double mid = std::sqrt(lo * hi);
            if (est(mid) > target) lo = mid;
            else hi = mid;
        }
        pick = hi;
    }
    float step = (float)pick;
    if ((double)step < guard) step = std::nextafter(step, INFINITY);
    return step;
}

double sampled_bpp(const Quantizer& Q, int64_t nb, int64_t sb, double delta, int threads, std::vector<Block>& blk,
                   std::vector<Hist>& hist) {
    const int64_t kb = (Q.C + 7) / 8;
    const int64_t chunk = 1024;
    parallel_for((sb + chunk - 1) / chunk, threads, [&](int64_t c, int) {
        for (int64_t i = c * chunk; i < std::min(sb, (c + 1) * chunk); ++i) {
            int64_t idx = (int64_t)(((__int128)i * nb) / sb);
            double y[8];
            Q.block_y(idx / kb, idx % kb, delta, y);
            blk[i] = nearest_e8(y);
        }
    });
    for (auto& h : hist) h.clear();
    for (int64_t i = 0; i < sb; ++i) {
        const Block& B = blk[i];
        hist[0].add(B.b);
        for (int j = 0; j < 8; ++j) hist[1 + 2 * j + B.b].add((B.q[j] - B.b) / 2);
    }
    uint64_t cnt[kLossyTables][256], totals[kLossyTables];
    for (int t = 0; t < kLossyTables; ++t) {
        int32_t lo, width;
        window_counts(hist[t], &lo, &width, cnt[t]);
        totals[t] = hist[t].total;
    }
    return estimate_bits(cnt, totals, sb);
}

ep_status encode_lossy(const void* w, int dt, int64_t R, int64_t C, const ep_encode_opts& o, int threads,
                       Bytes* out, std::string* why) {
    const int tr = o.tile_rows, n = o.prob_bits;
    const int64_t Rp = (R + tr - 1) / tr * tr, Cp = (C + kTileCols - 1) / kTileCols * kTileCols;
    const int64_t kb = Cp / 8;
    std::vector<float> scale(R, 0.0f);
    std::vector<uint16_t> qmax(R, 0);
    bool finite = true;
    // row scales (column-order fp64 sums) and the input check
    parallel_for(R, threads, [&](int64_t r, int) {
        double acc = 0.0;
        for (int64_t j = 0; j < C; ++j) {
            double v = widen(w, dt, r * C + j);
            if (!std::isfinite(v)) finite = false;
            acc += v * v;
        }
        scale[r] = C ? (float)std::sqrt(acc / (double)C) : 0.0f;
        if (!std::isfinite(scale[r])) finite = false;
    });
    if (!finite) {
        *why = "lossy input holds a non-finite value (or a row whose sum of squares overflows)";
        return EP_ERANGE;
    }
    Quantizer Q{w, dt, R, C, scale};
    float step = 1.0f;
    if (R > 0 && C > 0) {
        // U = max |w / s| over nonzero rows
        std::vector<double> umax(R, 0.0);
        parallel_for(R, threads, [&](int64_t r, int) {
            if (scale[r] == 0.0f) return;
            double m = 0.0;
            for (int64_t j = 0; j < C; ++j) m = std::max(m, std::fabs(widen(w, dt, r * C + j) / (double)scale[r]));
            umax[r] = m;
        });
        double U = 0.0;
        for (double u : umax) U = std::max(U, u);
        const int64_t nb = R * ((C + 7) / 8);
        const int64_t sb = std::min<int64_t>(nb, kSampleBlocks);
        std::vector<Block> blk(sb);
        std::vector<Hist> hist(kLossyTables);
        step = search_step(U, o.target_bpp, [&](double d) { return sampled_bpp(Q, nb, sb, d, threads, blk, hist); });
    }
    // full quantization, row-parallel, with per-worker table histograms
    std::vector<int16_t> q(Rp * Cp, 0);
    std::vector<uint8_t> coset(Rp * kb, 0);
    const int workers = (int)std::max<int64_t>(1, std::min<int64_t>(threads, std::max<int64_t>(Rp, 1)));
    std::vector<std::vector<uint32_t>> wh(workers, std::vector<uint32_t>(kLossyTables * 2 * kValueSpan, 0));
    std::atomic<bool> range_ok{true};
    parallel_for(Rp, workers, [&](int64_t r, int k) {
        uint32_t* h = wh[k].data();
        uint32_t rowmax = 0;
        for (int64_t c8 = 0; c8 < kb; ++c8) {
            double y[8];
            Q.block_y(r, c8, (double)step, y);
            Block B = nearest_e8(y);
            coset[r * kb + c8] = (uint8_t)B.b;
            h[B.b + kValueSpan] += 1;
            for (int j = 0; j < 8; ++j) {
                int32_t qv = B.q[j];
                q[r * Cp + 8 * c8 + j] = (int16_t)qv;
                int32_t x = (qv - B.b) / 2;
                if (x <= -kValueSpan || x >= kValueSpan) range_ok = false;
                else h[(1 + 2 * j + B.b) * 2 * kValueSpan + x + kValueSpan] += 1;
                if (r < R && 8 * c8 + j < C) rowmax = std::max<uint32_t>(rowmax, (uint32_t)std::abs(qv));
            }
        }
        if (r < R) qmax[r] = (uint16_t)rowmax;
    });
    if (!range_ok) {
        *why = "lattice coordinate beyond the int16 escape range";
        return EP_ERANGE;
    }
    std::vector<Table> tables(kLossyTables);
    std::vector<EncTable> enc(kLossyTables);
    for (int t = 0; t < kLossyTables; ++t) {
        Hist H;
        for (int32_t x = -kValueSpan + 1; x < kValueSpan; ++x) {
            uint64_t c = 0;
            for (int k = 0; k < workers; ++k) c += wh[k][t * 2 * kValueSpan + x + kValueSpan];
            if (c) H.add(x, c);
        }
        uint64_t cnt[256];
        window_counts(H, &tables[t].lo, &tables[t].width, cnt);
        if (!normalize_freq(cnt, n, tables[t].freq)) {
            *why = "frequency normalization failed";
            return EP_ERANGE;
        }
        make_enc_table(tables[t].freq, &enc[t]);
    }
    wh.clear();
    const int64_t tiles_c = Cp / kTileCols, n_tiles = (Rp / tr) * tiles_c;
    std::atomic<uint32_t> n_esc{0};
    TileSet ts = encode_tiles(n_tiles, 9 * tr, n, enc, true, threads,
                              [&](int64_t tile, uint8_t* tab, uint8_t* sym, uint16_t* esc) {
        const int64_t r0 = tile / tiles_c * tr, k0 = tile % tiles_c * kLanes;
        uint32_t local = 0;
        for (int bs = 0; bs < tr; ++bs)
            for (int l = 0; l < kLanes; ++l) {
                int rr, kk;
                block_of(o.layout, tr, l, bs, &rr, &kk);
                const int64_t r = r0 + rr, k = k0 + kk;
                const int b = coset[r * kb + k];
                int base = 9 * bs * kLanes + l;
                tab[base] = 0;
                sym[base] = (uint8_t)(b - tables[0].lo);
                esc[base] = 0;
                for (int j = 0; j < 8; ++j) {
                    base += kLanes;
                    const int ti = 1 + 2 * j + b;
                    const Table& T = tables[ti];
                    const int32_t x = (q[r * Cp + 8 * k + j] - b) / 2;
                    tab[base] = (uint8_t)ti;
                    if (x >= T.lo && x < T.lo + T.width) {
                        sym[base] = (uint8_t)(x - T.lo);
                        esc[base] = 0;
                    } else {
                        sym[base] = kEscape;
                        esc[base] = (uint16_t)(int16_t)x;
                        ++local;
                    }
                }
            }
        n_esc += local;
    });
    serialize(EP_MODE_LOSSY_E8, dt, R, C, tr, o.layout, n, tables, step, (float)o.target_bpp, scale, qmax, ts, n_esc.load(), out);
    return EP_OK;
}

// ------------------------------------------------------------------------------ lossless
ep_status encode_lossless(const void* w, int dt, int64_t R, int64_t C, const ep_encode_opts& o, int threads,
                          Bytes* out, std::string* why) {
    const int tr = o.tile_rows, n = o.prob_bits;
    const int P = element_bytes(dt);
    const int64_t Rp = (R + tr - 1) / tr * tr, Cp = (C + kTileCols - 1) / kTileCols * kTileCols;
    const uint8_t* src = static_cast<const uint8_t*>(w);
    auto element = [&](int64_t r, int64_t c) -> uint32_t {
        if (r >= R || c >= C) return 0;
        const uint8_t* p = src + (size_t)(r * C + c) * P;
        uint32_t v = 0;
        for (int k = P - 1; k >= 0; --k) v = v << 8 | p[k];
        return v;
    };
    const int workers = (int)std::max<int64_t>(1, std::min<int64_t>(threads, std::max<int64_t>(Rp, 1)));
    std::vector<std::vector<uint64_t>> wh(workers, std::vector<uint64_t>(4 * 256, 0));
    parallel_for(Rp, workers, [&](int64_t r, int k) {
        uint64_t* h = wh[k].data();
        for (int64_t c = 0; c < Cp; ++c) {
            uint32_t v = element(r, c);
            for (int p = 0; p < P; ++p) h[p * 256 + (v >> (8 * (P - 1 - p)) & 0xFF)] += 1;
        }
    });
    std::vector<Table> tables(P);
    std::vector<EncTable> enc(P);
    for (int p = 0; p < P; ++p) {
        uint64_t cnt[256] = {};
        for (int k = 0; k < workers; ++k)
            for (int s = 0; s < 256; ++s) cnt[s] += wh[k][p * 256 + s];
        tables[p].lo = 0;
        tables[p].width = 256;
        if (!normalize_freq(cnt, n, tables[p].freq)) {
            *why = "frequency normalization failed";
            return EP_ERANGE;
        }
        make_enc_table(tables[p].freq, &enc[p]);
    }
    const int64_t tiles_c = Cp / kTileCols, n_tiles = (Rp / tr) * tiles_c;
    const int steps = tr * 8 * P;
    TileSet ts = encode_tiles(n_tiles, steps, n, enc, false, threads,
                              [&](int64_t tile, uint8_t* tab, uint8_t* sym, uint16_t*) {
        const int64_t r0 = tile / tiles_c * tr, c0 = tile % tiles_c * kTileCols;
        for (int rr = 0; rr < tr; ++rr)
            for (int e = 0; e < 8; ++e)
                for (int l = 0; l < kLanes; ++l) {
                    const uint32_t v = element(r0 + rr, c0 + 8 * l + e);
                    for (int p = 0; p < P; ++p) {
                        const int idx = ((rr * 8 + e) * P + p) * kLanes + l;
                        tab[idx] = (uint8_t)p;
                        sym[idx] = (uint8_t)(v >> (8 * (P - 1 - p)));
                    }
                }
    });
    (void)why;
    serialize(EP_MODE_LOSSLESS, dt, R, C, tr, 0, n, tables, 0.0f, 0.0f, {}, {}, ts, 0, out);
    return EP_OK;
}

// ------------------------------------------------------------------------------ exponent-coded BF16
// Lossless BF16 as the guide's DFloat11 config ("Choose a compression contract"), read after the
// published DFloat11 split: the exponent byte of every element is coded by the tile rANS (one
// table, one step per element, steps row -> element, lane l on columns 8l..8l+7), and sign and
// mantissa are stored uncoded as (sign << 7) | mantissa in a raw plane [Rp][Cp] shaped like the
// zero-padded matrix, so that the decoder reads each lane's 8 bytes of a row with one load.
ep_status encode_lossless_exp(const void* w, int64_t R, int64_t C, const ep_encode_opts& o, int threads,
                              Bytes* out, std::string* why) {
    const int tr = o.tile_rows, n = o.prob_bits;
    const int64_t Rp = (R + tr - 1) / tr * tr, Cp = (C + kTileCols - 1) / kTileCols * kTileCols;
    const uint16_t* src = static_cast<const uint16_t*>(w);
    auto element = [&](int64_t r, int64_t c) -> uint32_t { return r < R && c < C ? src[r * C + c] : 0u; };
    std::vector<uint8_t> raw((size_t)(Rp * Cp));
    const int workers = (int)std::max<int64_t>(1, std::min<int64_t>(threads, std::max<int64_t>(Rp, 1)));
    std::vector<std::vector<uint64_t>> wh(workers, std::vector<uint64_t>(256, 0));
    parallel_for(Rp, workers, [&](int64_t r, int k) {
        uint64_t* h = wh[k].data();
        for (int64_t c = 0; c < Cp; ++c) {
            const uint32_t v = element(r, c);
            h[v >> 7 & 0xFF] += 1;
            raw[(size_t)(r * Cp + c)] = (uint8_t)((v >> 8 & 0x80u) | (v & 0x7Fu));
        }
    });
    std::vector<Table> tables(1);
    std::vector<EncTable> enc(1);
    uint64_t cnt[256] = {};
    for (int k = 0; k < workers; ++k)
        for (int s = 0; s < 256; ++s) cnt[s] += wh[k][s];
    tables[0].lo = 0;
    tables[0].width = 256;
    if (!normalize_freq(cnt, n, tables[0].freq)) {
        *why = "frequency normalization failed";
        return EP_ERANGE;
    }
    make_enc_table(tables[0].freq, &enc[0]);
    const int64_t tiles_c = Cp / kTileCols, n_tiles = (Rp / tr) * tiles_c;
    TileSet ts = encode_tiles(n_tiles, tr * 8, n, enc, false, threads,
                              [&](int64_t tile, uint8_t* tab, uint8_t* sym, uint16_t*) {
        const int64_t r0 = tile / tiles_c * tr, c0 = tile % tiles_c * kTileCols;
        for (int rr = 0; rr < tr; ++rr)
            for (int e = 0; e < 8; ++e)
                for (int l = 0; l < kLanes; ++l) {
                    const int idx = (rr * 8 + e) * kLanes + l;
                    tab[idx] = 0;
                    sym[idx] = (uint8_t)(element(r0 + rr, c0 + 8 * l + e) >> 7);
                }
    });
    serialize(EP_MODE_LOSSLESS_EXP, EP_BF16, R, C, tr, 0, n, tables, 0.0f, 0.0f, {}, {}, ts, 0, out, &raw);
    return EP_OK;
}

}  // namespace

bool normalize_frequencies(const uint64_t cnt[256], int n, uint32_t f[256]) { return normalize_freq(cnt, n, f); }

double sample_estimate(const uint64_t (*cnt)[256], const uint64_t* totals, int64_t sb) {
    return estimate_bits(cnt, totals, sb);
}

float choose_step(double U, double target, const std::function<double(double)>& est) {
    return search_step(U, target, est);
}

uint64_t serialize_lossy(int dt, int64_t R, int64_t C, int tile_rows, int layout, int n, const std::vector<Table>& tables,
                         float step, float target, const std::vector<float>& scale, const std::vector<uint16_t>& qmax,
                         uint64_t payload_len, std::vector<uint32_t>&& offsets, uint32_t n_esc, uint32_t payload_crc,
                         Bytes* out) {
    TileSet ts;
    ts.offsets = std::move(offsets);
    ts.external_len = payload_len;
    return serialize(EP_MODE_LOSSY_E8, dt, R, C, tile_rows, layout, n, tables, step, target, scale, qmax, ts, n_esc, out,
                     nullptr, &payload_crc);
}

ep_status encode(const void* w, int dt, int64_t R, int64_t C, const ep_encode_opts& o, Bytes* out,
                 std::string* why) {
    int threads = o.n_threads > 0 ? o.n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
    threads = std::min(threads, 64);
    if (o.mode == EP_MODE_LOSSY_E8) return encode_lossy(w, dt, R, C, o, threads, out, why);
    if (o.mode == EP_MODE_LOSSLESS_EXP) return encode_lossless_exp(w, R, C, o, threads, out, why);
    return encode_lossless(w, dt, R, C, o, threads, out, why);
}

}  // namespace ep
