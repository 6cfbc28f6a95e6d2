/*
 * EPK1 oracle: a plain, slow, scalar CPU encoder/decoder for entropy-coded E8 weight streams.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg load this file's library. The product library shares no code, header, table or
 * helper with it, and neither side includes or links the other.
 *
 * Sources. The method is described by three pages, cited below by short tags:
 *   [A]  "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates"
 *        (paper listing 2609.34185v1), Abstract.
 *   [G]  "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", by section.
 *   [P]  "EntroPack 開源：模型壓縮不必只選 4 位元，如何配合顯示記憶體預算？", by section.
 * [A] names the steps: rows scaled to unit size and quantized to the E8 lattice, a conditional
 * model of the lattice coordinates, a step size picked from a size estimate on a sample, entropy
 * coding in tiles that decode on their own, and reconstruction into BF16/FP16/FP8/INT8 containers.
 * Every finer rule (norm, tie-breaking, alphabet, rANS parameters, tile geometry, byte layout,
 * rounding) is a reading where the pages are silent; each is marked "reading:" where it is used.
 *
 * Published algorithms restated from their mathematics (no code taken from anywhere):
 *   - nearest point of D_n and of the coset union D_n u (D_n + 1/2): Conway & Sloane, "Fast
 *     quantizing and decoding algorithms for lattice quantizers and codes", IEEE Trans. IT 1982;
 *   - range-variant asymmetric numeral systems (rANS): Duda, arXiv:1311.2540; interleaved
 *     states: Giesen, arXiv:1402.3392;
 *   - CRC-32 (IEEE 802.3, reflected polynomial 0xEDB88320).
 *
 * Parity status of each part (what pins it is listed in the test files):
 *   E8 nearest point       pinned: brute-force search, lattice invariants, second moment of E8
 *   row scale              pinned: closed form
 *   table normalization    pinned: invariants (sum, support), single-symbol case
 *   table windows          pinned: brute force over every window start (constructed ties, best
 *                          window at either end of the range, random heavy tails) and the tables
 *                          of real streams against histograms of their decoded coordinates
 *   lossy tile layouts     pinned: an independent Python reader of the stream bytes gives the
 *                          decoder's coordinates and cosets (escapes, ragged shapes, 32-row tiles,
 *                          both layouts); both layouts decode to the same weights
 *   rANS tile coder        pinned: exact round trips, final state, an independent Python decoder
 *   rate search            pinned: monotone estimate, Gaussian closed form, |payload - target|
 *   containers             pinned: library casts (torch CPU) for BF16/FP16/FP8, integer closed form
 *   lossless byte planes   pinned: bit-exact round trips on special values
 *   exponent-coded BF16    pinned: bit-exact round trips on special values, raw plane closed
 *                          form, exponent table from the exponent histogram
 *   accounting             pinned: identity actual_bpp = 8 * bytes / (R * C)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ECORRUPT (-2)
#define OR_EUNSUPPORTED (-3)
#define OR_ERANGE (-4)
#define OR_ENOMEM (-6)

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_F8E4M3 = 3, DT_I8 = 4, DT_U8 = 5 };
enum { MODE_LOSSY = 0, MODE_LOSSLESS = 1, MODE_LOSSLESS_EXP = 2 };

#define LANES 32
#define TILE_COLS 256
#define HEADER_BYTES 128
#define ESC_SYM 255
#define RANS_L 65536u          /* reading: 32-bit state, lower bound 2^16, 16-bit I/O words */
#define N_LOSSY_TABLES 17      /* reading: coset table + 8 positions x 2 cosets */
#define SAMPLE_BLOCKS 65536    /* reading: rate-search sample size */
#define SEARCH_ITERS 48

/* ------------------------------------------------------------------------------------------ */
/* little-endian byte access                                                                   */
/* ------------------------------------------------------------------------------------------ */
static void put16(uint8_t* p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t* p, uint32_t v) {
    for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static void put64(uint8_t* p, uint64_t v) {
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get32(const uint8_t* p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static uint64_t get64(const uint8_t* p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
    return v;
}
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* CRC-32 (IEEE), bit by bit from the reflected polynomial; crc32_more continues a register over
   further bytes (start 0xFFFFFFFF, final value complemented), so that disjoint ranges can be
   checked as one message. */
static uint32_t crc32_more(uint32_t c, const uint8_t* p, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        c ^= p[i];
        for (int k = 0; k < 8; ++k) c = (c & 1u) ? (c >> 1) ^ 0xEDB88320u : (c >> 1);
    }
    return c;
}
static uint32_t crc32_ieee(const uint8_t* p, size_t n) { return crc32_more(0xFFFFFFFFu, p, n) ^ 0xFFFFFFFFu; }

/* ------------------------------------------------------------------------------------------ */
/* number formats, from their definitions                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Round a finite value to a binary floating-point format with p significand bits (hidden bit
 * included) and minimum normal exponent emin, to nearest with ties to even, keeping subnormals.
 * No exponent upper limit is applied here; callers treat overflow. */
static double round_to_format(double v, int p, int emin) {
    if (v == 0.0) return v;
    int e;
    frexp(fabs(v), &e);            /* |v| = m * 2^e with m in [0.5, 1): floor(log2|v|) = e - 1 */
    int ex = e - 1;
    if (ex < emin) ex = emin;      /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, ex - (p - 1));
    return nearbyint(v / quantum) * quantum;   /* default rounding mode: nearest, ties to even */
}

/* decode a stored source element to double (exact for every supported type) */
static double bf16_bits_to_double(uint32_t h) { return (double)f32_from_bits(h << 16); }
static double f16_bits_to_double(uint32_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

/* IEEE binary32 -> bfloat16 (8-bit exponent, 7 stored mantissa bits), round to nearest even. */
uint16_t or_f32_to_bf16(float f) {
    uint32_t u = bits_from_f32(f);
    uint32_t sign = u & 0x80000000u;
    if (isnan(f)) return (uint16_t)((sign >> 16) | 0x7FC0u);
    if (isinf(f)) return (uint16_t)((sign >> 16) | 0x7F80u);
    double r = round_to_format((double)f, 8, -126);
    double maxv = ldexp(2.0 - ldexp(1.0, -7), 127);
    if (fabs(r) > maxv) return (uint16_t)((sign >> 16) | 0x7F80u);
    uint32_t rb = bits_from_f32((float)r);     /* exact: a bfloat16 value is a binary32 value */
    return (uint16_t)(((rb >> 16) & 0x7FFFu) | (sign >> 16));
}

/* IEEE binary32 -> binary16, round to nearest even, subnormals kept, overflow to infinity. */
uint16_t or_f32_to_f16(float f) {
    uint32_t sign = (bits_from_f32(f) >> 16) & 0x8000u;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double r = fabs(round_to_format((double)f, 11, -14));
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (r == 0.0) return (uint16_t)sign;
    int e;
    frexp(r, &e);
    int ex = e - 1;
    if (ex < -14) return (uint16_t)(sign | (uint32_t)(r / ldexp(1.0, -24)));   /* subnormal */
    uint32_t mant = (uint32_t)((r / ldexp(1.0, ex) - 1.0) * 1024.0);
    return (uint16_t)(sign | ((uint32_t)(ex + 15) << 10) | mant);
}

/* IEEE binary32 -> OCP FP8 E4M3FN (bias 7, largest finite 448, no infinities), round to nearest
 * even, then saturate to +-448 (reading: saturating cast, as a weight container has no use for
 * NaN on overflow). */
uint8_t or_f32_to_e4m3(float f) {
    uint32_t sign = (bits_from_f32(f) >> 24) & 0x80u;
    if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
    double r = isinf(f) ? 448.0 : fabs(round_to_format((double)f, 4, -6));
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return (uint8_t)sign;
    int e;
    frexp(r, &e);
    int ex = e - 1;
    if (ex < -6) return (uint8_t)(sign | (uint32_t)(r / ldexp(1.0, -9)));       /* subnormal */
    uint32_t mant = (uint32_t)((r / ldexp(1.0, ex) - 1.0) * 8.0);
    return (uint8_t)(sign | ((uint32_t)(ex + 7) << 3) | mant);
}

static int elem_bytes(int dt) {
    switch (dt) {
        case DT_F32: return 4;
        case DT_BF16: case DT_F16: return 2;
        case DT_F8E4M3: case DT_I8: case DT_U8: return 1;
        default: return 0;
    }
}

/* value of element i of a lossy-mode source (fp32, bf16 or fp16), widened exactly */
static double src_value(const void* w, int dt, int64_t i) {
    if (dt == DT_F32) return (double)((const float*)w)[i];
    if (dt == DT_BF16) return bf16_bits_to_double(((const uint16_t*)w)[i]);
    return f16_bits_to_double(((const uint16_t*)w)[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* E8 nearest point. [A, Abstract]: normalized rows are quantized on the E8 lattice.           */
/* Reading: E8 = D8 u (D8 + 1/2), unimodular scaling, lattice spacing set by the step.          */
/* ------------------------------------------------------------------------------------------ */

/* Nearest point of D8 = { a in Z^8 : sum(a) even } to v (Conway & Sloane): round every coordinate
 * half-to-even; if the coordinate sum is odd, move the coordinate with the largest rounding error
 * (lowest index on ties) one step towards v (upwards when its error is zero). */
static void d8_nearest(const double v[8], double a[8]) {
    long sum = 0;
    for (int i = 0; i < 8; ++i) {
        a[i] = nearbyint(v[i]);
        sum += (long)a[i];
    }
    if (sum & 1) {
        int k = 0;
        double worst = -1.0;
        for (int i = 0; i < 8; ++i) {
            double err = fabs(v[i] - a[i]);
            if (err > worst) { worst = err; k = i; }
        }
        a[k] += (v[k] >= a[k]) ? 1.0 : -1.0;
    }
}

/* Nearest E8 point: the closer of the D8 candidate and the (D8 + 1/2) candidate; equal distances
 * go to the integer coset. Output: doubled coordinates q = 2p (all even for coset 0, all odd for
 * coset 1) and the coset bit. */
static void e8_nearest(const double y[8], int32_t q[8], int* coset) {
    double c0[8], c1[8], t[8];
    d8_nearest(y, c0);
    for (int i = 0; i < 8; ++i) t[i] = y[i] - 0.5;
    d8_nearest(t, c1);
    for (int i = 0; i < 8; ++i) c1[i] += 0.5;
    double d0 = 0.0, d1 = 0.0;
    for (int i = 0; i < 8; ++i) {
        d0 += (y[i] - c0[i]) * (y[i] - c0[i]);
        d1 += (y[i] - c1[i]) * (y[i] - c1[i]);
    }
    int b = (d0 <= d1) ? 0 : 1;
    for (int i = 0; i < 8; ++i) q[i] = (int32_t)(2.0 * (b ? c1[i] : c0[i]));
    *coset = b;
}

void or_e8_nearest_batch(const double* y, int64_t n, int32_t* q, int32_t* coset) {
    for (int64_t k = 0; k < n; ++k) {
        int b;
        e8_nearest(y + 8 * k, q + 8 * k, &b);
        coset[k] = b;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Row scale. [A, Abstract]: rows are normalized. Reading: unit-RMS rows; the sum of squares over */
/* the real columns is accumulated in fp64 in column order, divided by C, square-rooted in fp64  */
/* and rounded once to fp32.                                                                    */
/* ------------------------------------------------------------------------------------------ */
static float row_scale(const void* w, int dt, int64_t r, int64_t C) {
    double acc = 0.0;
    if (C == 0) return 0.0f;
    for (int64_t j = 0; j < C; ++j) {
        double v = src_value(w, dt, r * C + j);
        acc += v * v;
    }
    return (float)sqrt(acc / (double)C);
}

/* ------------------------------------------------------------------------------------------ */
/* Symbol model. [A, Abstract]: the lattice coordinates are coded with a conditional model.     */
/* Reading: 17 static tables per tensor: table 0 codes the coset bit; table 1 + 2j + b codes    */
/* coordinate j of a block in coset b. Each table keeps a window of at most 255 consecutive     */
/* values; values outside it are coded as symbol 255 (escape) followed by a raw 16-bit word.     */
/* ------------------------------------------------------------------------------------------ */
#define HIST_SPAN 65536
#define HIST_OFF 32768

typedef struct {
    uint64_t* hist;        /* [HIST_SPAN] counts of coordinate value x (index x + HIST_OFF) */
    uint64_t total;
    int32_t vmin, vmax;
} value_hist;

typedef struct {
    int32_t lo;            /* first value of the window */
    int32_t S;             /* window width (1..255 lossy, 256 lossless) */
    uint64_t cnt[256];     /* symbol counts: 0..S-1 in-window, 255 escape */
    uint32_t f[256];       /* normalized frequencies, sum = 2^n */
    uint32_t c[256];       /* cumulative frequencies in symbol order */
} sym_table;

static void hist_reset(value_hist* h) {
    memset(h->hist, 0, sizeof(uint64_t) * HIST_SPAN);
    h->total = 0;
    h->vmin = INT32_MAX;
    h->vmax = INT32_MIN;
}
static void hist_add(value_hist* h, int32_t x) {
    h->hist[x + HIST_OFF]++;
    h->total++;
    if (x < h->vmin) h->vmin = x;
    if (x > h->vmax) h->vmax = x;
}

/* Window choice: the whole observed range when it has at most 255 values, else the 255-wide
 * window holding the most occurrences (smallest start on ties). */
static void choose_window(const value_hist* h, sym_table* T) {
    memset(T->cnt, 0, sizeof T->cnt);
    if (h->total == 0) { T->lo = 0; T->S = 1; return; }
    int32_t range = h->vmax - h->vmin + 1;
    if (range <= 255) {
        T->lo = h->vmin;
        T->S = range;
    } else {
        uint64_t best = 0, sum = 0;
        int32_t best_lo = h->vmin;
        for (int32_t x = h->vmin; x < h->vmin + 255; ++x) sum += h->hist[x + HIST_OFF];
        best = sum;
        for (int32_t lo = h->vmin + 1; lo + 254 <= h->vmax; ++lo) {
            sum += h->hist[lo + 254 + HIST_OFF];
            sum -= h->hist[lo - 1 + HIST_OFF];
            if (sum > best) { best = sum; best_lo = lo; }
        }
        T->lo = best_lo;
        T->S = 255;
    }
    uint64_t inside = 0;
    for (int32_t s = 0; s < T->S; ++s) {
        T->cnt[s] = h->hist[T->lo + s + HIST_OFF];
        inside += T->cnt[s];
    }
    T->cnt[ESC_SYM] = h->total - inside;
}

/* The window rule on its own, for its pins: the histogram of n coordinate values (each within
 * [-32768, 32767]), then choose_window; returns the window start, width and escape count. */
int or_choose_window(const int32_t* values, int64_t n, int32_t* lo, int32_t* S, uint64_t* n_escaped) {
    value_hist h;
    sym_table T;
    h.hist = (uint64_t*)malloc(sizeof(uint64_t) * HIST_SPAN);
    if (!h.hist) return OR_ENOMEM;
    hist_reset(&h);
    for (int64_t i = 0; i < n; ++i) {
        if (values[i] < -HIST_OFF || values[i] >= HIST_SPAN - HIST_OFF) { free(h.hist); return OR_EINVAL; }
        hist_add(&h, values[i]);
    }
    choose_window(&h, &T);
    *lo = T.lo;
    *S = T.S;
    *n_escaped = T.cnt[ESC_SYM];
    free(h.hist);
    return OR_OK;
}

/* Normalization of counts to frequencies summing to M = 2^n (reading):
 *   f_s = max(1, floor(c_s M / T)) for every present symbol, 0 otherwise;
 *   a shortfall is added to the most frequent symbol (lowest index on ties);
 *   an excess is removed one unit at a time from the symbol with the largest f among those
 *   with f > 1 (lowest index on ties).
 * An empty table gets f_0 = M. */
int or_normalize(const uint64_t* cnt, int prob_bits, uint32_t* f) {
    uint32_t M = 1u << prob_bits;
    uint64_t T = 0;
    for (int s = 0; s < 256; ++s) T += cnt[s];
    memset(f, 0, 256 * sizeof(uint32_t));
    if (T == 0) { f[0] = M; return OR_OK; }
    uint64_t sum = 0;
    for (int s = 0; s < 256; ++s) {
        if (cnt[s] == 0) continue;
        uint64_t v = (cnt[s] * (uint64_t)M) / T;
        f[s] = (uint32_t)(v < 1 ? 1 : v);
        sum += f[s];
    }
    if (sum < M) {
        int top = 0;
        for (int s = 1; s < 256; ++s)
            if (cnt[s] > cnt[top]) top = s;
        f[top] += (uint32_t)(M - sum);
        sum = M;
    }
    while (sum > M) {
        int top = -1;
        for (int s = 0; s < 256; ++s)
            if (f[s] > 1 && (top < 0 || f[s] > f[top])) top = s;
        if (top < 0) return OR_ERANGE;     /* more present symbols than M: cannot happen for n >= 8 */
        f[top] -= 1;
        sum -= 1;
    }
    return OR_OK;
}

static void cumulate(const uint32_t* f, uint32_t* c) {
    uint32_t acc = 0;
    for (int s = 0; s < 256; ++s) { c[s] = acc; acc += f[s]; }
}

/* ------------------------------------------------------------------------------------------ */
/* rANS tile coder. [A, Abstract]: entropy coding in tiles that decode on their own.            */
/* Reading: every tile has 32 interleaved states (Giesen). Each step codes one symbol per lane. */
/* Decoding step t: every lane decodes its symbol; lanes whose state fell below L then take one */
/* refill word each, in ascending lane order; then lanes that decoded the escape symbol take    */
/* one raw word each, in ascending lane order. The encoder runs the steps backwards and stacks  */
/* words in the mirror order, so that the reversed stack is the decoder's reading order.        */
/* Tile bytes: 32 little-endian u32 final encoder states (lane 0 first), the u16 words, and one */
/* zero u16 when the word count is odd.                                                         */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    uint32_t f[256], c[256];
    uint8_t* lut;          /* [2^n] slot -> symbol */
} rans_table;

static int rans_table_init(rans_table* t, const uint32_t* f, int n) {
    uint32_t M = 1u << n;
    memcpy(t->f, f, sizeof t->f);
    cumulate(t->f, t->c);
    t->lut = (uint8_t*)malloc(M);
    if (!t->lut) return OR_ENOMEM;
    for (int s = 0; s < 256; ++s)
        for (uint32_t k = t->c[s]; k < t->c[s] + t->f[s]; ++k) t->lut[k] = (uint8_t)s;
    return OR_OK;
}
static void rans_table_free(rans_table* t) { free(t->lut); t->lut = NULL; }

/* Encode one tile of n_steps x 32 symbols. tab/sym/esc are indexed [step * 32 + lane];
 * esc is read where the symbol equals esc_sym (esc_sym < 0: no escapes). stack must hold
 * 64 * n_steps words. Writes the tile bytes to out (capacity 128 + 4 * 32 * n_steps + 4) and
 * returns the byte count. */
static size_t rans_encode_tile(const rans_table* tabs, int n, int n_steps, const uint8_t* tab,
                               const uint8_t* sym, const uint16_t* esc, int esc_sym,
                               uint16_t* stack, uint8_t* out) {
    uint32_t M = 1u << n;
    uint32_t x[LANES];
    size_t sp = 0;
    for (int l = 0; l < LANES; ++l) x[l] = RANS_L;
    for (int t = n_steps - 1; t >= 0; --t) {
        uint16_t R[LANES];
        int has[LANES];
        for (int l = 0; l < LANES; ++l) {
            const rans_table* T = &tabs[tab[t * LANES + l]];
            uint32_t s = sym[t * LANES + l];
            uint64_t f = T->f[s];
            uint64_t xmax = (uint64_t)((RANS_L >> n) << 16) * f;
            uint64_t v = x[l];
            has[l] = 0;
            if (v >= xmax) {
                R[l] = (uint16_t)(v & 0xFFFFu);
                v >>= 16;
                has[l] = 1;
            }
            v = (v / f) * M + (v % f) + T->c[s];
            x[l] = (uint32_t)v;
        }
        for (int l = LANES - 1; l >= 0; --l)
            if (esc_sym >= 0 && sym[t * LANES + l] == (uint8_t)esc_sym) stack[sp++] = esc[t * LANES + l];
        for (int l = LANES - 1; l >= 0; --l)
            if (has[l]) stack[sp++] = R[l];
    }
    for (int l = 0; l < LANES; ++l) put32(out + 4 * l, x[l]);
    size_t pos = 4 * LANES;
    for (size_t i = 0; i < sp; ++i, pos += 2) put16(out + pos, stack[sp - 1 - i]);
    if (sp & 1) { put16(out + pos, 0); pos += 2; }
    return pos;
}

/* Table choice for the next decoding step, given the symbols decoded so far. */
typedef void (*table_fn)(void* ctx, int step, uint8_t tab_out[LANES]);

/* Decode one tile. sym_out/esc_out are [n_steps * 32]. final_states (optional) receives the
 * states after the last step. Returns OR_OK, or OR_ECORRUPT when the words run out, the tile
 * length disagrees with the words consumed, or a final state differs from L. */
static int rans_decode_tile(const rans_table* tabs, int n, int n_steps, const uint8_t* tile,
                            size_t tile_len, table_fn next_tables, void* ctx, int esc_sym,
                            uint8_t* sym_out, uint16_t* esc_out, uint32_t* final_states) {
    uint32_t M = 1u << n;
    uint32_t x[LANES];
    if (tile_len < 4 * LANES) return OR_ECORRUPT;
    for (int l = 0; l < LANES; ++l) x[l] = get32(tile + 4 * l);
    size_t pos = 4 * LANES;
    for (int t = 0; t < n_steps; ++t) {
        uint8_t tab[LANES];
        next_tables(ctx, t, tab);
        for (int l = 0; l < LANES; ++l) {
            const rans_table* T = &tabs[tab[l]];
            uint32_t slot = x[l] & (M - 1);
            uint32_t s = T->lut[slot];
            x[l] = T->f[s] * (x[l] >> n) + slot - T->c[s];
            sym_out[t * LANES + l] = (uint8_t)s;
            esc_out[t * LANES + l] = 0;
        }
        for (int l = 0; l < LANES; ++l) {
            if (x[l] < RANS_L) {
                if (pos + 2 > tile_len) return OR_ECORRUPT;
                x[l] = (x[l] << 16) | get16(tile + pos);
                pos += 2;
            }
        }
        if (esc_sym >= 0) {
            for (int l = 0; l < LANES; ++l) {
                if (sym_out[t * LANES + l] == (uint8_t)esc_sym) {
                    if (pos + 2 > tile_len) return OR_ECORRUPT;
                    esc_out[t * LANES + l] = (uint16_t)get16(tile + pos);
                    pos += 2;
                }
            }
        }
    }
    size_t words = (pos - 4 * LANES) / 2;
    size_t expect = 4 * LANES + 2 * words + ((words & 1) ? 2 : 0);
    if (expect != tile_len) return OR_ECORRUPT;
    for (int l = 0; l < LANES; ++l) {
        if (final_states) final_states[l] = x[l];
        if (x[l] != RANS_L) return OR_ECORRUPT;
    }
    return OR_OK;
}

/* Generic tile codec entry points used by the tests (tables given as raw frequencies
 * [n_tables][256] summing to 2^n; table choice per step and lane given up front). */
typedef struct { const uint8_t* tab; } fixed_tab_ctx;
static void fixed_tables(void* ctx, int step, uint8_t out[LANES]) {
    const fixed_tab_ctx* c = (const fixed_tab_ctx*)ctx;
    memcpy(out, c->tab + (size_t)step * LANES, LANES);
}

int or_rans_encode(int n_tables, const uint32_t* freqs, int prob_bits, int n_steps,
                   const uint8_t* tab, const uint8_t* sym, const uint16_t* esc, int esc_sym,
                   uint8_t* out, size_t cap, size_t* out_len) {
    rans_table* T = (rans_table*)calloc((size_t)n_tables, sizeof(rans_table));
    uint16_t* stack = (uint16_t*)malloc(sizeof(uint16_t) * 64 * (size_t)n_steps + 2);
    int rc = OR_OK;
    if (!T || !stack) { rc = OR_ENOMEM; goto done; }
    for (int i = 0; i < n_tables; ++i)
        if ((rc = rans_table_init(&T[i], freqs + 256 * i, prob_bits)) != OR_OK) goto done;
    for (int k = 0; k < n_steps * LANES; ++k)
        if (tab[k] >= n_tables || T[tab[k]].f[sym[k]] == 0) { rc = OR_EINVAL; goto done; }
    if (cap < 4 * LANES + 4 * (size_t)LANES * n_steps + 4) { rc = OR_EINVAL; goto done; }
    *out_len = rans_encode_tile(T, prob_bits, n_steps, tab, sym, esc, esc_sym, stack, out);
done:
    if (T) for (int i = 0; i < n_tables; ++i) rans_table_free(&T[i]);
    free(T);
    free(stack);
    return rc;
}

int or_rans_decode(int n_tables, const uint32_t* freqs, int prob_bits, int n_steps,
                   const uint8_t* tab, int esc_sym, const uint8_t* tile, size_t tile_len,
                   uint8_t* sym_out, uint16_t* esc_out, uint32_t* final_states) {
    rans_table* T = (rans_table*)calloc((size_t)n_tables, sizeof(rans_table));
    int rc = OR_OK;
    if (!T) return OR_ENOMEM;
    for (int i = 0; i < n_tables; ++i)
        if ((rc = rans_table_init(&T[i], freqs + 256 * i, prob_bits)) != OR_OK) goto done;
    fixed_tab_ctx ctx = { tab };
    rc = rans_decode_tile(T, prob_bits, n_steps, tile, tile_len, fixed_tables, &ctx, esc_sym,
                          sym_out, esc_out, final_states);
done:
    for (int i = 0; i < n_tables; ++i) rans_table_free(&T[i]);
    free(T);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Quantization of a whole matrix. Reading: blocks are 8 consecutive columns of one row; the    */
/* matrix is zero-padded to whole tiles; y = w / (s_r * step) in fp64; zero rows give q = 0.    */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    int64_t R, C, Rp, Cp;
    int tile_rows;
    float* scale;          /* [R] */
    uint16_t* qmax;        /* [R] */
    int16_t* q;            /* [Rp * Cp] doubled coordinates */
    uint8_t* coset;        /* [Rp * Cp / 8] */
} quantized;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* the 8 input values of block (r, k) after scaling by 1 / (s * delta); zero outside the matrix */
static void block_y(const void* w, int dt, int64_t R, int64_t C, const float* scale, double delta,
                    int64_t r, int64_t k, double y[8]) {
    for (int i = 0; i < 8; ++i) {
        int64_t col = 8 * k + i;
        if (r >= R || col >= C || scale[r] == 0.0f) { y[i] = 0.0; continue; }
        y[i] = src_value(w, dt, r * C + col) / ((double)scale[r] * delta);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Sampled rate estimate and step search. [A, Abstract]: the step size comes from a storage     */
/* estimate on a sample, so the full stream is encoded once.                                    */
/* Reading: S_b = min(NB, 65536) blocks at indices floor(i NB / S_b) of the row-major real      */
/* blocks; est = (sum over tables and symbols of -c log2(c / T) + 16 per escape) / (8 S_b) bits */
/* per weight; the step is bisected in log2 between max(2^-12, 2 (U + 1) / 32767) and 64 for 48 */
/* iterations, keeping the end whose estimate is at or below the target.                        */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const void* w; int dt; int64_t R, C;
    const float* scale;
    int64_t nb, sb;
    value_hist h[N_LOSSY_TABLES];
} estimator;

static double estimate_bpp(estimator* E, double delta) {
    for (int t = 0; t < N_LOSSY_TABLES; ++t) hist_reset(&E->h[t]);
    int64_t kb = ceil_div(E->C, 8);
    for (int64_t i = 0; i < E->sb; ++i) {
        int64_t idx = (int64_t)(((__int128)i * E->nb) / E->sb);
        int64_t r = idx / kb, k = idx % kb;
        double y[8];
        int32_t q[8];
        int b;
        block_y(E->w, E->dt, E->R, E->C, E->scale, delta, r, k, y);
        e8_nearest(y, q, &b);
        hist_add(&E->h[0], b);
        for (int j = 0; j < 8; ++j) hist_add(&E->h[1 + 2 * j + b], (q[j] - b) / 2);
    }
    double bits = 0.0;
    for (int t = 0; t < N_LOSSY_TABLES; ++t) {
        sym_table T;
        choose_window(&E->h[t], &T);
        double tot = (double)E->h[t].total;
        for (int s = 0; s < 256; ++s) {
            if (T.cnt[s] == 0) continue;
            double c = (double)T.cnt[s];
            bits -= c * log2(c / tot);
        }
        bits += 16.0 * (double)T.cnt[ESC_SYM];
    }
    return bits / (8.0 * (double)E->sb);
}

static double max_abs_normalized(const void* w, int dt, int64_t R, int64_t C, const float* scale) {
    double U = 0.0;
    for (int64_t r = 0; r < R; ++r) {
        if (scale[r] == 0.0f) continue;
        for (int64_t j = 0; j < C; ++j) {
            double v = fabs(src_value(w, dt, r * C + j) / (double)scale[r]);
            if (v > U) U = v;
        }
    }
    return U;
}

static int estimator_init(estimator* E, const void* w, int dt, int64_t R, int64_t C, const float* scale) {
    E->w = w; E->dt = dt; E->R = R; E->C = C; E->scale = scale;
    E->nb = R * ceil_div(C, 8);
    E->sb = E->nb < SAMPLE_BLOCKS ? E->nb : SAMPLE_BLOCKS;
    for (int t = 0; t < N_LOSSY_TABLES; ++t) {
        E->h[t].hist = (uint64_t*)malloc(sizeof(uint64_t) * HIST_SPAN);
        if (!E->h[t].hist) return OR_ENOMEM;
    }
    return OR_OK;
}
static void estimator_free(estimator* E) {
    for (int t = 0; t < N_LOSSY_TABLES; ++t) free(E->h[t].hist);
}

static float select_step(estimator* E, double target, double U) {
    double guard = 2.0 * (U + 1.0) / 32767.0;
    double lo = ldexp(1.0, -12);
    if (guard > lo) lo = guard;
    double hi = 64.0, chosen;
    if (estimate_bpp(E, lo) <= target) chosen = lo;
    else if (estimate_bpp(E, hi) > target) chosen = hi;
    else {
        for (int it = 0; it < SEARCH_ITERS; ++it) {
            double mid = sqrt(lo * hi);
            if (estimate_bpp(E, mid) > target) lo = mid;
            else hi = mid;
        }
        chosen = hi;
    }
    float d = (float)chosen;
    if ((double)d < guard) d = nextafterf(d, INFINITY);
    return d;
}

static int compute_scales(const void* w, int dt, int64_t R, int64_t C, float* scale) {
    for (int64_t r = 0; r < R; ++r) {
        scale[r] = row_scale(w, dt, r, C);
        if (!isfinite(scale[r])) return OR_ERANGE;
    }
    return OR_OK;
}

double or_estimate_bpp(const void* w, int dt, int64_t R, int64_t C, double delta) {
    float* scale = (float*)malloc(sizeof(float) * (size_t)(R > 0 ? R : 1));
    estimator E;
    double est = -1.0;
    memset(&E, 0, sizeof E);
    if (!scale) return -1.0;
    if (compute_scales(w, dt, R, C, scale) == OR_OK && estimator_init(&E, w, dt, R, C, scale) == OR_OK)
        est = estimate_bpp(&E, delta);
    estimator_free(&E);
    free(scale);
    return est;
}

float or_select_step(const void* w, int dt, int64_t R, int64_t C, double target) {
    float* scale = (float*)malloc(sizeof(float) * (size_t)(R > 0 ? R : 1));
    estimator E;
    float d = -1.0f;
    memset(&E, 0, sizeof E);
    if (!scale) return -1.0f;
    if (compute_scales(w, dt, R, C, scale) == OR_OK && estimator_init(&E, w, dt, R, C, scale) == OR_OK)
        d = select_step(&E, target, max_abs_normalized(w, dt, R, C, scale));
    estimator_free(&E);
    free(scale);
    return d;
}

/* ------------------------------------------------------------------------------------------ */
/* Stream layout (reading). Little-endian. A 128-byte header, then sections, each starting at a */
/* 16-byte boundary: row_scale f32[R], row_qmax u16[R] (both empty in lossless mode), tables    */
/* (per table: i16 lo, u16 S, u16 escape frequency, u16 freq[S]), tile_index u32[n_tiles + 1]   */
/* (offsets in 4-byte units from the payload start), in the exponent-coded mode the raw plane   */
/* u8[Rp][Cp] (offset and CRC-32 in header bytes 96 and 104), payload. Format version 2: header */
/* bytes 112..115 hold the CRC-32 of every other byte outside the payload and the raw plane;    */
/* byte 116 is the lossy tile layout (block_of), 0 in the lossless modes.                      */
/* [G, "Start with a tensor round trip"]: the reported bitrate includes the metadata, so        */
/* actual_bpp = 8 total / (R C).                                                                 */
/* ------------------------------------------------------------------------------------------ */
enum {
    H_MAGIC = 0, H_VERSION = 4, H_MODE = 6, H_DTYPE = 7, H_ROWS = 8, H_COLS = 12,
    H_TILE_ROWS = 16, H_TILE_COLS = 18, H_LANES = 20, H_PROB_BITS = 22, H_NTABLES = 23,
    H_STEP = 24, H_TARGET = 28, H_NTILES = 32, H_NESC = 36, H_OFF_SCALE = 40, H_OFF_QMAX = 48,
    H_OFF_TABLES = 56, H_OFF_INDEX = 64, H_OFF_PAYLOAD = 72, H_TOTAL = 80, H_CRC = 88,
    H_OFF_RAW = 96, H_RAW_CRC = 104,   /* exponent-coded mode only; zero in the other modes */
    H_META_CRC = 112,                  /* CRC-32 of all bytes but the payload, the raw plane and this field */
    H_LAYOUT = 116                     /* lossy tile layout (reading R27): 0 or 1; 0 in the lossless modes */
};
#define FORMAT_VERSION 2

/* The metadata CRC-32 (reading R22 of the format: with the payload and raw-plane CRCs, every bit of
   a stream is covered): the message is the stream with the payload, the raw plane (if any) and the
   four CRC bytes at 112 left out, in stream order. */
static uint32_t meta_crc(const uint8_t* s, uint64_t o_raw, uint64_t raw_len, uint64_t o_pl) {
    uint32_t c = crc32_more(0xFFFFFFFFu, s, H_META_CRC);
    uint64_t from = H_META_CRC + 4;
    if (raw_len > 0) {
        c = crc32_more(c, s + from, (size_t)(o_raw - from));
        from = o_raw + raw_len;
    }
    c = crc32_more(c, s + from, (size_t)(o_pl - from));
    return c ^ 0xFFFFFFFFu;
}

static size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

typedef struct {
    int mode, dtype, tile_rows, prob_bits, n_tables, layout;
    int64_t R, C, Rp, Cp, tiles_r, tiles_c;
    uint32_t n_tiles, n_esc;
    float step, target;
    const uint8_t* scale_bytes;     /* unaligned views into the stream: read with get16/get32 */
    const uint8_t* qmax_bytes;
    const uint8_t* index_bytes;
    const uint8_t* payload;
    uint64_t payload_len;
    const uint8_t* raw;             /* exponent-coded mode: sign/mantissa bytes [Rp][Cp] */
    uint64_t raw_len;
    int32_t lo[N_LOSSY_TABLES];
    int32_t S[N_LOSSY_TABLES];
    uint32_t freq[N_LOSSY_TABLES][256];
} parsed;

static int dtype_planes(int dt) { return elem_bytes(dt); }

static int parse_stream(const uint8_t* s, size_t len, parsed* P) {
    memset(P, 0, sizeof *P);
    if (!s || len < HEADER_BYTES) return OR_ECORRUPT;
    if (memcmp(s + H_MAGIC, "EPK1", 4) != 0 || get16(s + H_VERSION) != FORMAT_VERSION) return OR_ECORRUPT;
    P->mode = s[H_MODE];
    P->dtype = s[H_DTYPE];
    P->R = get32(s + H_ROWS);
    P->C = get32(s + H_COLS);
    P->tile_rows = (int)get16(s + H_TILE_ROWS);
    P->prob_bits = s[H_PROB_BITS];
    P->n_tables = s[H_NTABLES];
    P->step = f32_from_bits(get32(s + H_STEP));
    P->target = f32_from_bits(get32(s + H_TARGET));
    P->n_tiles = get32(s + H_NTILES);
    P->n_esc = get32(s + H_NESC);
    P->layout = s[H_LAYOUT];
    if (P->layout > 1 || (P->layout != 0 && P->mode != MODE_LOSSY)) return OR_ECORRUPT;
    if (P->mode != MODE_LOSSY && P->mode != MODE_LOSSLESS && P->mode != MODE_LOSSLESS_EXP) return OR_ECORRUPT;
    if (P->mode == MODE_LOSSLESS_EXP && P->dtype != DT_BF16) return OR_ECORRUPT;
    if (P->mode == MODE_LOSSY && P->dtype != DT_F32 && P->dtype != DT_BF16 && P->dtype != DT_F16)
        return OR_ECORRUPT;
    if (P->mode == MODE_LOSSLESS && elem_bytes(P->dtype) == 0) return OR_ECORRUPT;
    if (P->tile_rows != 16 && P->tile_rows != 32) return OR_ECORRUPT;
    if (get16(s + H_TILE_COLS) != TILE_COLS || get16(s + H_LANES) != LANES) return OR_ECORRUPT;
    if (P->prob_bits < 10 || P->prob_bits > 12) return OR_ECORRUPT;
    int want_tables = P->mode == MODE_LOSSY ? N_LOSSY_TABLES : P->mode == MODE_LOSSLESS_EXP ? 1 : dtype_planes(P->dtype);
    if (P->n_tables != want_tables) return OR_ECORRUPT;
    if (P->mode == MODE_LOSSY && !(isfinite(P->step) && P->step > 0.0f)) return OR_ECORRUPT;
    P->Rp = ceil_div(P->R, P->tile_rows) * P->tile_rows;
    P->Cp = ceil_div(P->C, TILE_COLS) * TILE_COLS;
    P->tiles_r = P->Rp / P->tile_rows;
    P->tiles_c = P->Cp / TILE_COLS;
    if ((int64_t)P->n_tiles != P->tiles_r * P->tiles_c) return OR_ECORRUPT;
    uint64_t o_sc = get64(s + H_OFF_SCALE), o_qm = get64(s + H_OFF_QMAX), o_tb = get64(s + H_OFF_TABLES);
    uint64_t o_ix = get64(s + H_OFF_INDEX), o_pl = get64(s + H_OFF_PAYLOAD), total = get64(s + H_TOTAL);
    if (total != len) return OR_ECORRUPT;
    if (!(HEADER_BYTES <= o_sc && o_sc <= o_qm && o_qm <= o_tb && o_tb <= o_ix && o_ix <= o_pl && o_pl <= total))
        return OR_ECORRUPT;
    uint64_t rows_meta = P->mode == MODE_LOSSY ? (uint64_t)P->R : 0;
    if (o_qm - o_sc < 4 * rows_meta || o_tb - o_qm < 2 * rows_meta) return OR_ECORRUPT;
    if (o_pl - o_ix < 4 * ((uint64_t)P->n_tiles + 1)) return OR_ECORRUPT;
    P->scale_bytes = s + o_sc;
    P->qmax_bytes = s + o_qm;
    P->index_bytes = s + o_ix;
    P->payload = s + o_pl;
    P->payload_len = total - o_pl;
    if (P->payload_len % 4) return OR_ECORRUPT;
    uint64_t o_raw = get64(s + H_OFF_RAW);
    if (P->mode == MODE_LOSSLESS_EXP) {
        P->raw_len = (uint64_t)P->Rp * (uint64_t)P->Cp;
        if (o_raw % 16 || o_raw < o_ix + 4 * ((uint64_t)P->n_tiles + 1) || o_raw + P->raw_len > o_pl) return OR_ECORRUPT;
        P->raw = s + o_raw;
        if (crc32_ieee(P->raw, (size_t)P->raw_len) != get32(s + H_RAW_CRC)) return OR_ECORRUPT;
    } else if (o_raw != 0 || get32(s + H_RAW_CRC) != 0) {
        return OR_ECORRUPT;
    }
    /* tables */
    uint32_t M = 1u << P->prob_bits;
    uint64_t pos = o_tb;
    for (int t = 0; t < P->n_tables; ++t) {
        if (pos + 6 > o_ix) return OR_ECORRUPT;
        int32_t lo = (int16_t)get16(s + pos);
        int32_t S = (int32_t)get16(s + pos + 2);
        uint32_t esc = get16(s + pos + 4);
        pos += 6;
        int maxS = P->mode == MODE_LOSSY ? 255 : 256;
        if (S < 1 || S > maxS || pos + 2 * (uint64_t)S > o_ix) return OR_ECORRUPT;
        if (P->mode != MODE_LOSSY && (lo != 0 || S != 256 || esc != 0)) return OR_ECORRUPT;
        /* reading: a coordinate x must give a doubled coordinate 2x + b that fits int16, the
         * range the encoder's step bound keeps every value in */
        if (P->mode == MODE_LOSSY && t > 0 && (lo < -16384 || lo + S - 1 > 16383)) return OR_ECORRUPT;
        if (P->mode == MODE_LOSSY && t == 0 && (lo < 0 || lo + S - 1 > 1 || esc != 0)) return OR_ECORRUPT;
        uint64_t sum = esc;
        memset(P->freq[t], 0, sizeof P->freq[t]);
        for (int32_t k = 0; k < S; ++k) {
            P->freq[t][k] = get16(s + pos + 2 * (uint64_t)k);
            sum += P->freq[t][k];
        }
        if (P->mode == MODE_LOSSY) P->freq[t][ESC_SYM] += esc;   /* S <= 255: slot 255 is escape */
        pos += 2 * (uint64_t)S;
        if (sum != M) return OR_ECORRUPT;
        P->lo[t] = lo;
        P->S[t] = S;
    }
    /* tile index */
    uint64_t prev = 0;
    for (uint32_t i = 0; i <= P->n_tiles; ++i) {
        uint64_t v = get32(P->index_bytes + 4 * (uint64_t)i);
        if (i == 0 && v != 0) return OR_ECORRUPT;
        if (i > 0 && v < prev + LANES) return OR_ECORRUPT;     /* at least the 32 states */
        prev = v;
    }
    if (4 * prev != P->payload_len) return OR_ECORRUPT;
    if (crc32_ieee(P->payload, (size_t)P->payload_len) != get32(s + H_CRC)) return OR_ECORRUPT;
    if (meta_crc(s, o_raw, P->raw_len, o_pl) != get32(s + H_META_CRC)) return OR_ECORRUPT;
    if (P->mode == MODE_LOSSY)
        for (int64_t r = 0; r < P->R; ++r) {
            float v = f32_from_bits(get32(P->scale_bytes + 4 * r));
            if (!(isfinite(v) && v >= 0.0f)) return OR_ECORRUPT;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Lossy encoder. [A, Abstract]: row normalization -> E8 -> conditional model -> sampled rate   */
/* search -> tile entropy coding. Reading of the tile geometry: a tile covers tile_rows rows x  */
/* 256 columns, i.e. tile_rows x 32 E8 blocks of 8 columns, coded by 32 interleaved states in   */
/* tile_rows block steps; at block step s, step 9s codes the coset bit of each lane's block and */
/* steps 9s+1+j code its coordinate j with table 1 + 2j + b. Which block a lane codes at block  */
/* step s is the layout (block_of).                                                             */
/* ------------------------------------------------------------------------------------------ */
/* Reading R27: the pages interleave 32 states per tile but do not say which state codes which  */
/* block. Layout 0: lane l codes block column l of tile row s (the rows in turn). Layout 1: with */
/* G = 32 / tile_rows lanes per row, lane l codes tile row l mod tile_rows at block column     */
/* G s + floor(l / tile_rows), so every block step covers all tile rows. Both layouts code the  */
/* same symbols with the same tables; only their order across the states differs.              */
static void block_of(int layout, int tile_rows, int l, int s, int* rr, int* kk) {
    if (layout == 0) {
        *rr = s;
        *kk = l;
    } else {
        *rr = l % tile_rows;
        *kk = (LANES / tile_rows) * s + l / tile_rows;
    }
}
static void lossy_symbol(const sym_table* T, int32_t x, uint8_t* sym, uint16_t* esc) {
    if (x >= T->lo && x < T->lo + T->S) { *sym = (uint8_t)(x - T->lo); *esc = 0; }
    else { *sym = ESC_SYM; *esc = (uint16_t)(int16_t)x; }
}

typedef struct {
    uint8_t* buf; size_t len, cap;
} bytes_out;

static int out_reserve(bytes_out* o, size_t extra) {
    if (o->len + extra <= o->cap) return OR_OK;
    size_t nc = o->cap ? o->cap : 4096;
    while (nc < o->len + extra) nc *= 2;
    uint8_t* nb = (uint8_t*)realloc(o->buf, nc);
    if (!nb) return OR_ENOMEM;
    memset(nb + o->cap, 0, nc - o->cap);
    o->buf = nb;
    o->cap = nc;
    return OR_OK;
}

/* Writes header + metadata sections + payload. tables: n_tables entries (lo, S, f). */
static int serialize(bytes_out* o, int mode, int dt, int64_t R, int64_t C, int tile_rows, int layout, int prob_bits,
                     int n_tables, const int32_t* lo, const int32_t* S, uint32_t (*f)[256],
                     float step, float target, const float* scale, const uint16_t* qmax,
                     const uint32_t* tile_off /* [n_tiles + 1], 4-byte units */, uint32_t n_tiles,
                     const uint8_t* payload, uint64_t payload_len, uint32_t n_esc,
                     const uint8_t* raw /* exponent-coded mode, else NULL */, uint64_t raw_len) {
    uint64_t rows_meta = mode == MODE_LOSSY ? (uint64_t)R : 0;
    uint64_t tables_len = 0;
    for (int t = 0; t < n_tables; ++t) tables_len += 6 + 2 * (uint64_t)S[t];
    uint64_t o_sc = HEADER_BYTES;
    uint64_t o_qm = align16(o_sc + 4 * rows_meta);
    uint64_t o_tb = align16(o_qm + 2 * rows_meta);
    uint64_t o_ix = align16(o_tb + tables_len);
    uint64_t o_raw = raw ? align16(o_ix + 4 * ((uint64_t)n_tiles + 1)) : 0;
    uint64_t o_pl = raw ? align16(o_raw + raw_len) : align16(o_ix + 4 * ((uint64_t)n_tiles + 1));
    uint64_t total = o_pl + payload_len;
    if (out_reserve(o, (size_t)total) != OR_OK) return OR_ENOMEM;
    uint8_t* s = o->buf;
    memset(s, 0, (size_t)total);
    memcpy(s + H_MAGIC, "EPK1", 4);
    put16(s + H_VERSION, FORMAT_VERSION);
    s[H_MODE] = (uint8_t)mode;
    s[H_DTYPE] = (uint8_t)dt;
    put32(s + H_ROWS, (uint32_t)R);
    put32(s + H_COLS, (uint32_t)C);
    put16(s + H_TILE_ROWS, (uint32_t)tile_rows);
    s[H_LAYOUT] = (uint8_t)layout;
    put16(s + H_TILE_COLS, TILE_COLS);
    put16(s + H_LANES, LANES);
    s[H_PROB_BITS] = (uint8_t)prob_bits;
    s[H_NTABLES] = (uint8_t)n_tables;
    put32(s + H_STEP, bits_from_f32(step));
    put32(s + H_TARGET, bits_from_f32(target));
    put32(s + H_NTILES, n_tiles);
    put32(s + H_NESC, n_esc);
    put64(s + H_OFF_SCALE, o_sc);
    put64(s + H_OFF_QMAX, o_qm);
    put64(s + H_OFF_TABLES, o_tb);
    put64(s + H_OFF_INDEX, o_ix);
    put64(s + H_OFF_PAYLOAD, o_pl);
    put64(s + H_TOTAL, total);
    put32(s + H_CRC, crc32_ieee(payload, (size_t)payload_len));
    if (raw) {
        put64(s + H_OFF_RAW, o_raw);
        put32(s + H_RAW_CRC, crc32_ieee(raw, (size_t)raw_len));
        if (raw_len) memcpy(s + o_raw, raw, (size_t)raw_len);
    }
    for (uint64_t r = 0; r < rows_meta; ++r) {
        put32(s + o_sc + 4 * r, bits_from_f32(scale[r]));
        put16(s + o_qm + 2 * r, qmax[r]);
    }
    uint64_t pos = o_tb;
    for (int t = 0; t < n_tables; ++t) {
        put16(s + pos, (uint32_t)(uint16_t)(int16_t)lo[t]);
        put16(s + pos + 2, (uint32_t)S[t]);
        put16(s + pos + 4, mode == MODE_LOSSY ? f[t][ESC_SYM] : 0);
        pos += 6;
        for (int32_t k = 0; k < S[t]; ++k, pos += 2) put16(s + pos, f[t][k]);
    }
    for (uint32_t i = 0; i <= n_tiles; ++i) put32(s + o_ix + 4 * (uint64_t)i, tile_off[i]);
    if (payload_len) memcpy(s + o_pl, payload, (size_t)payload_len);   /* an empty matrix has no payload */
    put32(s + H_META_CRC, meta_crc(s, o_raw, raw ? raw_len : 0, o_pl));
    o->len = (size_t)total;
    return OR_OK;
}

static int encode_lossy(const void* w, int dt, int64_t R, int64_t C, double target, int prob_bits,
                        int tile_rows, int layout, bytes_out* o) {
    int rc = OR_OK;
    int64_t Rp = ceil_div(R, tile_rows) * tile_rows, Cp = ceil_div(C, TILE_COLS) * TILE_COLS;
    int64_t kb = Cp / 8;
    float* scale = (float*)calloc((size_t)(R > 0 ? R : 1), sizeof(float));
    uint16_t* qmax = (uint16_t*)calloc((size_t)(R > 0 ? R : 1), sizeof(uint16_t));
    int16_t* q = (int16_t*)calloc((size_t)(Rp * Cp > 0 ? Rp * Cp : 1), sizeof(int16_t));
    uint8_t* coset = (uint8_t*)calloc((size_t)(Rp * kb > 0 ? Rp * kb : 1), 1);
    estimator E;
    memset(&E, 0, sizeof E);
    value_hist h[N_LOSSY_TABLES];
    memset(h, 0, sizeof h);
    sym_table T[N_LOSSY_TABLES];
    rans_table RT[N_LOSSY_TABLES];
    memset(RT, 0, sizeof RT);
    uint8_t *tab = NULL, *sym = NULL;
    uint16_t *esc = NULL, *stack = NULL;
    uint32_t* tile_off = NULL;
    if (!scale || !qmax || !q || !coset) { rc = OR_ENOMEM; goto done; }
    if ((rc = compute_scales(w, dt, R, C, scale)) != OR_OK) goto done;
    if (R > 0 && C > 0) {
        if ((rc = estimator_init(&E, w, dt, R, C, scale)) != OR_OK) goto done;
    }
    float step = (R > 0 && C > 0) ? select_step(&E, target, max_abs_normalized(w, dt, R, C, scale)) : 1.0f;
    /* full quantization with the chosen step */
    for (int64_t r = 0; r < Rp; ++r)
        for (int64_t k = 0; k < kb; ++k) {
            double y[8];
            int32_t qq[8];
            int b;
            block_y(w, dt, R, C, scale, (double)step, r, k, y);
            e8_nearest(y, qq, &b);
            coset[r * kb + k] = (uint8_t)b;
            for (int i = 0; i < 8; ++i) {
                q[r * Cp + 8 * k + i] = (int16_t)qq[i];
                int64_t col = 8 * k + i;
                if (r < R && col < C) {
                    uint32_t a = (uint32_t)abs(qq[i]);
                    if (a > qmax[r]) qmax[r] = (uint16_t)a;
                }
            }
        }
    /* tables from the counts of every coded block (padding included) */
    for (int t = 0; t < N_LOSSY_TABLES; ++t) {
        h[t].hist = (uint64_t*)malloc(sizeof(uint64_t) * HIST_SPAN);
        if (!h[t].hist) { rc = OR_ENOMEM; goto done; }
        hist_reset(&h[t]);
    }
    for (int64_t r = 0; r < Rp; ++r)
        for (int64_t k = 0; k < kb; ++k) {
            int b = coset[r * kb + k];
            hist_add(&h[0], b);
            for (int j = 0; j < 8; ++j) hist_add(&h[1 + 2 * j + b], (q[r * Cp + 8 * k + j] - b) / 2);
        }
    int32_t lo[N_LOSSY_TABLES], S[N_LOSSY_TABLES];
    uint32_t f[N_LOSSY_TABLES][256];
    for (int t = 0; t < N_LOSSY_TABLES; ++t) {
        choose_window(&h[t], &T[t]);
        if ((rc = or_normalize(T[t].cnt, prob_bits, T[t].f)) != OR_OK) goto done;
        cumulate(T[t].f, T[t].c);
        lo[t] = T[t].lo;
        S[t] = T[t].S;
        memcpy(f[t], T[t].f, sizeof f[t]);
        if ((rc = rans_table_init(&RT[t], T[t].f, prob_bits)) != OR_OK) goto done;
    }
    /* tiles */
    int64_t tr_n = Rp / tile_rows, tc_n = Cp / TILE_COLS;
    uint32_t n_tiles = (uint32_t)(tr_n * tc_n);
    int n_steps = 9 * tile_rows;
    size_t tile_cap = 4 * LANES + 4 * (size_t)LANES * n_steps + 4;
    bytes_out pl = { NULL, 0, 0 };
    tab = (uint8_t*)malloc((size_t)n_steps * LANES);
    sym = (uint8_t*)malloc((size_t)n_steps * LANES);
    esc = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n_steps * LANES);
    stack = (uint16_t*)malloc(sizeof(uint16_t) * 64 * (size_t)n_steps + 2);
    tile_off = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)n_tiles + 1));
    if (!tab || !sym || !esc || !stack || !tile_off) { rc = OR_ENOMEM; goto done; }
    uint32_t n_esc = 0;
    tile_off[0] = 0;
    for (int64_t tr = 0; tr < tr_n; ++tr)
        for (int64_t tc = 0; tc < tc_n; ++tc) {
            for (int bs = 0; bs < tile_rows; ++bs)
                for (int l = 0; l < LANES; ++l) {
                    int rr, kk;
                    block_of(layout, tile_rows, l, bs, &rr, &kk);
                    int64_t r = tr * tile_rows + rr, k = tc * LANES + kk;
                    int b = coset[r * kb + k];
                    int t0 = 9 * bs;
                    tab[t0 * LANES + l] = 0;
                    sym[t0 * LANES + l] = (uint8_t)(b - T[0].lo);
                    esc[t0 * LANES + l] = 0;
                    for (int j = 0; j < 8; ++j) {
                        int t = t0 + 1 + j, ti = 1 + 2 * j + b;
                        int32_t x = (q[r * Cp + 8 * k + j] - b) / 2;
                        tab[t * LANES + l] = (uint8_t)ti;
                        lossy_symbol(&T[ti], x, &sym[t * LANES + l], &esc[t * LANES + l]);
                        if (sym[t * LANES + l] == ESC_SYM) n_esc++;
                    }
                }
            if ((rc = out_reserve(&pl, tile_cap)) != OR_OK) { free(pl.buf); goto done; }
            size_t nbytes = rans_encode_tile(RT, prob_bits, n_steps, tab, sym, esc, ESC_SYM, stack, pl.buf + pl.len);
            pl.len += nbytes;
            tile_off[tr * tc_n + tc + 1] = (uint32_t)(pl.len / 4);
        }
    rc = serialize(o, MODE_LOSSY, dt, R, C, tile_rows, layout, prob_bits, N_LOSSY_TABLES, lo, S, f, step,
                   (float)target, scale, qmax, tile_off, n_tiles, pl.buf, pl.len, n_esc, NULL, 0);
    free(pl.buf);
done:
    for (int t = 0; t < N_LOSSY_TABLES; ++t) { free(h[t].hist); rans_table_free(&RT[t]); }
    estimator_free(&E);
    free(scale); free(qmax); free(q); free(coset);
    free(tab); free(sym); free(esc); free(stack); free(tile_off);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Lossless mode. [G, "Choose a compression contract"] names a lossless tile-ANS configuration  */
/* across dtypes; [P, "無損方案追求逐位元恢復"]: lossless means every original bit comes back.     */
/* Reading: each element is split into byte planes (most significant first), each plane has    */
/* one order-0 table over 256 symbols (no escape), same tiles and lanes as the lossy mode;      */
/* lane l owns columns 8l..8l+7 of the tile; steps run row -> element -> plane.                 */
/* ------------------------------------------------------------------------------------------ */
static uint32_t elem_bits(const void* w, int eb, int64_t i) {
    const uint8_t* p = (const uint8_t*)w + (size_t)i * eb;
    uint32_t v = 0;
    for (int k = eb - 1; k >= 0; --k) v = (v << 8) | p[k];   /* native little-endian element */
    return v;
}

static int encode_lossless(const void* w, int dt, int64_t R, int64_t C, int prob_bits, int tile_rows, bytes_out* o) {
    int rc = OR_OK;
    int P = dtype_planes(dt);
    int64_t Rp = ceil_div(R, tile_rows) * tile_rows, Cp = ceil_div(C, TILE_COLS) * TILE_COLS;
    uint64_t cnt[4][256];
    uint32_t f[N_LOSSY_TABLES][256];
    int32_t lo[4] = { 0, 0, 0, 0 }, S[4] = { 256, 256, 256, 256 };
    rans_table RT[4];
    memset(cnt, 0, sizeof cnt);
    memset(RT, 0, sizeof RT);
    uint8_t *tab = NULL, *sym = NULL;
    uint16_t *esc = NULL, *stack = NULL;
    uint32_t* tile_off = NULL;
    bytes_out pl = { NULL, 0, 0 };
    for (int64_t r = 0; r < Rp; ++r)
        for (int64_t c = 0; c < Cp; ++c) {
            uint32_t v = (r < R && c < C) ? elem_bits(w, P, r * C + c) : 0;
            for (int p = 0; p < P; ++p) cnt[p][(v >> (8 * (P - 1 - p))) & 0xFF]++;
        }
    for (int p = 0; p < P; ++p) {
        if ((rc = or_normalize(cnt[p], prob_bits, f[p])) != OR_OK) goto done;
        if ((rc = rans_table_init(&RT[p], f[p], prob_bits)) != OR_OK) goto done;
    }
    int64_t tr_n = Rp / tile_rows, tc_n = Cp / TILE_COLS;
    uint32_t n_tiles = (uint32_t)(tr_n * tc_n);
    int n_steps = tile_rows * 8 * P;
    size_t tile_cap = 4 * LANES + 4 * (size_t)LANES * n_steps + 4;
    tab = (uint8_t*)malloc((size_t)n_steps * LANES);
    sym = (uint8_t*)malloc((size_t)n_steps * LANES);
    esc = (uint16_t*)calloc((size_t)n_steps * LANES, sizeof(uint16_t));
    stack = (uint16_t*)malloc(sizeof(uint16_t) * 64 * (size_t)n_steps + 2);
    tile_off = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)n_tiles + 1));
    if (!tab || !sym || !esc || !stack || !tile_off) { rc = OR_ENOMEM; goto done; }
    tile_off[0] = 0;
    for (int64_t tr = 0; tr < tr_n; ++tr)
        for (int64_t tc = 0; tc < tc_n; ++tc) {
            for (int rr = 0; rr < tile_rows; ++rr)
                for (int e = 0; e < 8; ++e)
                    for (int p = 0; p < P; ++p)
                        for (int l = 0; l < LANES; ++l) {
                            int64_t r = tr * tile_rows + rr, c = tc * TILE_COLS + 8 * l + e;
                            uint32_t v = (r < R && c < C) ? elem_bits(w, P, r * C + c) : 0;
                            int t = (rr * 8 + e) * P + p;
                            tab[t * LANES + l] = (uint8_t)p;
                            sym[t * LANES + l] = (uint8_t)((v >> (8 * (P - 1 - p))) & 0xFF);
                        }
            if ((rc = out_reserve(&pl, tile_cap)) != OR_OK) goto done;
            pl.len += rans_encode_tile(RT, prob_bits, n_steps, tab, sym, esc, -1, stack, pl.buf + pl.len);
            tile_off[tr * tc_n + tc + 1] = (uint32_t)(pl.len / 4);
        }
    rc = serialize(o, MODE_LOSSLESS, dt, R, C, tile_rows, 0, prob_bits, P, lo, S, f, 0.0f, 0.0f, NULL, NULL,
                   tile_off, n_tiles, pl.buf, pl.len, 0, NULL, 0);
done:
    for (int p = 0; p < 4; ++p) rans_table_free(&RT[p]);
    free(pl.buf); free(tab); free(sym); free(esc); free(stack); free(tile_off);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Exponent-coded lossless BF16. [G, "Choose a compression contract"] names a DFloat11 config   */
/* for lossless BF16 without describing it. Reading (after the published DFloat11 idea): the    */
/* 8-bit exponent of every element is entropy coded, here with the same tile rANS as the other  */
/* modes (one order-0 table over 256 symbols, one step per element, steps row -> element,      */
/* lane l owning columns 8l..8l+7 of the tile), and sign and mantissa are stored uncoded as one */
/* byte per element, (sign << 7) | mantissa, in a plane [Rp][Cp] laid out like the padded       */
/* matrix (padding elements are +0.0: exponent 0 and raw byte 0).                              */
/* ------------------------------------------------------------------------------------------ */
static uint32_t bf16_exponent(uint32_t v) { return (v >> 7) & 0xFFu; }
static uint32_t bf16_raw_byte(uint32_t v) { return ((v >> 8) & 0x80u) | (v & 0x7Fu); }
static uint32_t bf16_join(uint32_t e, uint32_t r) { return ((r & 0x80u) << 8) | (e << 7) | (r & 0x7Fu); }

static int encode_lossless_exp(const void* w, int64_t R, int64_t C, int prob_bits, int tile_rows, bytes_out* o) {
    int rc = OR_OK;
    int64_t Rp = ceil_div(R, tile_rows) * tile_rows, Cp = ceil_div(C, TILE_COLS) * TILE_COLS;
    uint64_t cnt[256];
    uint32_t f[N_LOSSY_TABLES][256];
    int32_t lo[1] = { 0 }, S[1] = { 256 };
    rans_table RT[1];
    memset(cnt, 0, sizeof cnt);
    memset(RT, 0, sizeof RT);
    uint8_t *tab = NULL, *sym = NULL, *raw = NULL;
    uint16_t *esc = NULL, *stack = NULL;
    uint32_t* tile_off = NULL;
    bytes_out pl = { NULL, 0, 0 };
    raw = (uint8_t*)calloc((size_t)(Rp * Cp > 0 ? Rp * Cp : 1), 1);
    if (!raw) { rc = OR_ENOMEM; goto done; }
    for (int64_t r = 0; r < Rp; ++r)
        for (int64_t c = 0; c < Cp; ++c) {
            uint32_t v = (r < R && c < C) ? elem_bits(w, 2, r * C + c) : 0;
            cnt[bf16_exponent(v)]++;
            raw[r * Cp + c] = (uint8_t)bf16_raw_byte(v);
        }
    if ((rc = or_normalize(cnt, prob_bits, f[0])) != OR_OK) goto done;
    if ((rc = rans_table_init(&RT[0], f[0], prob_bits)) != OR_OK) goto done;
    int64_t tr_n = Rp / tile_rows, tc_n = Cp / TILE_COLS;
    uint32_t n_tiles = (uint32_t)(tr_n * tc_n);
    int n_steps = tile_rows * 8;
    size_t tile_cap = 4 * LANES + 4 * (size_t)LANES * n_steps + 4;
    tab = (uint8_t*)calloc((size_t)n_steps * LANES, 1);
    sym = (uint8_t*)malloc((size_t)n_steps * LANES);
    esc = (uint16_t*)calloc((size_t)n_steps * LANES, sizeof(uint16_t));
    stack = (uint16_t*)malloc(sizeof(uint16_t) * 64 * (size_t)n_steps + 2);
    tile_off = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)n_tiles + 1));
    if (!tab || !sym || !esc || !stack || !tile_off) { rc = OR_ENOMEM; goto done; }
    tile_off[0] = 0;
    for (int64_t tr = 0; tr < tr_n; ++tr)
        for (int64_t tc = 0; tc < tc_n; ++tc) {
            for (int rr = 0; rr < tile_rows; ++rr)
                for (int e = 0; e < 8; ++e)
                    for (int l = 0; l < LANES; ++l) {
                        int64_t r = tr * tile_rows + rr, c = tc * TILE_COLS + 8 * l + e;
                        uint32_t v = (r < R && c < C) ? elem_bits(w, 2, r * C + c) : 0;
                        sym[(rr * 8 + e) * LANES + l] = (uint8_t)bf16_exponent(v);
                    }
            if ((rc = out_reserve(&pl, tile_cap)) != OR_OK) goto done;
            pl.len += rans_encode_tile(RT, prob_bits, n_steps, tab, sym, esc, -1, stack, pl.buf + pl.len);
            tile_off[tr * tc_n + tc + 1] = (uint32_t)(pl.len / 4);
        }
    rc = serialize(o, MODE_LOSSLESS_EXP, DT_BF16, R, C, tile_rows, 0, prob_bits, 1, lo, S, f, 0.0f, 0.0f, NULL, NULL,
                   tile_off, n_tiles, pl.buf, pl.len, 0, raw, (uint64_t)(Rp * Cp));
done:
    rans_table_free(&RT[0]);
    free(pl.buf); free(tab); free(sym); free(esc); free(stack); free(tile_off); free(raw);
    return rc;
}

int or_compress(const void* w, int src_dtype, int64_t rows, int64_t cols, int mode, double target_bpp,
                int prob_bits, int tile_rows, int layout, uint8_t** out, size_t* out_len, double* actual_bpp) {
    if (!out || !out_len || rows < 0 || cols < 0 || (rows * cols > 0 && !w)) return OR_EINVAL;
    if (rows > 0xFFFFFFFFll || cols >= (1ll << 28)) return OR_ERANGE;
    if (prob_bits < 10 || prob_bits > 12 || (tile_rows != 16 && tile_rows != 32)) return OR_EINVAL;
    if (layout < 0 || layout > 1 || (layout != 0 && mode != MODE_LOSSY)) return OR_EINVAL;
    bytes_out o = { NULL, 0, 0 };
    int rc;
    if (mode == MODE_LOSSY) {
        if (src_dtype != DT_F32 && src_dtype != DT_BF16 && src_dtype != DT_F16) return OR_EUNSUPPORTED;
        if (!(target_bpp > 0.0 && target_bpp <= 32.0)) return OR_EINVAL;
        for (int64_t i = 0; i < rows * cols; ++i)
            if (!isfinite(src_value(w, src_dtype, i))) return OR_ERANGE;
        rc = encode_lossy(w, src_dtype, rows, cols, target_bpp, prob_bits, tile_rows, layout, &o);
    } else if (mode == MODE_LOSSLESS) {
        if (elem_bytes(src_dtype) == 0) return OR_EUNSUPPORTED;
        rc = encode_lossless(w, src_dtype, rows, cols, prob_bits, tile_rows, &o);
    } else if (mode == MODE_LOSSLESS_EXP) {
        if (src_dtype != DT_BF16) return OR_EUNSUPPORTED;
        rc = encode_lossless_exp(w, rows, cols, prob_bits, tile_rows, &o);
    } else {
        return OR_EINVAL;
    }
    if (rc != OR_OK) { free(o.buf); return rc; }
    *out = o.buf;
    *out_len = o.len;
    if (actual_bpp) *actual_bpp = rows * cols > 0 ? 8.0 * (double)o.len / ((double)rows * (double)cols) : 0.0;
    return OR_OK;
}

void or_free(void* p) { free(p); }

/* ------------------------------------------------------------------------------------------ */
/* Decoder and reconstruction. [A, Abstract]: decoding and weight reconstruction are fused;     */
/* reconstruction; containers BF16, FP16, FP8, INT8 with the bitrate independent of precision.  */
/* Reading: alpha_r = fp32(h s_r) with h = step / 2; BF16 and FP16 are RNE casts of             */
/* fp32(q alpha_r); FP8 E4M3 stores fp32(q h) with s_r as the per-row dequantization scale; INT8 */
/* stores round-half-away(q / k_r) with k_r = max(1, ceil(qmax_r / 127)) and the scale           */
/* fp32(alpha_r k_r).                                                                           */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    const parsed* P;
    int rows;                       /* tile rows */
    const uint8_t* sym;             /* decoded symbols so far, [steps * 32] */
} lossy_tab_ctx;

static void lossy_tables(void* vctx, int step, uint8_t out[LANES]) {
    lossy_tab_ctx* c = (lossy_tab_ctx*)vctx;
    int m = step % 9;
    for (int l = 0; l < LANES; ++l) {
        if (m == 0) { out[l] = 0; continue; }
        int b = c->P->lo[0] + c->sym[(step - m) * LANES + l];
        out[l] = (uint8_t)(1 + 2 * (m - 1) + b);
    }
}

typedef struct {
    rans_table T[N_LOSSY_TABLES];
    int n;
} decoder_tables;

static int decoder_tables_init(decoder_tables* D, const parsed* P) {
    memset(D, 0, sizeof *D);
    D->n = P->n_tables;
    for (int t = 0; t < P->n_tables; ++t) {
        int rc = rans_table_init(&D->T[t], P->freq[t], P->prob_bits);
        if (rc != OR_OK) return rc;
    }
    return OR_OK;
}
static void decoder_tables_free(decoder_tables* D) {
    for (int t = 0; t < D->n; ++t) rans_table_free(&D->T[t]);
}

/* Decode tile `tile` of a lossy stream into doubled coordinates qt[tile_rows][256] and cosets
 * bt[tile_rows][32]. */
static int decode_lossy_tile(const parsed* P, const decoder_tables* D, uint32_t tile, int16_t* qt,
                             uint8_t* bt, uint8_t* sym, uint16_t* esc) {
    uint64_t a = get32(P->index_bytes + 4 * (uint64_t)tile), b = get32(P->index_bytes + 4 * ((uint64_t)tile + 1));
    lossy_tab_ctx ctx = { P, P->tile_rows, sym };
    int n_steps = 9 * P->tile_rows;
    int rc = rans_decode_tile(D->T, P->prob_bits, n_steps, P->payload + 4 * a, (size_t)(4 * (b - a)),
                              lossy_tables, &ctx, ESC_SYM, sym, esc, NULL);
    if (rc != OR_OK) return rc;
    for (int bs = 0; bs < P->tile_rows; ++bs)
        for (int l = 0; l < LANES; ++l) {
            int rr, kk;
            block_of(P->layout, P->tile_rows, l, bs, &rr, &kk);
            int t0 = 9 * bs;
            int cb = P->lo[0] + sym[t0 * LANES + l];
            bt[rr * LANES + kk] = (uint8_t)cb;
            for (int j = 0; j < 8; ++j) {
                int t = t0 + 1 + j, ti = 1 + 2 * j + cb;
                uint8_t s = sym[t * LANES + l];
                int32_t x = (s == ESC_SYM) ? (int32_t)(int16_t)esc[t * LANES + l] : P->lo[ti] + s;
                qt[rr * TILE_COLS + 8 * kk + j] = (int16_t)(2 * x + cb);
            }
        }
    return OR_OK;
}

/* Decode tile `tile` of a lossless stream into element bit patterns vt[tile_rows][256]. */
typedef struct { int P; } lossless_ctx;
static void lossless_tables(void* vctx, int step, uint8_t out[LANES]) {
    int P = ((lossless_ctx*)vctx)->P;
    for (int l = 0; l < LANES; ++l) out[l] = (uint8_t)(step % P);
}

static int decode_lossless_tile(const parsed* P, const decoder_tables* D, uint32_t tile, uint32_t* vt,
                                uint8_t* sym, uint16_t* esc) {
    uint64_t a = get32(P->index_bytes + 4 * (uint64_t)tile), b = get32(P->index_bytes + 4 * ((uint64_t)tile + 1));
    int np = P->n_tables;
    lossless_ctx ctx = { np };
    int n_steps = P->tile_rows * 8 * np;
    int rc = rans_decode_tile(D->T, P->prob_bits, n_steps, P->payload + 4 * a, (size_t)(4 * (b - a)),
                              lossless_tables, &ctx, -1, sym, esc, NULL);
    if (rc != OR_OK) return rc;
    for (int rr = 0; rr < P->tile_rows; ++rr)
        for (int e = 0; e < 8; ++e)
            for (int l = 0; l < LANES; ++l) {
                uint32_t v = 0;
                for (int p = 0; p < np; ++p) v = (v << 8) | sym[((rr * 8 + e) * np + p) * LANES + l];
                vt[rr * TILE_COLS + 8 * l + e] = v;
            }
    return OR_OK;
}

/* Decode tile `tile` of an exponent-coded stream into BF16 bit patterns vt[tile_rows][256]. */
static int decode_exp_tile(const parsed* P, const decoder_tables* D, uint32_t tile, uint32_t* vt,
                           uint8_t* sym, uint16_t* esc) {
    uint64_t a = get32(P->index_bytes + 4 * (uint64_t)tile), b = get32(P->index_bytes + 4 * ((uint64_t)tile + 1));
    lossless_ctx ctx = { 1 };
    int n_steps = P->tile_rows * 8;
    int rc = rans_decode_tile(D->T, P->prob_bits, n_steps, P->payload + 4 * a, (size_t)(4 * (b - a)),
                              lossless_tables, &ctx, -1, sym, esc, NULL);
    if (rc != OR_OK) return rc;
    int64_t tr = tile / P->tiles_c, tc = tile % P->tiles_c;
    for (int rr = 0; rr < P->tile_rows; ++rr)
        for (int e = 0; e < 8; ++e)
            for (int l = 0; l < LANES; ++l) {
                int64_t r = tr * P->tile_rows + rr, c = tc * TILE_COLS + 8 * l + e;
                uint32_t rb = P->raw[r * P->Cp + c];
                vt[rr * TILE_COLS + 8 * l + e] = bf16_join(sym[(rr * 8 + e) * LANES + l], rb);
            }
    return OR_OK;
}

/* Decode tile `tile` of either lossless mode. */
static int decode_bits_tile(const parsed* P, const decoder_tables* D, uint32_t tile, uint32_t* vt,
                            uint8_t* sym, uint16_t* esc) {
    return P->mode == MODE_LOSSLESS_EXP ? decode_exp_tile(P, D, tile, vt, sym, esc)
                                        : decode_lossless_tile(P, D, tile, vt, sym, esc);
}

static int container_bytes(int ct) { return elem_bytes(ct); }

/* One reconstructed element of a lossy stream, written as container `ct` at dst. */
static void reconstruct(const parsed* P, int ct, int64_t r, int32_t q, uint8_t* dst) {
    float s = f32_from_bits(get32(P->scale_bytes + 4 * r));
    float h = P->step / 2.0f;
    float alpha = h * s;
    if (ct == DT_BF16) put16(dst, or_f32_to_bf16((float)q * alpha));
    else if (ct == DT_F16) put16(dst, or_f32_to_f16((float)q * alpha));
    else if (ct == DT_F8E4M3) dst[0] = or_f32_to_e4m3((float)q * h);
    else if (ct == DT_I8) {
        int32_t qm = (int32_t)get16(P->qmax_bytes + 2 * r);
        int32_t k = (qm + 126) / 127;
        if (k < 1) k = 1;
        int32_t a = q < 0 ? -q : q;
        int32_t v = (2 * a + k) / (2 * k);
        dst[0] = (uint8_t)(int8_t)(q < 0 ? -v : v);
    }
}

static float row_out_scale(const parsed* P, int ct, int64_t r) {
    float s = f32_from_bits(get32(P->scale_bytes + 4 * r));
    if (ct == DT_F8E4M3) return s;
    int32_t qm = (int32_t)get16(P->qmax_bytes + 2 * r);
    int32_t k = (qm + 126) / 127;
    if (k < 1) k = 1;
    float alpha = (P->step / 2.0f) * s;
    return alpha * (float)k;
}

typedef struct {
    const parsed* P;
    const decoder_tables* D;
    int container;
    uint8_t* out;           /* [R][C] elements of the container */
    int16_t* qout;          /* [R][C] doubled coordinates or NULL */
    uint8_t* bout;          /* [R][ceil(C/8)] cosets or NULL */
    int64_t t_begin, t_end;
    int rc;
} decode_job;

static void* decode_worker(void* arg) {
    decode_job* J = (decode_job*)arg;
    const parsed* P = J->P;
    int np = P->mode == MODE_LOSSY ? 9 : 8 * P->n_tables;
    size_t nsym = (size_t)P->tile_rows * np * LANES;
    uint8_t* sym = (uint8_t*)malloc(nsym);
    uint16_t* esc = (uint16_t*)malloc(nsym * sizeof(uint16_t));
    int16_t* qt = (int16_t*)malloc(sizeof(int16_t) * P->tile_rows * TILE_COLS);
    uint32_t* vt = (uint32_t*)malloc(sizeof(uint32_t) * P->tile_rows * TILE_COLS);
    uint8_t* bt = (uint8_t*)malloc((size_t)P->tile_rows * LANES);
    int eb = container_bytes(J->container);
    int64_t kb = ceil_div(P->C, 8);
    J->rc = OR_OK;
    if (!sym || !esc || !qt || !vt || !bt) { J->rc = OR_ENOMEM; goto done; }
    for (int64_t t = J->t_begin; t < J->t_end; ++t) {
        int64_t tr = t / P->tiles_c, tc = t % P->tiles_c;
        int rc = P->mode == MODE_LOSSY ? decode_lossy_tile(P, J->D, (uint32_t)t, qt, bt, sym, esc)
                                       : decode_bits_tile(P, J->D, (uint32_t)t, vt, sym, esc);
        if (rc != OR_OK) { J->rc = rc; goto done; }
        for (int rr = 0; rr < P->tile_rows; ++rr) {
            int64_t r = tr * P->tile_rows + rr;
            if (r >= P->R) break;
            for (int c = 0; c < TILE_COLS; ++c) {
                int64_t col = tc * TILE_COLS + c;
                if (col >= P->C) break;
                int64_t i = r * P->C + col;
                if (P->mode == MODE_LOSSY) {
                    if (J->qout) J->qout[i] = qt[rr * TILE_COLS + c];
                    if (J->bout && (c % 8) == 0) J->bout[r * kb + col / 8] = bt[rr * LANES + c / 8];
                    if (J->out) reconstruct(P, J->container, r, qt[rr * TILE_COLS + c], J->out + (size_t)i * eb);
                } else if (J->out) {
                    uint32_t v = vt[rr * TILE_COLS + c];
                    for (int k = 0; k < eb; ++k) J->out[(size_t)i * eb + k] = (uint8_t)(v >> (8 * k));
                }
            }
        }
    }
done:
    free(sym); free(esc); free(qt); free(vt); free(bt);
    return NULL;
}

static int run_decode(const parsed* P, int container, uint8_t* out, int16_t* qout, uint8_t* bout, int n_threads) {
    decoder_tables D;
    int rc = decoder_tables_init(&D, P);
    if (rc != OR_OK) { decoder_tables_free(&D); return rc; }
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    decode_job jobs[256];
    pthread_t th[256];
    int running[256];
    int64_t per = ceil_div((int64_t)P->n_tiles, n_threads);
    for (int i = 0; i < n_threads; ++i) {
        int64_t b = i * per, e = (i + 1) * per;
        if (e > (int64_t)P->n_tiles) e = P->n_tiles;
        jobs[i] = (decode_job){ P, &D, container, out, qout, bout, b, e, OR_OK };
        running[i] = 0;
        if (b >= e) continue;
        if (n_threads == 1) decode_worker(&jobs[i]);
        else if (pthread_create(&th[i], NULL, decode_worker, &jobs[i]) == 0) running[i] = 1;
        else decode_worker(&jobs[i]);                 /* no thread available: run inline */
    }
    for (int i = 0; i < n_threads; ++i)
        if (running[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < n_threads; ++i)
        if (jobs[i].rc != OR_OK && rc == OR_OK) rc = jobs[i].rc;
    decoder_tables_free(&D);
    return rc;
}

static int container_ok(const parsed* P, int container) {
    if (P->mode != MODE_LOSSY) return container == P->dtype;
    return container == DT_BF16 || container == DT_F16 || container == DT_F8E4M3 || container == DT_I8;
}

/* Full decode of a stream into `container` ([R][C], row-major). row_scale (lossy FP8 / INT8
 * only, else ignored) receives the per-row dequantization scale. */
int or_decompress(const uint8_t* s, size_t len, int container, void* out, float* row_scale, int n_threads) {
    parsed P;
    int rc = parse_stream(s, len, &P);
    if (rc != OR_OK) return rc;
    if (!container_ok(&P, container)) return OR_EUNSUPPORTED;
    if (!out && P.R * P.C > 0) return OR_EINVAL;
    if (P.mode == MODE_LOSSY && (container == DT_F8E4M3 || container == DT_I8)) {
        if (!row_scale) return OR_EINVAL;
        for (int64_t r = 0; r < P.R; ++r) row_scale[r] = row_out_scale(&P, container, r);
    }
    return run_decode(&P, container, (uint8_t*)out, NULL, NULL, n_threads);
}

/* Decoded doubled coordinates q [R][C] (lossy) and optionally cosets [R][ceil(C/8)]. */
int or_decode_symbols(const uint8_t* s, size_t len, int16_t* q, uint8_t* coset, int n_threads) {
    parsed P;
    int rc = parse_stream(s, len, &P);
    if (rc != OR_OK) return rc;
    if (P.mode != MODE_LOSSY) return OR_EUNSUPPORTED;
    return run_decode(&P, DT_BF16, NULL, q, coset, n_threads);
}

/* Decode only the listed tiles. out receives, per listed tile, tile_rows x 256 container
 * elements (padding positions included, as decoded); qout (optional) the doubled coordinates;
 * scale_out (optional, FP8 and INT8 containers of a lossy stream) the output scale of each of
 * the tile's rows, as or_decompress gives it (0 for padding rows). */
int or_decompress_tiles(const uint8_t* s, size_t len, int container, const uint32_t* tiles, int n,
                        void* out, int16_t* qout, float* scale_out) {
    parsed P;
    int rc = parse_stream(s, len, &P);
    if (rc != OR_OK) return rc;
    if (!container_ok(&P, container)) return OR_EUNSUPPORTED;
    decoder_tables D;
    rc = decoder_tables_init(&D, &P);
    int np = P.mode == MODE_LOSSY ? 9 : 8 * P.n_tables;
    size_t nsym = (size_t)P.tile_rows * np * LANES;
    uint8_t* sym = (uint8_t*)malloc(nsym);
    uint16_t* esc = (uint16_t*)malloc(nsym * sizeof(uint16_t));
    int16_t* qt = (int16_t*)malloc(sizeof(int16_t) * P.tile_rows * TILE_COLS);
    uint32_t* vt = (uint32_t*)malloc(sizeof(uint32_t) * P.tile_rows * TILE_COLS);
    uint8_t* bt = (uint8_t*)malloc((size_t)P.tile_rows * LANES);
    int eb = container_bytes(container);
    size_t per_tile = (size_t)P.tile_rows * TILE_COLS;
    if (rc == OR_OK && (!sym || !esc || !qt || !vt || !bt)) rc = OR_ENOMEM;
    for (int i = 0; rc == OR_OK && i < n; ++i) {
        if (tiles[i] >= P.n_tiles) { rc = OR_EINVAL; break; }
        int64_t tr = tiles[i] / P.tiles_c;
        rc = P.mode == MODE_LOSSY ? decode_lossy_tile(&P, &D, tiles[i], qt, bt, sym, esc)
                                  : decode_bits_tile(&P, &D, tiles[i], vt, sym, esc);
        if (rc != OR_OK) break;
        for (int rr = 0; rr < P.tile_rows; ++rr) {
            int64_t r = tr * P.tile_rows + rr;
            if (scale_out && P.mode == MODE_LOSSY && (container == DT_F8E4M3 || container == DT_I8))
                scale_out[(size_t)i * P.tile_rows + rr] = r < P.R ? row_out_scale(&P, container, r) : 0.0f;
            for (int c = 0; c < TILE_COLS; ++c) {
                size_t o = (size_t)i * per_tile + (size_t)rr * TILE_COLS + c;
                if (P.mode == MODE_LOSSY) {
                    if (qout) qout[o] = qt[rr * TILE_COLS + c];
                    if (out) {
                        if (r < P.R) reconstruct(&P, container, r, qt[rr * TILE_COLS + c], (uint8_t*)out + o * eb);
                        else memset((uint8_t*)out + o * eb, 0, (size_t)eb);
                    }
                } else if (out) {
                    for (int k = 0; k < eb; ++k) ((uint8_t*)out)[o * eb + k] = (uint8_t)(vt[rr * TILE_COLS + c] >> (8 * k));
                }
            }
        }
    }
    free(sym); free(esc); free(qt); free(vt); free(bt);
    decoder_tables_free(&D);
    return rc;
}

/* Header fields and section sizes of a validated stream, for the accounting tests.
 * info[0..12] = R, C, mode, dtype, tile_rows, prob_bits, n_tiles, n_escapes, payload bytes (the
 * tile payload, plus the raw plane in the exponent-coded mode), metadata bytes (total - payload),
 * state bytes (4 * 32 * n_tiles), total bytes, tile layout;
 * fstep receives the step and target. */
int or_stream_info(const uint8_t* s, size_t len, int64_t* info, float* fstep) {
    parsed P;
    int rc = parse_stream(s, len, &P);
    if (rc != OR_OK) return rc;
    info[0] = P.R; info[1] = P.C; info[2] = P.mode; info[3] = P.dtype; info[4] = P.tile_rows;
    info[5] = P.prob_bits; info[6] = P.n_tiles; info[7] = P.n_esc;
    info[8] = (int64_t)(P.payload_len + P.raw_len);       /* coded words plus uncoded raw bytes */
    info[9] = (int64_t)(len - P.payload_len - P.raw_len); info[10] = 4ll * LANES * P.n_tiles; info[11] = (int64_t)len;
    info[12] = P.layout;
    fstep[0] = P.step;
    fstep[1] = P.target;
    return OR_OK;
}

/* Tables of a validated stream: lo[t], S[t], f[t][256] for t < n_tables. Returns n_tables. */
int or_stream_tables(const uint8_t* s, size_t len, int32_t* lo, int32_t* S, uint32_t* f) {
    parsed P;
    int rc = parse_stream(s, len, &P);
    if (rc != OR_OK) return rc;
    for (int t = 0; t < P.n_tables; ++t) {
        lo[t] = P.lo[t];
        S[t] = P.S[t];
        memcpy(f + 256 * t, P.freq[t], 256 * sizeof(uint32_t));
    }
    return P.n_tables;
}

float or_row_scale(const void* w, int dt, int64_t R, int64_t C, int64_t r) {
    (void)R;
    return row_scale(w, dt, r, C);
}

/* ------------------------------------------------------------------------------------------ */
/* FP8 linear forward: activations. [A, Abstract] lists FP8 among the containers the decoded    */
/* weights go to; a layer that multiplies in FP8 also needs its activations in FP8. Reading     */
/* (the pages give no rule): per-row (per-token) scaling to the E4M3 range, amax_m =            */
/* max_k |x_mk| (exact in fp32), s_m = fp32(amax_m / 448), q_mk = E4M3(fp32(x_mk * fp32(448 /   */
/* amax_m))) with the same saturating round-to-nearest-even cast as the weight container; a    */
/* row with amax_m = 0 gets s_m = 0 and codes 0, and amax_m is raised to 2^-100 when smaller,   */
/* so that 448 / amax_m stays finite. Y[m][n] is then s_m * s_w[n] * sum_k x8_mk w8_nk, in      */
/* BF16. Inputs must be finite.                                                                 */
/* ------------------------------------------------------------------------------------------ */
int or_quantize_rows_e4m3(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s) {
    if (M < 0 || K < 0 || (M * K > 0 && (!x || !q)) || (M > 0 && !s)) return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(f32_from_bits((uint32_t)x[m * K + k] << 16));
            if (!isfinite(v)) return OR_ERANGE;
            if (v > amax) amax = v;
        }
        if (amax == 0.0f) {
            s[m] = 0.0f;
            for (int64_t k = 0; k < K; ++k) q[m * K + k] = 0;
            continue;
        }
        if (amax < 0x1p-100f) amax = 0x1p-100f;
        s[m] = amax / 448.0f;
        float inv = 448.0f / amax;
        for (int64_t k = 0; k < K; ++k) q[m * K + k] = or_f32_to_e4m3(f32_from_bits((uint32_t)x[m * K + k] << 16) * inv);
    }
    return OR_OK;
}
