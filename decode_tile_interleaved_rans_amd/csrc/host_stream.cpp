// Host-side validation of a stream before anything reaches the device, so that a damaged or
// incomplete stream stops with a clear error instead of a wrong tensor ("EntroPack PyTorch
// Guide", sections "Test saved artifacts and reloads before deployment" and "Diagnose
// compression failures in the correct order": the saved object must hold everything the decoder
// needs).
#include <cmath>
#include <cstring>

#include "ep_internal.h"

namespace ep {
namespace {

inline uint32_t r16(const uint8_t* p) { return (uint32_t)p[0] | (uint32_t)p[1] << 8; }
inline uint32_t r32(const uint8_t* p) { return r16(p) | r16(p + 2) << 16; }
inline uint64_t r64(const uint8_t* p) { return (uint64_t)r32(p) | (uint64_t)r32(p + 4) << 32; }
inline float rf32(const uint8_t* p) {
    uint32_t u = r32(p);
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

struct CrcTable {
    uint32_t t[256];
    CrcTable() {
        for (uint32_t i = 0; i < 256; ++i) {
            uint32_t c = i;
            for (int k = 0; k < 8; ++k) c = c & 1 ? 0xEDB88320u ^ (c >> 1) : c >> 1;
            t[i] = c;
        }
    }
};

ep_status bad(std::string* why, const char* msg) {
    if (why) *why = msg;
    return EP_ECORRUPT;
}

}  // namespace

int element_bytes(int dtype) {
    switch (dtype) {
        case EP_F32: return 4;
        case EP_BF16:
        case EP_F16: return 2;
        case EP_F8E4M3:
        case EP_I8:
        case EP_U8: return 1;
        default: return 0;
    }
}

namespace {
uint32_t crc32_add(uint32_t c, const uint8_t* p, size_t n) {
    static const CrcTable T;
    for (size_t i = 0; i < n; ++i) c = T.t[(c ^ p[i]) & 0xFF] ^ (c >> 8);
    return c;
}
}  // namespace

uint32_t crc32(const uint8_t* p, size_t n) { return ~crc32_add(0xFFFFFFFFu, p, n); }

uint32_t meta_crc32(const uint8_t* s, uint64_t off_raw, uint64_t raw_len, uint64_t off_payload) {
    const uint64_t after = kMetaCrc + 4;
    uint32_t c = crc32_add(0xFFFFFFFFu, s, kMetaCrc);
    if (raw_len) {
        c = crc32_add(c, s + after, off_raw - after);
        c = crc32_add(c, s + off_raw + raw_len, off_payload - (off_raw + raw_len));
    } else {
        c = crc32_add(c, s + after, off_payload - after);
    }
    return ~c;
}

ep_status parse_stream(const uint8_t* s, size_t len, StreamView* v, std::string* why) {
    *v = StreamView{};
    if (!s || len < (size_t)kHeaderBytes) return bad(why, "stream shorter than its 128-byte header");
    if (std::memcmp(s, "EPK1", 4) != 0) return bad(why, "bad magic (not an EPK1 stream)");
    if (r16(s + kVersion) != (uint32_t)kFormatVersion) return bad(why, "unsupported stream version");
    v->base = s;
    v->len = len;
    v->mode = s[kMode];
    v->dtype = s[kDtype];
    v->rows = r32(s + kRows);
    v->cols = r32(s + kCols);
    v->tile_rows = (int)r16(s + kTileRows);
    v->layout = s[kLayout];
    v->prob_bits = s[kProbBits];
    v->n_tables = s[kNumTables];
    v->step = rf32(s + kStep);
    v->target = rf32(s + kTarget);
    v->n_tiles = r32(s + kNumTiles);
    v->n_escapes = r32(s + kNumEscapes);
    const bool lossy = v->mode == EP_MODE_LOSSY_E8;
    const bool split = v->mode == EP_MODE_LOSSLESS_EXP;
    if (!lossy && !split && v->mode != EP_MODE_LOSSLESS) return bad(why, "unknown mode");
    if (split && v->dtype != EP_BF16) return bad(why, "exponent-coded lossless stream with a dtype other than bf16");
    if (lossy && v->dtype != EP_F32 && v->dtype != EP_BF16 && v->dtype != EP_F16)
        return bad(why, "lossy stream with a source dtype other than f32/bf16/f16");
    if (!lossy && element_bytes(v->dtype) == 0) return bad(why, "unknown source dtype");
    if (v->tile_rows != 16 && v->tile_rows != 32) return bad(why, "tile_rows must be 16 or 32");
    if (v->layout > 1 || (v->layout != 0 && !lossy)) return bad(why, "tile layout must be 0, or 1 in the lossy mode");
    if (r16(s + kTileColsField) != (uint32_t)kTileCols || r16(s + kLanesField) != (uint32_t)kLanes)
        return bad(why, "tile width must be 256 columns and 32 lanes");
    if (v->prob_bits < 10 || v->prob_bits > 12) return bad(why, "prob_bits outside 10..12");
    const int want_tables = lossy ? kLossyTables : split ? 1 : element_bytes(v->dtype);
    if (v->n_tables != want_tables) return bad(why, "wrong number of tables for the mode");
    if (lossy && !(std::isfinite(v->step) && v->step > 0.0f)) return bad(why, "step must be finite and > 0");
    v->tiles_r = (v->rows + v->tile_rows - 1) / v->tile_rows;
    v->tiles_c = (v->cols + kTileCols - 1) / kTileCols;
    if ((uint64_t)v->n_tiles != (uint64_t)(v->tiles_r * v->tiles_c)) return bad(why, "tile count disagrees with the shape");
    v->off_scale = r64(s + kOffScale);
    v->off_qmax = r64(s + kOffQmax);
    v->off_tables = r64(s + kOffTables);
    v->off_index = r64(s + kOffIndex);
    v->off_payload = r64(s + kOffPayload);
    const uint64_t total = r64(s + kTotalLen);
    if (total != len) return bad(why, "stream length differs from the header's total (truncated or padded)");
    if (!((uint64_t)kHeaderBytes <= v->off_scale && v->off_scale <= v->off_qmax && v->off_qmax <= v->off_tables &&
          v->off_tables <= v->off_index && v->off_index <= v->off_payload && v->off_payload <= total))
        return bad(why, "section offsets out of order or out of range");
    if ((v->off_scale | v->off_qmax | v->off_tables | v->off_index | v->off_payload) & 15)
        return bad(why, "section offsets must be 16-byte aligned");
    const uint64_t meta_rows = lossy ? (uint64_t)v->rows : 0;
    if (v->off_qmax - v->off_scale < 4 * meta_rows || v->off_tables - v->off_qmax < 2 * meta_rows)
        return bad(why, "row metadata sections too short");
    if (v->off_payload - v->off_index < 4 * ((uint64_t)v->n_tiles + 1)) return bad(why, "tile index section too short");
    v->payload_len = total - v->off_payload;
    if (v->payload_len % 4) return bad(why, "payload length not a multiple of 4");
    v->off_raw = r64(s + kOffRaw);
    if (split) {
        v->raw_len = (uint64_t)(v->tiles_r * v->tile_rows) * (uint64_t)(v->tiles_c * kTileCols);
        if ((v->off_raw & 15) || v->off_raw < v->off_index + 4 * ((uint64_t)v->n_tiles + 1) ||
            v->off_raw + v->raw_len > v->off_payload)
            return bad(why, "raw sign/mantissa plane out of place or too short");
        if (crc32(s + v->off_raw, v->raw_len) != r32(s + kRawCrc)) return bad(why, "raw plane CRC-32 mismatch");
    } else if (v->off_raw != 0 || r32(s + kRawCrc) != 0) {
        return bad(why, "raw plane fields set in a stream without a raw plane");
    }
    // tables
    const uint32_t M = 1u << v->prob_bits;
    uint64_t pos = v->off_tables;
    v->tables.resize(v->n_tables);
    for (int t = 0; t < v->n_tables; ++t) {
        if (pos + 6 > v->off_index) return bad(why, "table section truncated");
        Table& T = v->tables[t];
        T.lo = (int16_t)r16(s + pos);
        T.width = (int32_t)r16(s + pos + 2);
        const uint32_t esc = r16(s + pos + 4);
        pos += 6;
        if (T.width < 1 || T.width > (lossy ? 255 : 256) || pos + 2 * (uint64_t)T.width > v->off_index)
            return bad(why, "table window width out of range");
        if (!lossy && (T.lo != 0 || T.width != 256 || esc != 0)) return bad(why, "lossless tables cover 0..255 without escape");
        // a coordinate x must give a doubled coordinate 2x + b that fits int16 (the range the
        // encoder's step bound keeps every value in)
        if (lossy && t > 0 && (T.lo < -16384 || T.lo + T.width - 1 > 16383))
            return bad(why, "table window beyond the doubled-coordinate range");
        if (lossy && t == 0 && (T.lo < 0 || T.lo + T.width - 1 > 1 || esc != 0)) return bad(why, "coset table must cover {0,1}");
        std::memset(T.freq, 0, sizeof T.freq);
        uint64_t sum = esc;
        for (int k = 0; k < T.width; ++k) {
            T.freq[k] = r16(s + pos + 2 * (uint64_t)k);
            sum += T.freq[k];
        }
        if (lossy) T.freq[kEscape] += esc;
        pos += 2 * (uint64_t)T.width;
        if (sum != M) return bad(why, "table frequencies do not sum to 2^prob_bits");
    }
    // tile index: starts at 0, each tile holds at least its 32 states, ends at the payload end
    const uint8_t* idx = s + v->off_index;
    if (r32(idx) != 0) return bad(why, "tile index must start at 0");
    uint64_t prev = 0;
    for (uint32_t i = 1; i <= v->n_tiles; ++i) {
        uint64_t cur = r32(idx + 4 * (uint64_t)i);
        if (cur < prev + kLanes) return bad(why, "tile offsets not increasing by at least the 32 states");
        prev = cur;
    }
    if (4 * prev != v->payload_len) return bad(why, "tile index does not end at the payload end");
    if (crc32(s + v->off_payload, v->payload_len) != r32(s + kPayloadCrc)) return bad(why, "payload CRC-32 mismatch");
    if (meta_crc32(s, v->off_raw, v->raw_len, v->off_payload) != r32(s + kMetaCrc))
        return bad(why, "metadata CRC-32 mismatch (header, row metadata, tables or tile index damaged)");
    if (lossy)
        for (int64_t r = 0; r < v->rows; ++r) {
            float sc = rf32(s + v->off_scale + 4 * r);
            if (!(std::isfinite(sc) && sc >= 0.0f)) return bad(why, "row scale not finite and >= 0");
        }
    // an intact stream wider than the encoders write (they refuse cols >= 2^28): the decode
    // kernels address an output row through a buffer resource of cols x element bytes (< 2^31)
    if (v->cols >= (1ll << 28)) {
        if (why) *why = "stream with 2^28 or more columns (beyond the supported width)";
        return EP_ERANGE;
    }
    return EP_OK;
}

void fill_info(const StreamView& v, ep_info* info) {
    std::memset(info, 0, sizeof *info);
    info->rows = v.rows;
    info->cols = v.cols;
    info->mode = v.mode;
    info->src_dtype = v.dtype;
    info->tile_rows = v.tile_rows;
    info->layout = v.layout;
    info->prob_bits = v.prob_bits;
    info->n_tiles = v.n_tiles;
    info->n_escapes = v.n_escapes;
    info->step = v.step;
    info->target_bpp = v.target;
    info->total_bytes = v.len;
    info->payload_bytes = v.payload_len + v.raw_len;
    info->state_bytes = 4ull * kLanes * v.n_tiles;
    info->meta_bytes = v.len - info->payload_bytes;
    info->actual_bpp = v.rows * v.cols > 0 ? 8.0 * (double)v.len / ((double)v.rows * (double)v.cols) : 0.0;
}

}  // namespace ep
