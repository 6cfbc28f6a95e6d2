// Internal declarations shared by the host encoder, the stream validator, the C ABI and the
// kernel launchers of the MI355X tile-rANS codec.
//
// Stream layout (EPK1, little-endian). A 128-byte header, then sections that each start on a
// 16-byte boundary: row scales f32[R] and row max |q| u16[R] (lossy only), the symbol tables
// (per table: i16 window start, u16 window width S, u16 escape frequency, u16 freq[S]), the tile
// index u32[n_tiles + 1] (offsets in 4-byte units from the payload start) and the payload.
// A tile is 32 u32 rANS states followed by its u16 words (plus one zero pad word when their
// count is odd). An exponent-coded lossless BF16 stream also holds a raw plane u8[Rp][Cp] of
// (sign << 7) | mantissa bytes between the index and the payload (offset and CRC-32 in header
// bytes 96 and 104, zero in the other modes). The pages fix none of this; it is this codec's own
// container for tile-wise entropy coding where every tile decodes on its own (EntroPack paper,
// Abstract).
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <functional>
#include <new>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "entropack.h"

namespace ep {

constexpr int kLanes = 32;             // interleaved rANS states per tile
constexpr int kTileCols = 256;         // columns per tile: 32 lanes x one 8-wide E8 block
constexpr int kHeaderBytes = 128;
constexpr int kLossyTables = 17;       // coset bit + 8 coordinate positions x 2 cosets
constexpr int kEscape = 255;           // escape symbol of the lossy coordinate tables
constexpr uint32_t kRansLow = 1u << 16;

// header field offsets
enum HeaderField : int {
    kMagic = 0, kVersion = 4, kMode = 6, kDtype = 7, kRows = 8, kCols = 12, kTileRows = 16,
    kTileColsField = 18, kLanesField = 20, kProbBits = 22, kNumTables = 23, kStep = 24,
    kTarget = 28, kNumTiles = 32, kNumEscapes = 36, kOffScale = 40, kOffQmax = 48,
    kOffTables = 56, kOffIndex = 64, kOffPayload = 72, kTotalLen = 80, kPayloadCrc = 88,
    kOffRaw = 96, kRawCrc = 104, kMetaCrc = 112, kLayout = 116
};
constexpr int kFormatVersion = 2;      // 2: the metadata CRC-32 at byte 112

// Which block of a tile lane l codes at block step s (a tile is tile_rows x 32 blocks of 8
// columns, coded in tile_rows block steps). The pages interleave 32 states per tile without fixing
// this (reading R27). Layout 0: tile row s, block column l. Layout 1: tile row l mod tile_rows,
// block column (32 / tile_rows) s + l / tile_rows, so every block step covers all tile rows: at
// step s of a 16-row tile pair a wave holds a 16 x 32 block, one MFMA B operand. (constexpr:
// callable from device code too.)
constexpr void block_of(int layout, int tile_rows, int l, int s, int* rr, int* kk) {
    if (layout == 0) {
        *rr = s;
        *kk = l;
    } else {
        *rr = l % tile_rows;
        *kk = (kLanes / tile_rows) * s + l / tile_rows;
    }
}

struct Table {
    int32_t lo = 0;        // first coordinate value of the window (lossless: 0)
    int32_t width = 1;     // window width S
    uint32_t freq[256];    // normalized frequency per symbol (escape at 255 for lossy tables)
};

// A malloc-backed byte buffer: streams are built in place and handed to the caller, who frees
// them with ep_free, so no copy of a stream is made on the way out.
struct Bytes {
    uint8_t* p = nullptr;
    size_t n = 0;
    Bytes() = default;
    Bytes(const Bytes&) = delete;
    Bytes& operator=(const Bytes&) = delete;
    ~Bytes() { std::free(p); }
    // size uninitialized bytes; throws std::bad_alloc when the allocation fails
    void allocate(size_t size) {
        std::free(p);
        p = static_cast<uint8_t*>(std::malloc(size ? size : 1));
        n = p ? size : 0;
        if (!p) throw std::bad_alloc();
    }
    uint8_t* data() { return p; }
    size_t size() const { return n; }
    uint8_t* release() {
        uint8_t* r = p;
        p = nullptr;
        n = 0;
        return r;
    }
};

// A validated stream (views into the caller's bytes).
struct StreamView {
    const uint8_t* base = nullptr;
    size_t len = 0;
    int mode = 0, dtype = 0, tile_rows = 16, prob_bits = 12, n_tables = 0;
    int layout = 0;                      // lossy tile layout (block_of)
    int64_t rows = 0, cols = 0, tiles_r = 0, tiles_c = 0;
    uint32_t n_tiles = 0, n_escapes = 0;
    float step = 0.0f, target = 0.0f;
    uint64_t off_scale = 0, off_qmax = 0, off_tables = 0, off_index = 0, off_payload = 0;
    uint64_t payload_len = 0;
    uint64_t off_raw = 0, raw_len = 0;   // exponent-coded mode: raw plane [Rp][Cp]
    std::vector<Table> tables;
};

int element_bytes(int dtype);
uint32_t crc32(const uint8_t* p, size_t n);
// CRC-32 of every stream byte outside the payload, the raw plane (exponent-coded mode; raw_len 0
// otherwise) and the metadata CRC field itself: header bytes [0, 112) and [116, 128), the row
// metadata, tables, tile index and all padding. Together with the payload and raw-plane CRCs it
// makes every bit of a stream checked.
uint32_t meta_crc32(const uint8_t* s, uint64_t off_raw, uint64_t raw_len, uint64_t off_payload);

// Validation (host). Returns EP_OK or EP_ECORRUPT with a message in *why.
ep_status parse_stream(const uint8_t* s, size_t len, StreamView* out, std::string* why);
void fill_info(const StreamView& v, ep_info* info);

// Host encoder.
ep_status encode(const void* w, int dtype, int64_t rows, int64_t cols, const ep_encode_opts& o,
                 Bytes* out, std::string* why);

// Pieces of the host encoder that the device encoder shares (same arithmetic, so that both
// produce the same bytes).
constexpr int kSampleBlocks = 65536;   // rate-search sample
constexpr int kSearchIters = 48;       // log-bisection steps of the rate search
constexpr int32_t kValueSpan = 1 << 15;
bool normalize_frequencies(const uint64_t cnt[256], int n, uint32_t f[256]);
double sample_estimate(const uint64_t (*cnt)[256], const uint64_t* totals, int64_t sb);
float choose_step(double U, double target, const std::function<double(double)>& est);
// Header, row metadata, tables and tile index of a lossy stream whose payload (payload_len bytes,
// CRC-32 payload_crc) the caller writes itself at the returned offset of *out.
uint64_t serialize_lossy(int dt, int64_t R, int64_t C, int tile_rows, int layout, int n, const std::vector<Table>& tables,
                         float step, float target, const std::vector<float>& scale, const std::vector<uint16_t>& qmax,
                         uint64_t payload_len, std::vector<uint32_t>&& offsets, uint32_t n_esc, uint32_t payload_crc,
                         Bytes* out);

// Device encoder (lossy mode): the same stream as encode() from a weight in device memory.
ep_status encode_lossy_device(const void* dev_w, int dt, int64_t rows, int64_t cols, const ep_encode_opts& o,
                              hipStream_t stream, Bytes* out, std::string* why);

}  // namespace ep
