// C ABI of the tile-rANS weight codec: argument checks, stream upload, and kernel dispatch.
// The calls and their contracts are documented in include/entropack.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "entropack.h"
#include "ep_internal.h"
#include "fused.h"
#include "gemm.h"
#include "kernels.h"
#include "static_scratch.h"

struct ep_handle {
    ep::StreamView view;        // header fields and tables (the view's byte pointers are not kept)
    ep_info info;
    uint8_t* dev = nullptr;     // one allocation: stream copy | table blob | error flag
    size_t stream_off = 0, tables_off = 0, err_off = 0, bytes = 0;
    int device = 0;
};

namespace {

thread_local std::string g_err;

ep_status fail(ep_status st, const std::string& msg) {
    try {
        g_err = msg;
    } catch (...) {
        g_err.clear();                             // no memory for the message: keep the status
    }
    return st;
}

// Every exported call runs its body through this, so that no C++ exception crosses the C ABI: a
// failed host allocation becomes EP_ENOMEM, anything else EP_EINVAL with its message.
template <class F>
ep_status guarded(F&& body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(EP_ENOMEM, "host allocation failed");
    } catch (const std::exception& e) {
        return fail(EP_EINVAL, e.what());
    } catch (...) {
        return fail(EP_EINVAL, "unexpected error");
    }
}

ep_status hip_fail(hipError_t e, const char* what) {
    return fail(e == hipErrorOutOfMemory ? EP_ENOMEM : EP_EHIP,
                std::string(what) + ": " + hipGetErrorString(e));
}

size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device decode tables (layout in kernels.h): per table, the slot -> symbol LUT and one 8-byte
// entry per symbol holding its frequency (bit 31: escape), its cumulative frequency plus the LDS
// offset of the lookup's LUT group, and the value the symbol stands for.
std::vector<uint8_t> build_tables(const ep::StreamView& v) {
    const int n = v.prob_bits;
    const size_t M = (size_t)1 << n;
    std::vector<uint8_t> blob(ep::table_blob_bytes(v.n_tables, n), 0);
    uint8_t* lut = blob.data();
    uint32_t* ent = reinterpret_cast<uint32_t*>(blob.data() + ((size_t)v.n_tables << n));
    for (int t = 0; t < v.n_tables; ++t) {
        const ep::Table& T = v.tables[t];
        const bool coord = v.mode == EP_MODE_LOSSY_E8 && t > 0;
        const uint32_t base = coord ? (uint32_t)((t - 1) & 1) << n : 0u;
        uint32_t c = 0;
        for (int s = 0; s < 256; ++s) {
            const uint32_t f = T.freq[s];
            int32_t value;
            if (v.mode != EP_MODE_LOSSY_E8) value = s;
            else if (t == 0) value = T.lo + s;
            else value = (s == ep::kEscape || s >= T.width) ? 0 : 2 * (T.lo + s) + ((t - 1) & 1);
            ent[2 * ((size_t)t * 256 + s)] = f | (coord && s == ep::kEscape ? 0x80000000u : 0u);
            ent[2 * ((size_t)t * 256 + s) + 1] = ((c + base) & 0xFFFFu) | (uint32_t)(uint16_t)(int16_t)value << 16;
            for (uint32_t k = 0; k < f; ++k) lut[(size_t)t * M + c + k] = (uint8_t)s;
            c += f;
        }
    }
    return blob;
}

ep::MatDesc desc_for(const ep_handle* h, int container, void* out, float* scale) {
    const ep::StreamView& v = h->view;
    const uint8_t* s = h->dev + h->stream_off;
    ep::MatDesc d{};
    d.payload = reinterpret_cast<const uint32_t*>(s + v.off_payload);
    d.index = reinterpret_cast<const uint32_t*>(s + v.off_index);
    d.row_scale = reinterpret_cast<const float*>(s + v.off_scale);
    d.row_qmax = reinterpret_cast<const uint16_t*>(s + v.off_qmax);
    d.raw = v.mode == EP_MODE_LOSSLESS_EXP ? s + v.off_raw : nullptr;
    d.tables = h->dev + h->tables_off;
    d.out = out;
    d.scale_out = scale;
    d.err = reinterpret_cast<int*>(h->dev + h->err_off);
    d.rows = (uint32_t)v.rows;
    d.cols = (uint32_t)v.cols;
    d.tiles_c = (uint32_t)v.tiles_c;
    d.pairs_c = (uint32_t)((v.tiles_c + 1) / 2);
    d.payload_bytes = (uint32_t)v.payload_len;
    d.step = v.step;
    d.prob_bits = (uint8_t)v.prob_bits;
    d.tile_rows = (uint8_t)v.tile_rows;
    d.layout = (uint8_t)v.layout;
    d.container = (uint8_t)container;
    d.n_tables = (uint8_t)v.n_tables;
    d.mode = (uint8_t)v.mode;
    d.pair_cost = ep::pair_cost_of(v.mode, v.tile_rows, v.n_tables);
    if (v.mode == EP_MODE_LOSSY_E8)
        for (int t = 1; t < v.n_tables && t <= 16; ++t)
            if (v.tables[t].freq[ep::kEscape] != 0) d.esc_tables |= (uint16_t)(1u << (t - 1));
    return d;
}

// Launch the matrices in groups of at most kMaxGroup.
hipError_t launch_all(const std::vector<ep::MatDesc>& ds, hipStream_t stream) {
    for (size_t i = 0; i < ds.size(); i += ep::kMaxGroup) {
        const int n = (int)std::min<size_t>(ep::kMaxGroup, ds.size() - i);
        hipError_t e = ep::launch_group(ds.data() + i, n, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Library-owned device workspaces of the linear forwards, one per (device, stream). A forward
// holds the pool's lock from taking its workspace until its launches are queued and an event is
// recorded behind them (WsLease::queued). A buffer is freed only after its entry's event has
// completed: when it must grow, or when its device has more than kMaxWsPerDevice entries and it
// is the least recently used one (the stream it served may be gone; its event is still valid).
// So no queued launch reads freed memory, and no caller holds a pointer that another frees.
struct WsEntry {
    int device;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
    hipEvent_t done;            // recorded behind the last forward that used the buffer
    uint64_t tick;              // last use, for eviction
};
constexpr int kMaxWsPerDevice = 4;
std::mutex g_ws_mu;
std::vector<WsEntry> g_ws;
uint64_t g_ws_tick = 0;

hipError_t ws_retire(WsEntry& e) {
    hipError_t r = hipSuccess;
    if (e.done) {
        r = hipEventSynchronize(e.done);
        const hipError_t r2 = hipEventDestroy(e.done);
        if (r == hipSuccess) r = r2;
        e.done = nullptr;
    }
    if (e.ptr) {
        const hipError_t r2 = hipFree(e.ptr);
        if (r == hipSuccess) r = r2;
        e.ptr = nullptr;
    }
    e.bytes = 0;
    return r;
}

// Device scratch of one forward: the pool's buffer for (device, stream), held under the pool
// lock, or (no-allocation entry point) the caller-independent static buffer of the device.
struct WsLease {
    std::unique_lock<std::mutex> lock;
    WsEntry* entry = nullptr;   // null for the static buffer
    hipStream_t stream = nullptr;
    void* ptr = nullptr;
    size_t bytes = 0;
    bool recorded = false;
    // After the forward's launches are queued: mark the buffer as in use by them.
    hipError_t queued() {
        recorded = true;
        return entry ? hipEventRecord(entry->done, stream) : hipSuccess;
    }
    // A forward that stops on an error after some launches were queued still marks the buffer
    // (before the lock, declared first, is released), so that a later grow waits for them.
    ~WsLease() {
        if (entry && !recorded) (void)hipEventRecord(entry->done, stream);
    }
};

hipError_t ws_acquire(int device, hipStream_t stream, size_t need, WsLease* L) {
    L->lock = std::unique_lock<std::mutex>(g_ws_mu);
    L->stream = stream;
    WsEntry* e = nullptr;
    for (WsEntry& x : g_ws)
        if (x.device == device && x.stream == stream) e = &x;
    if (!e) {
        int count = 0;
        size_t lru = g_ws.size();
        for (size_t i = 0; i < g_ws.size(); ++i) {
            if (g_ws[i].device != device) continue;
            ++count;
            if (lru == g_ws.size() || g_ws[i].tick < g_ws[lru].tick) lru = i;
        }
        if (count >= kMaxWsPerDevice) {
            hipError_t r = ws_retire(g_ws[lru]);
            g_ws.erase(g_ws.begin() + (std::ptrdiff_t)lru);
            if (r != hipSuccess) return r;
        }
        WsEntry n{device, stream, nullptr, 0, nullptr, 0};
        hipError_t r = hipEventCreateWithFlags(&n.done, hipEventDisableTiming);
        if (r != hipSuccess) return r;
        g_ws.push_back(n);
        e = &g_ws.back();
    }
    if (e->bytes < need) {
        // earlier forwards on this stream may still read the old buffer: wait for them
        hipError_t r = hipEventSynchronize(e->done);
        if (r == hipSuccess && e->ptr) r = hipFree(e->ptr);
        e->ptr = nullptr;
        e->bytes = 0;
        if (r != hipSuccess) return r;
        r = hipMalloc(&e->ptr, need);
        if (r != hipSuccess) {
            e->ptr = nullptr;
            return r;
        }
        e->bytes = need;
    }
    e->tick = ++g_ws_tick;
    L->entry = e;
    L->ptr = e->ptr;
    L->bytes = e->bytes;
    return hipSuccess;
}

bool container_ok(const ep_handle* h, int ct) {
    if (h->view.mode != EP_MODE_LOSSY_E8) return ct == h->view.dtype;
    return ct == EP_BF16 || ct == EP_F16 || ct == EP_F8E4M3 || ct == EP_I8;
}

// A handle's device copy lives on the device it was uploaded to; a kernel on another device must
// not be handed its pointers.
ep_status on_its_device(const ep_handle* h) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != h->device)
        return fail(EP_EINVAL, "the handle was uploaded to device " + std::to_string(h->device) + " but device " +
                                   std::to_string(dev) + " is current");
    return EP_OK;
}

ep_status check_decode_args(const ep_handle* h, ep_dtype ct, void* out, float* scale) {
    if (!h) return fail(EP_EINVAL, "null handle");
    if (ep_status st = on_its_device(h); st != EP_OK) return st;
    if (!container_ok(h, ct))
        return fail(EP_EUNSUPPORTED, h->view.mode != EP_MODE_LOSSY_E8
                                         ? "a lossless stream decodes only to its own dtype"
                                         : "lossy streams decode to BF16, F16, F8E4M3 or I8");
    if (!out && h->view.rows * h->view.cols > 0) return fail(EP_EINVAL, "null output pointer");
    const bool wants_scale = h->view.mode == EP_MODE_LOSSY_E8 && (ct == EP_F8E4M3 || ct == EP_I8);
    if (wants_scale && !scale && h->view.rows > 0) return fail(EP_EINVAL, "F8E4M3 and I8 need a row-scale output");
    if (!wants_scale && scale) return fail(EP_EINVAL, "row-scale output given for a container without one");
    return EP_OK;
}

// The device's static scratch for the no-allocation forward: the whole buffer, or EP_ERANGE when
// a call needs more than it holds.
ep_status take_static(size_t need, WsLease* L) {
    if (need > ep::kStaticScratchBytes)
        return fail(EP_ERANGE, "the call needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                   std::to_string(ep::kStaticScratchBytes) + " of the static buffer");
    void* p = nullptr;
    hipError_t e = ep::static_scratch(&p);
    if (e != hipSuccess) return hip_fail(e, "locating the static scratch buffer");
    L->entry = nullptr;
    L->ptr = p;
    L->bytes = ep::kStaticScratchBytes;
    return EP_OK;
}

// Whether an M x N x K product of a decoded slice (or the plain FP8 GEMM) goes to hipBLASLt rather
// than the library's own kernel: from 512 rows always; above the fused kernel's 64 rows when K is
// at most 4096 (the own kernel's split-K only pays on long K); from 256 rows when N <= 4096 (its
// 256 x 256 tiles then need split-K to fill the CUs). Measured as whole forwards on 13 layer
// shapes (2048^2 ... 8192^2 and the DiT-like 11520 x 3840, 10240 x 3840, 3840 x 10240, 3840^2):
// at 512 and 768 rows hipBLASLt cuts the summed time by 14% and 22%; from 65 to 384 rows the
// K <= 4096 part cuts it by 4-9% (BF16) and 1-5% (FP8), e.g. 11520 x 3840 at 128 rows 124 -> 99 us;
// the own kernel stays faster on long K with few rows (8192^2 at 256 rows: 88 against 102 us,
// 4096 x 16384 at 128 rows: 97 against 121 us). Every repeat gave the same bits.
bool use_gemm_library(int64_t M, int64_t N, int64_t K) {
    return M >= 512 || (M > 64 && K <= 4096) || (M >= 256 && N <= 4096);
}

// Largest BF16 slice of a layer's weight decoded at once (see linear_forward), and the hipBLASLt
// workspace of a slice GEMM.
constexpr size_t kSliceBytes = 128u << 20;
constexpr size_t kLtWorkspace = 32u << 20;

// Compressed linear forward. The weight is decoded once per call, one slice of output rows at a
// time, into the forward's scratch, and each slice's GEMM writes its columns of Y. A slice of at
// most kSliceBytes is large enough to keep every CU's decode block busy and, with the
// activations, small enough to stay in the 256 MB Infinity Cache between the decode that writes
// it and the GEMM that reads it (128 MiB measured best against 64 and 256 for M = 256 ... 4096).
// `fixed`: the scratch is the device's static buffer (no allocation), whose size bounds the slice.
ep_status linear_forward(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias, void* dev_y,
                         hipStream_t s, bool fixed) {
    if (!w) return fail(EP_EINVAL, "null handle");
    if (ep_status st = on_its_device(w); st != EP_OK) return st;
    if (w->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
    const int64_t N = w->view.rows, K = w->view.cols;
    if (M < 0) return fail(EP_EINVAL, "negative M");
    if (M == 0 || N == 0) return EP_OK;
    if (!dev_y || (K > 0 && !dev_x)) return fail(EP_EINVAL, "null pointer");
    if (M > INT32_MAX || N > INT32_MAX) return fail(EP_ERANGE, "M and out_features must be below 2^31");
    if (K % 8) return fail(EP_EINVAL, "in_features must be a multiple of 8");
    if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
    WsLease ws;
    if (K == 0 || (M <= 4 && w->view.layout == 0)) {
        // a few activation rows: decoding fused with the matrix-vector products, the weight never
        // written out; fp32 partial sums per tile pair column in the scratch, then their sum in
        // column order, rounded (+ bias) to BF16 (also the empty product of in_features 0)
        const int64_t pcs = K > 0 ? (int64_t)((w->view.tiles_c + 1) / 2) : 0;
        const size_t need = std::max<size_t>(256, sizeof(float) * (size_t)pcs * (size_t)M * (size_t)N);
        if (fixed) {
            if (ep_status st = take_static(need, &ws); st != EP_OK) return st;
        } else if ((he = ws_acquire(dev, s, need, &ws)) != hipSuccess) {
            return hip_fail(he, "hipMalloc for the linear forward workspace");
        }
        float* part = static_cast<float*>(ws.ptr);
        ep::MatDesc d = desc_for(w, M == 1 ? ep::CT_GEMV1 : M == 2 ? ep::CT_GEMV2 : ep::CT_GEMV4, part, nullptr);
        d.gemv_x = static_cast<const uint16_t*>(dev_x);
        d.gemv_m = (uint8_t)M;
        hipError_t e = pcs > 0 ? ep::launch_gemv(d, s) : hipSuccess;
        if (e == hipSuccess)
            e = ep::launch_gemv_finish(part, pcs, static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y), M,
                                       N, s);
        if (e == hipSuccess) e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "fused matrix-vector launch");
    }
    if (const ep::MatDesc d = desc_for(w, ep::CT_BF16, nullptr, nullptr); ep::fused_fits(d, M)) {
        // up to 16 activation rows (64 in the row layout): every tile pair decoded straight into
        // the B operand of the BF16 MFMA (through LDS in layout 0, from the decoder's registers in
        // the row layout), its fp32 partial sums in the scratch, then summed in order
        const size_t need = ep::fused_partial_bytes(d, M);
        if (fixed) {
            if (ep_status st = take_static(need, &ws); st != EP_OK) return st;
        } else if ((he = ws_acquire(dev, s, need, &ws)) != hipSuccess) {
            return hip_fail(he, "hipMalloc for the linear forward workspace");
        }
        hipError_t e = ep::launch_fused(d, static_cast<const uint16_t*>(dev_x), M, static_cast<float*>(ws.ptr),
                                        static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y), s);
        if (e == hipSuccess) e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "fused decode + MFMA launch");
    }
    const int tr = w->view.tile_rows;
    // Slices multiplied by hipBLASLt where use_gemm_library says so (its tuned kernels beat the own
    // 256 x 256 one at prefill sizes: 4096 x 8192 x 8192, 363 against 441 us); elsewhere the own
    // kernel, split-K when its tiles cannot fill the CUs. Not in the no-allocation variant: the
    // library's handle allocates on first use.
    const bool lt = !fixed && use_gemm_library(M, N, K);
    // K splits of the GEMM, chosen for the whole layer so that every slice adds its partial sums in
    // the same order; the split partial tiles of a slice follow its decoded rows in the scratch
    const int splits = lt ? 1 : ep::gemm_splits((int)M, (int)N, (int)K);
    const size_t part_per_row = splits > 1 ? (size_t)splits * (size_t)M * sizeof(float) : 0;
    int64_t slice = (int64_t)(fixed ? ep::kStaticScratchBytes / (2 * (size_t)K + part_per_row)
                                    : kSliceBytes / (2 * (size_t)K)) / tr * tr;
    if (slice < tr) {
        if (fixed) return fail(EP_ERANGE, "in_features too large for the static scratch (one 16-row slice must fit)");
        slice = tr;
    }
    if (slice > N) slice = (N + tr - 1) / tr * tr;
    const size_t slice_bytes = up((size_t)slice * (size_t)K * 2, 256);
    const size_t o_lt = up(slice_bytes + (size_t)slice * part_per_row, 256);
    const size_t need = o_lt + (lt ? kLtWorkspace : 0);
    if (fixed) {
        if (ep_status st = take_static(need, &ws); st != EP_OK) return st;
    } else if ((he = ws_acquire(dev, s, need, &ws)) != hipSuccess) {
        return hip_fail(he, "hipMalloc for the linear forward workspace");
    }
    uint16_t* scratch = static_cast<uint16_t*>(ws.ptr);
    const ep::MatDesc full = desc_for(w, ep::CT_BF16, scratch, nullptr);
    for (int64_t r0 = 0; r0 < N; r0 += slice) {
        const int64_t rows = std::min<int64_t>(slice, N - r0);
        ep::MatDesc d = full;                  // rows r0 .. r0 + rows of the weight
        d.index += (size_t)(r0 / tr) * w->view.tiles_c;
        d.row_scale += r0;
        d.row_qmax += r0;
        d.rows = (uint32_t)rows;
        hipError_t e = ep::launch_group(&d, 1, s);
        if (e != hipSuccess) return hip_fail(e, "slice decode launch");
        ep::GemmArgs g{static_cast<const uint16_t*>(dev_x), scratch,
                       dev_bias ? static_cast<const uint16_t*>(dev_bias) + r0 : nullptr,
                       static_cast<uint16_t*>(dev_y) + r0, (int)M, (int)rows, (int)K, (int)K, (int)K, (int)N};
        g.splits = splits;
        g.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws.ptr) + slice_bytes);
        g.part_bytes = (size_t)slice * part_per_row;
        e = lt ? ep::lt_gemm(g, reinterpret_cast<uint8_t*>(ws.ptr) + o_lt, kLtWorkspace, s) : hipErrorNotSupported;
        if (e == hipErrorNotSupported) e = ep::launch_gemm(g, s);
        if (e != hipSuccess) return hip_fail(e, "slice gemm launch");
    }
    he = ws.queued();
    return he == hipSuccess ? EP_OK : hip_fail(he, "recording the workspace event");
}

}  // namespace

extern "C" {

const char* ep_last_error(void) { return g_err.c_str(); }

const char* ep_version(void) { return "entropack-mi355x 0.1 (EPK1, gfx950)"; }

void ep_free(void* p) { std::free(p); }

ep_status ep_compress(const void* host_w, ep_dtype src, int64_t rows, int64_t cols, const ep_encode_opts* opts,
                      uint8_t** out_stream, size_t* out_len, double* actual_bpp) {
    return guarded([&]() -> ep_status {
        if (!out_stream || !out_len) return fail(EP_EINVAL, "null output pointer");
        if (rows < 0 || cols < 0) return fail(EP_EINVAL, "negative shape");
        if (rows * cols > 0 && !host_w) return fail(EP_EINVAL, "null input");
        if (rows > 0xFFFFFFFFll || cols >= (1ll << 28)) return fail(EP_ERANGE, "shape too large (cols must be < 2^28)");
        ep_encode_opts o = opts ? *opts : ep_encode_opts{EP_MODE_LOSSY_E8, 4.0, 12, 16, 0, 0};
        if (o.prob_bits < 10 || o.prob_bits > 12) return fail(EP_EINVAL, "prob_bits must be 10..12");
        if (o.tile_rows != 16 && o.tile_rows != 32) return fail(EP_EINVAL, "tile_rows must be 16 or 32");
        if (o.layout < 0 || o.layout > 1 || (o.layout != 0 && o.mode != EP_MODE_LOSSY_E8))
            return fail(EP_EINVAL, "layout must be 0, or 1 in the lossy mode");
        if (o.mode == EP_MODE_LOSSY_E8) {
            if (src != EP_F32 && src != EP_BF16 && src != EP_F16)
                return fail(EP_EUNSUPPORTED, "lossy mode takes F32, BF16 or F16 input");
            if (!(o.target_bpp > 0.0 && o.target_bpp <= 32.0)) return fail(EP_EINVAL, "target_bpp must be in (0, 32]");
        } else if (o.mode == EP_MODE_LOSSLESS) {
            if (ep::element_bytes(src) == 0) return fail(EP_EUNSUPPORTED, "unknown dtype");
        } else if (o.mode == EP_MODE_LOSSLESS_EXP) {
            if (src != EP_BF16) return fail(EP_EUNSUPPORTED, "exponent-coded lossless mode takes BF16 input");
        } else {
            return fail(EP_EINVAL, "unknown mode");
        }
        ep::Bytes buf;
        std::string why;
        ep_status st;
        try {
            st = ep::encode(host_w, src, rows, cols, o, &buf, &why);
        } catch (const std::bad_alloc&) {
            return fail(EP_ENOMEM, "host allocation failed while encoding");
        }
        if (st != EP_OK) return fail(st, why);
        const size_t len = buf.size();
        *out_stream = buf.release();
        *out_len = len;
        if (actual_bpp) *actual_bpp = rows * cols > 0 ? 8.0 * (double)len / ((double)rows * (double)cols) : 0.0;
        return EP_OK;
    });
}

ep_status ep_stream_info(const uint8_t* host_stream, size_t len, ep_info* out) {
    return guarded([&]() -> ep_status {
        if (!host_stream || !out) return fail(EP_EINVAL, "null pointer");
        ep::StreamView v;
        std::string why;
        ep_status st = ep::parse_stream(host_stream, len, &v, &why);
        if (st != EP_OK) return fail(st, why);
        ep::fill_info(v, out);
        return EP_OK;
    });
}

ep_status ep_upload(const uint8_t* host_stream, size_t len, void* hip_stream, ep_handle** out) {
    return guarded([&]() -> ep_status {
        if (!host_stream || !out) return fail(EP_EINVAL, "null pointer");
        *out = nullptr;
        std::unique_ptr<ep_handle> h(new ep_handle());   // freed on every early return or throw
        std::string why;
        ep_status st = ep::parse_stream(host_stream, len, &h->view, &why);
        if (st != EP_OK) return fail(st, why);
        ep::fill_info(h->view, &h->info);
        // the decode kernels address a stream's tile payload through one buffer resource, whose
        // size field is 32 bits
        if (h->view.payload_len >= (1ull << 32))
            return fail(EP_ERANGE, "tile payload of 4 GiB or more: split the matrix into several streams");
        std::vector<uint8_t> blob = build_tables(h->view);
        h->stream_off = 0;
        h->tables_off = up(len, 256);
        h->err_off = up(h->tables_off + blob.size(), 256);
        h->bytes = h->err_off + 256;
        hipError_t e = hipGetDevice(&h->device);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        e = hipMalloc(reinterpret_cast<void**>(&h->dev), h->bytes);
        if (e != hipSuccess) {
            h->dev = nullptr;
            return hip_fail(e, "hipMalloc for the stream");
        }
        e = hipMemcpyAsync(h->dev + h->stream_off, host_stream, len, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipMemcpyAsync(h->dev + h->tables_off, blob.data(), blob.size(), hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipMemsetAsync(h->dev + h->err_off, 0, 256, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) {
            (void)hipFree(h->dev);
            return hip_fail(e, "copying the stream to the device");
        }
        // the view's pointers referred to the caller's bytes: drop them
        h->view.base = nullptr;
        *out = h.release();
        return EP_OK;
    });
}

ep_status ep_handle_info(const ep_handle* h, ep_info* out) {
    return guarded([&]() -> ep_status {
        if (!h || !out) return fail(EP_EINVAL, "null pointer");
        *out = h->info;
        return EP_OK;
    });
}

void ep_release(ep_handle* h) {
    if (!h) return;
    if (h->dev) (void)hipFree(h->dev);
    delete h;
}

ep_status ep_decompress(const ep_handle* h, ep_dtype container, void* dev_out, float* dev_row_scale, void* hip_stream) {
    return guarded([&]() -> ep_status {
        ep_status st = check_decode_args(h, container, dev_out, dev_row_scale);
        if (st != EP_OK) return st;
        std::vector<ep::MatDesc> one{desc_for(h, (int)container, dev_out, dev_row_scale)};
        hipError_t e = launch_all(one, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return hip_fail(e, "decode launch");
        return EP_OK;
    });
}

ep_status ep_decompress_many(const ep_handle* const* hs, const ep_dtype* containers, void* const* dev_outs,
                             float* const* dev_row_scales, int count, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (count < 0 || (count > 0 && (!hs || !containers || !dev_outs))) return fail(EP_EINVAL, "null array");
        std::vector<ep::MatDesc> ds;
        for (int i = 0; i < count; ++i) {
            float* sc = dev_row_scales ? dev_row_scales[i] : nullptr;
            ep_status st = check_decode_args(hs[i], containers[i], dev_outs[i], sc);
            if (st != EP_OK) return fail(st, "matrix " + std::to_string(i) + ": " + g_err);
            ds.push_back(desc_for(hs[i], (int)containers[i], dev_outs[i], sc));
        }
        hipError_t e = launch_all(ds, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return hip_fail(e, "grouped decode launch");
        return EP_OK;
    });
}

ep_status ep_decode_symbols(const ep_handle* h, int16_t* dev_q, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (!h) return fail(EP_EINVAL, "null handle");
        if (ep_status st = on_its_device(h); st != EP_OK) return st;
        if (h->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "symbols exist only for lossy streams");
        if (!dev_q && h->view.rows * h->view.cols > 0) return fail(EP_EINVAL, "null output pointer");
        std::vector<ep::MatDesc> one{desc_for(h, ep::CT_Q16, dev_q, nullptr)};
        hipError_t e = launch_all(one, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return hip_fail(e, "decode launch");
        return EP_OK;
    });
}

ep_status ep_handle_check(ep_handle* h, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (!h) return fail(EP_EINVAL, "null handle");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        int flag = 0;
        hipError_t e = hipMemcpyAsync(&flag, h->dev + h->err_off, sizeof flag, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "reading the device error flag");
        if (flag) {
            e = hipMemsetAsync(h->dev + h->err_off, 0, sizeof(int), s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            return fail(EP_EDEVICE, std::string("decode kernel flagged the stream:") + (flag & 1 ? " word count" : "") +
                                        (flag & 2 ? " final state" : "") + (flag & 4 ? " kernel LDS layout" : ""));
        }
        return EP_OK;
    });
}

ep_status ep_gemm_bf16(const void* dev_x, const void* dev_w, int64_t M, int64_t N, int64_t K, void* dev_y,
                       void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (M < 0 || N < 0 || K < 0) return fail(EP_EINVAL, "negative size");
        if (M == 0 || N == 0) return EP_OK;
        if (!dev_x || !dev_w || !dev_y) return fail(EP_EINVAL, "null pointer");
        if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(EP_ERANGE, "M, N and K must be below 2^31");
        if (K % 8) return fail(EP_EINVAL, "K must be a multiple of 8");
        if ((reinterpret_cast<uintptr_t>(dev_x) | reinterpret_cast<uintptr_t>(dev_w)) & 15)
            return fail(EP_EINVAL, "X and W must be 16-byte aligned");
        ep::GemmArgs g{static_cast<const uint16_t*>(dev_x), static_cast<const uint16_t*>(dev_w), nullptr,
                       static_cast<uint16_t*>(dev_y), (int)M, (int)N, (int)K, (int)K, (int)K, (int)N};
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        g.splits = ep::gemm_splits((int)M, (int)N, (int)K);
        WsLease ws;
        if (g.splits > 1) {
            // the fp32 partial tiles of a split-K product live in the stream's workspace
            int dev = 0;
            hipError_t he = hipGetDevice(&dev);
            g.part_bytes = (size_t)g.splits * (size_t)M * (size_t)N * sizeof(float);
            if (he == hipSuccess) he = ws_acquire(dev, s, g.part_bytes, &ws);
            if (he != hipSuccess) return hip_fail(he, "hipMalloc for the GEMM workspace");
            g.part = static_cast<float*>(ws.ptr);
        }
        hipError_t e = ep::launch_gemm(g, s);
        if (e == hipSuccess) e = ws.queued();
        if (e != hipSuccess) return hip_fail(e, "gemm launch");
        return EP_OK;
    });
}

ep_status ep_linear_forward(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias, void* dev_y,
                            void* hip_stream) {
    return guarded([&]() -> ep_status {
        return linear_forward(w, dev_x, M, dev_bias, dev_y, static_cast<hipStream_t>(hip_stream), false);
    });
}

ep_status ep_linear_forward_many(const ep_handle* const* w, int count, const void* dev_x, int64_t M,
                                 const void* const* dev_bias, void* const* dev_y, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (count < 0 || count > ep::kMaxGroup) return fail(EP_ERANGE, "count must be 0 ... 32");
        if (count == 0) return EP_OK;
        if (!w || !dev_y) return fail(EP_EINVAL, "null pointer");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        // every layer checked before anything is queued
        for (int i = 0; i < count; ++i) {
            if (!w[i] || !dev_y[i]) return fail(EP_EINVAL, "null handle or output at layer " + std::to_string(i));
            if (ep_status st = on_its_device(w[i]); st != EP_OK) return st;
            if (w[i]->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
            if (w[i]->view.cols != w[0]->view.cols) return fail(EP_EINVAL, "the layers take inputs of different widths");
        }
        const int64_t K = w[0]->view.cols;
        if (M < 0) return fail(EP_EINVAL, "negative M");
        if (M == 0) return EP_OK;
        if (K > 0 && !dev_x) return fail(EP_EINVAL, "null pointer");
        std::vector<ep::MatDesc> ds;
        bool nonempty = true;
        for (int i = 0; i < count; ++i) {
            ds.push_back(desc_for(w[i], ep::CT_BF16, nullptr, nullptr));
            nonempty = nonempty && w[i]->view.rows > 0;
        }
        const bool fused = K > 0 && nonempty && ep::fused_many_fits(ds.data(), count, M);
        // More rows: when every layer's own forward would decode it as one whole-layer slice and
        // multiply it by hipBLASLt, the slices of all layers are decoded by one grouped launch and
        // then multiplied one by one (the same slices and GEMMs, so the same bits), while the group's
        // slices stay within the Infinity Cache's reach (192 MiB).
        bool grouped_slices = !fused && count > 1 && K > 0 && K % 8 == 0 && M > 64 && M <= INT32_MAX && dev_x &&
                              !(reinterpret_cast<uintptr_t>(dev_x) & 15);
        size_t slice_total = 0;
        for (int i = 0; i < count && grouped_slices; ++i) {
            const int64_t N = w[i]->view.rows;
            grouped_slices = N > 0 && N <= INT32_MAX && (size_t)N * (size_t)K * 2 <= kSliceBytes &&
                             use_gemm_library(M, N, K);
            slice_total += up((size_t)N * (size_t)K * 2, 256);
        }
        if (grouped_slices && slice_total <= (192u << 20)) {
            int dev = 0;
            hipError_t he = hipGetDevice(&dev);
            if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
            WsLease ws;
            if ((he = ws_acquire(dev, s, slice_total + kLtWorkspace, &ws)) != hipSuccess)
                return hip_fail(he, "hipMalloc for the linear forward workspace");
            uint8_t* base = static_cast<uint8_t*>(ws.ptr);
            std::vector<ep::MatDesc> dd;
            std::vector<uint16_t*> sl;
            size_t o = 0;
            for (int i = 0; i < count; ++i) {
                sl.push_back(reinterpret_cast<uint16_t*>(base + o));
                dd.push_back(desc_for(w[i], ep::CT_BF16, sl.back(), nullptr));
                o += up((size_t)w[i]->view.rows * (size_t)K * 2, 256);
            }
            hipError_t e = launch_all(dd, s);
            for (int i = 0; i < count && e == hipSuccess; ++i) {
                const int N = (int)w[i]->view.rows;
                ep::GemmArgs g{static_cast<const uint16_t*>(dev_x), sl[i],
                               dev_bias ? static_cast<const uint16_t*>(dev_bias[i]) : nullptr,
                               static_cast<uint16_t*>(dev_y[i]), (int)M, N, (int)K, (int)K, (int)K, N};
                g.splits = 1;
                g.part = nullptr;
                g.part_bytes = 0;
                e = ep::lt_gemm(g, base + slice_total, kLtWorkspace, s);
                if (e == hipErrorNotSupported) e = ep::launch_gemm(g, s);
            }
            if (e == hipSuccess) e = ws.queued();
            return e == hipSuccess ? EP_OK : hip_fail(e, "grouped slice decode + GEMM launch");
        }
        if (!fused) {
            // each layer's own forward, in order
            for (int i = 0; i < count; ++i)
                if (ep_status st = linear_forward(w[i], dev_x, M, dev_bias ? dev_bias[i] : nullptr, dev_y[i], s, false);
                    st != EP_OK)
                    return st;
            return EP_OK;
        }
        if (M > INT32_MAX) return fail(EP_ERANGE, "M must be below 2^31");
        if (K % 8) return fail(EP_EINVAL, "in_features must be a multiple of 8");
        if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
        int dev = 0;
        hipError_t he = hipGetDevice(&dev);
        if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
        std::vector<size_t> off(count + 1, 0);
        for (int i = 0; i < count; ++i) off[i + 1] = off[i] + up(ep::fused_partial_bytes(ds[i], M), 256);
        WsLease ws;
        if ((he = ws_acquire(dev, s, off[count], &ws)) != hipSuccess)
            return hip_fail(he, "hipMalloc for the linear forward workspace");
        std::vector<float*> parts(count);
        std::vector<const uint16_t*> bias(count);
        std::vector<uint16_t*> ys(count);
        for (int i = 0; i < count; ++i) {
            parts[i] = reinterpret_cast<float*>(static_cast<uint8_t*>(ws.ptr) + off[i]);
            bias[i] = dev_bias ? static_cast<const uint16_t*>(dev_bias[i]) : nullptr;
            ys[i] = static_cast<uint16_t*>(dev_y[i]);
        }
        hipError_t e = ep::launch_fused_many(ds.data(), count, static_cast<const uint16_t*>(dev_x), M, parts.data(),
                                             bias.data(), ys.data(), s);
        if (e == hipSuccess) e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "grouped fused decode + MFMA launch");
    });
}

ep_status ep_linear_forward_fp8_many(const ep_handle* const* w, int count, const void* dev_x, int64_t M,
                                     const void* const* dev_bias, void* const* dev_y, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (count < 0 || count > ep::kMaxGroup) return fail(EP_ERANGE, "count must be 0 ... 32");
        if (count == 0) return EP_OK;
        if (!w || !dev_y) return fail(EP_EINVAL, "null pointer");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        for (int i = 0; i < count; ++i) {
            if (!w[i] || !dev_y[i]) return fail(EP_EINVAL, "null handle or output at layer " + std::to_string(i));
            if (ep_status st = on_its_device(w[i]); st != EP_OK) return st;
            if (w[i]->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
            if (w[i]->view.cols != w[0]->view.cols) return fail(EP_EINVAL, "the layers take inputs of different widths");
        }
        const int64_t K = w[0]->view.cols;
        if (M < 0) return fail(EP_EINVAL, "negative M");
        if (M == 0) return EP_OK;
        if (K > 0 && !dev_x) return fail(EP_EINVAL, "null pointer");
        std::vector<ep::MatDesc> ds;
        bool nonempty = true;
        for (int i = 0; i < count; ++i) {
            ds.push_back(desc_for(w[i], ep::CT_F8E4M3, nullptr, nullptr));
            nonempty = nonempty && w[i]->view.rows > 0;
        }
        if (K == 0 || K % 16 || !nonempty || !ep::fused_many_fits(ds.data(), count, M)) {
            // each layer's own FP8 forward, in order
            for (int i = 0; i < count; ++i)
                if (ep_status st = ep_linear_forward_fp8(w[i], dev_x, M, dev_bias ? dev_bias[i] : nullptr, dev_y[i], hip_stream);
                    st != EP_OK)
                    return st;
            return EP_OK;
        }
        if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
        int dev = 0;
        hipError_t he = hipGetDevice(&dev);
        if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
        // workspace: X codes [M][K] | X scales [M] | each layer's fp32 partial sums
        const size_t o_xs = up((size_t)M * (size_t)K, 256);
        std::vector<size_t> off(count + 1, up(o_xs + 4 * (size_t)M, 256));
        for (int i = 0; i < count; ++i) off[i + 1] = off[i] + up(ep::fused_partial_bytes(ds[i], M), 256);
        WsLease ws;
        if ((he = ws_acquire(dev, s, off[count], &ws)) != hipSuccess)
            return hip_fail(he, "hipMalloc for the linear forward workspace");
        uint8_t* ws8 = static_cast<uint8_t*>(ws.ptr);
        float* xs = reinterpret_cast<float*>(ws8 + o_xs);
        std::vector<float*> parts(count);
        std::vector<const uint16_t*> bias(count);
        std::vector<uint16_t*> ys(count);
        for (int i = 0; i < count; ++i) {
            parts[i] = reinterpret_cast<float*>(ws8 + off[i]);
            bias[i] = dev_bias ? static_cast<const uint16_t*>(dev_bias[i]) : nullptr;
            ys[i] = static_cast<uint16_t*>(dev_y[i]);
        }
        // the activations quantized once for the group, as each layer's own forward quantizes them
        hipError_t e = ep::launch_quantize_rows_f8(static_cast<const uint16_t*>(dev_x), (int)M, (int)K, (int)K, ws8,
                                                   (int)K, xs, s);
        if (e == hipSuccess)
            e = ep::launch_fused_many_f8(ds.data(), count, ws8, xs, M, parts.data(), bias.data(), ys.data(), s);
        if (e == hipSuccess) e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "grouped fused FP8 decode + MFMA launch");
    });
}

ep_status ep_linear_forward_noalloc(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                                    void* dev_y, void* hip_stream) {
    return guarded([&]() -> ep_status {
        return linear_forward(w, dev_x, M, dev_bias, dev_y, static_cast<hipStream_t>(hip_stream), true);
    });
}

ep_status ep_compress_device(const void* dev_w, ep_dtype src, int64_t rows, int64_t cols, const ep_encode_opts* opts,
                             void* hip_stream, uint8_t** out_stream, size_t* out_len, double* actual_bpp) {
    return guarded([&]() -> ep_status {
        if (!out_stream || !out_len) return fail(EP_EINVAL, "null output pointer");
        if (rows < 0 || cols < 0) return fail(EP_EINVAL, "negative shape");
        if (rows * cols > 0 && !dev_w) return fail(EP_EINVAL, "null input");
        if (rows > 0xFFFFFFFFll || cols >= (1ll << 28)) return fail(EP_ERANGE, "shape too large (cols must be < 2^28)");
        ep_encode_opts o = opts ? *opts : ep_encode_opts{EP_MODE_LOSSY_E8, 4.0, 12, 16, 0, 0};
        if (o.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the device encoder codes the lossy mode");
        if (o.layout < 0 || o.layout > 1) return fail(EP_EINVAL, "layout must be 0 or 1");
        if (o.prob_bits < 10 || o.prob_bits > 12) return fail(EP_EINVAL, "prob_bits must be 10..12");
        if (o.tile_rows != 16 && o.tile_rows != 32) return fail(EP_EINVAL, "tile_rows must be 16 or 32");
        if (src != EP_F32 && src != EP_BF16 && src != EP_F16)
            return fail(EP_EUNSUPPORTED, "lossy mode takes F32, BF16 or F16 input");
        if (!(o.target_bpp > 0.0 && o.target_bpp <= 32.0)) return fail(EP_EINVAL, "target_bpp must be in (0, 32]");
        ep::Bytes buf;
        std::string why;
        ep_status st;
        try {
            st = ep::encode_lossy_device(dev_w, src, rows, cols, o, static_cast<hipStream_t>(hip_stream), &buf, &why);
        } catch (const std::bad_alloc&) {
            return fail(EP_ENOMEM, "host allocation failed while encoding");
        }
        if (st != EP_OK) return fail(st, why);
        const size_t len = buf.size();
        *out_stream = buf.release();
        *out_len = len;
        if (actual_bpp) *actual_bpp = rows * cols > 0 ? 8.0 * (double)len / ((double)rows * (double)cols) : 0.0;
        return EP_OK;
    });
}

ep_status ep_quantize_rows_fp8(const void* dev_x, int64_t M, int64_t K, uint8_t* dev_q, float* dev_scale,
                               void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (M < 0 || K < 0) return fail(EP_EINVAL, "negative size");
        if (M == 0) return EP_OK;
        if (!dev_x || !dev_q || !dev_scale) return fail(EP_EINVAL, "null pointer");
        if (M > INT32_MAX || K > INT32_MAX) return fail(EP_ERANGE, "M and K must be below 2^31");
        if (K % 16) return fail(EP_EINVAL, "K must be a multiple of 16");
        if ((reinterpret_cast<uintptr_t>(dev_x) | reinterpret_cast<uintptr_t>(dev_q)) & 15)
            return fail(EP_EINVAL, "X and Q must be 16-byte aligned");
        hipError_t e = ep::launch_quantize_rows_f8(static_cast<const uint16_t*>(dev_x), (int)M, (int)K, (int)K, dev_q,
                                                   (int)K, dev_scale, static_cast<hipStream_t>(hip_stream));
        return e == hipSuccess ? EP_OK : hip_fail(e, "quantize launch");
    });
}

ep_status ep_gemm_fp8(const uint8_t* dev_xq, const float* dev_xs, const uint8_t* dev_wq, const float* dev_ws,
                      int64_t M, int64_t N, int64_t K, const void* dev_bias, void* dev_y, void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (M < 0 || N < 0 || K < 0) return fail(EP_EINVAL, "negative size");
        if (M == 0 || N == 0) return EP_OK;
        if (!dev_xq || !dev_xs || !dev_wq || !dev_ws || !dev_y) return fail(EP_EINVAL, "null pointer");
        if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(EP_ERANGE, "M, N and K must be below 2^31");
        if (K % 16) return fail(EP_EINVAL, "K must be a multiple of 16");
        if ((reinterpret_cast<uintptr_t>(dev_xq) | reinterpret_cast<uintptr_t>(dev_wq)) & 15)
            return fail(EP_EINVAL, "X and W codes must be 16-byte aligned");
        ep::GemmF8Args g{dev_xq, dev_xs, dev_wq, dev_ws, static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y),
                         (int)M, (int)N, (int)K, (int)K, (int)K, (int)N};
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        // hipBLASLt where use_gemm_library says so, as for the FP8 forward's slices (its workspace
        // from the pool)
        hipError_t e = hipErrorNotSupported;
        WsLease ws;
        if (use_gemm_library(M, N, K)) {
            int dev = 0;
            e = hipGetDevice(&dev);
            if (e == hipSuccess) e = ws_acquire(dev, s, kLtWorkspace, &ws);
            if (e != hipSuccess) return hip_fail(e, "hipMalloc for the GEMM workspace");
            e = ep::lt_gemm_f8(g, ws.ptr, kLtWorkspace, s);
        }
        if (e == hipErrorNotSupported) e = ep::launch_gemm_f8(g, s);
        if (e == hipSuccess) e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "fp8 gemm launch");
    });
}

ep_status ep_linear_forward_fp8(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias, void* dev_y,
                                void* hip_stream) {
    return guarded([&]() -> ep_status {
        if (!w) return fail(EP_EINVAL, "null handle");
        if (ep_status st = on_its_device(w); st != EP_OK) return st;
        if (w->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
        const int64_t N = w->view.rows, K = w->view.cols;
        if (M < 0) return fail(EP_EINVAL, "negative M");
        if (M == 0 || N == 0) return EP_OK;
        if (!dev_y || (K > 0 && !dev_x)) return fail(EP_EINVAL, "null pointer");
        if (M > INT32_MAX || N > INT32_MAX) return fail(EP_ERANGE, "M and out_features must be below 2^31");
        if (K % 16) return fail(EP_EINVAL, "in_features must be a multiple of 16 for the FP8 forward");
        if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        int dev = 0;
        hipError_t we = hipGetDevice(&dev);
        if (we != hipSuccess) return hip_fail(we, "hipGetDevice");
        if (K == 0) {
            // in_features 0: an empty sum, Y = bias (or zeros)
            const hipError_t e = ep::launch_gemv_finish(nullptr, 0, static_cast<const uint16_t*>(dev_bias),
                                                        static_cast<uint16_t*>(dev_y), M, N, s);
            return e == hipSuccess ? EP_OK : hip_fail(e, "empty product launch");
        }
        if (const ep::MatDesc d = desc_for(w, ep::CT_F8E4M3, nullptr, nullptr); ep::fused_fits(d, M)) {
            // up to 16 activation rows (64 in the row layout): the activations quantized per row,
            // then every tile pair decoded straight into E4M3 codes as the B operand of the FP8
            // MFMA (through LDS in layout 0, from the decoder's registers in the row layout)
            // workspace: X codes [M][K] | X scales [M] | fp32 partial sums
            const size_t o_xs = up((size_t)M * (size_t)K, 256), o_pt = up(o_xs + 4 * (size_t)M, 256);
            const size_t need = o_pt + ep::fused_partial_bytes(d, M);
            WsLease ws;
            if ((we = ws_acquire(dev, s, need, &ws)) != hipSuccess)
                return hip_fail(we, "hipMalloc for the linear forward workspace");
            uint8_t* ws8 = static_cast<uint8_t*>(ws.ptr);
            float* xs = reinterpret_cast<float*>(ws8 + o_xs);
            hipError_t e = ep::launch_quantize_rows_f8(static_cast<const uint16_t*>(dev_x), (int)M, (int)K, (int)K, ws8,
                                                       (int)K, xs, s);
            if (e == hipSuccess)
                e = ep::launch_fused_f8(d, ws8, xs, M, reinterpret_cast<float*>(ws8 + o_pt),
                                        static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y), s);
            if (e == hipSuccess) e = ws.queued();
            return e == hipSuccess ? EP_OK : hip_fail(e, "fused FP8 decode + MFMA launch");
        }
        const int tr = w->view.tile_rows;
        int64_t slice = (int64_t)(kSliceBytes / (size_t)K) / tr * tr;
        if (slice < tr) slice = tr;
        if (slice > N) slice = (N + tr - 1) / tr * tr;
        // slices multiplied by hipBLASLt where use_gemm_library says so (as in the BF16 forward)
        const bool lt = use_gemm_library(M, N, K);
        // workspace: X codes [M][K] | X scales [M] | weight codes [slice][K] | weight scales [slice]
        // | hipBLASLt workspace
        const size_t o_xs = up((size_t)M * (size_t)K, 256), o_wq = up(o_xs + 4 * (size_t)M, 256);
        const size_t o_ws = up(o_wq + (size_t)slice * (size_t)K, 256), o_lt = up(o_ws + 4 * (size_t)slice, 256);
        const size_t need = o_lt + (lt ? kLtWorkspace : 0);
        WsLease ws;
        we = ws_acquire(dev, s, need, &ws);
        if (we != hipSuccess) return hip_fail(we, "hipMalloc for the linear forward workspace");
        uint8_t* ws8 = static_cast<uint8_t*>(ws.ptr);
        uint8_t* xq = ws8;
        float* xs = reinterpret_cast<float*>(ws8 + o_xs);
        uint8_t* wq = ws8 + o_wq;
        float* wsc = reinterpret_cast<float*>(ws8 + o_ws);
        hipError_t e = ep::launch_quantize_rows_f8(static_cast<const uint16_t*>(dev_x), (int)M, (int)K, (int)K, xq, (int)K,
                                                   xs, s);
        if (e != hipSuccess) return hip_fail(e, "quantize launch");
        const ep::MatDesc full = desc_for(w, ep::CT_F8E4M3, wq, wsc);
        for (int64_t r0 = 0; r0 < N; r0 += slice) {
            const int64_t rows = std::min<int64_t>(slice, N - r0);
            ep::MatDesc d = full;                  // rows r0 .. r0 + rows of the weight
            d.index += (size_t)(r0 / tr) * w->view.tiles_c;
            d.row_scale += r0;
            d.row_qmax += r0;
            d.rows = (uint32_t)rows;
            e = ep::launch_group(&d, 1, s);
            if (e != hipSuccess) return hip_fail(e, "slice decode launch");
            ep::GemmF8Args g{xq, xs, wq, wsc, dev_bias ? static_cast<const uint16_t*>(dev_bias) + r0 : nullptr,
                             static_cast<uint16_t*>(dev_y) + r0, (int)M, (int)rows, (int)K, (int)K, (int)K, (int)N};
            e = lt ? ep::lt_gemm_f8(g, ws8 + o_lt, kLtWorkspace, s) : hipErrorNotSupported;
            if (e == hipErrorNotSupported) e = ep::launch_gemm_f8(g, s);
            if (e != hipSuccess) return hip_fail(e, "slice fp8 gemm launch");
        }
        e = ws.queued();
        return e == hipSuccess ? EP_OK : hip_fail(e, "recording the workspace event");
    });
}

}  // extern "C"
