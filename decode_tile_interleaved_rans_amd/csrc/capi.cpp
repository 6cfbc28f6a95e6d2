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
#include "gemm.h"
#include "kernels.h"

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

// Library-owned device workspaces, one per (device, stream), grown on demand and kept until the
// process ends (work queued on the stream may still use a workspace after a call returns).
hipError_t workspace(int device, hipStream_t stream, size_t need, uint16_t** out) {
    struct Entry {
        int device;
        hipStream_t stream;
        uint16_t* ptr;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Entry> pool;
    std::lock_guard<std::mutex> lock(mu);
    for (Entry& e : pool) {
        if (e.device != device || e.stream != stream) continue;
        if (e.bytes < need) {
            // earlier calls on this stream may still read the old buffer: wait for them
            hipError_t r = hipStreamSynchronize(stream);
            if (r == hipSuccess) r = hipFree(e.ptr);
            if (r != hipSuccess) return r;
            e.ptr = nullptr;
            e.bytes = 0;
            r = hipMalloc(reinterpret_cast<void**>(&e.ptr), need);
            if (r != hipSuccess) return r;
            e.bytes = need;
        }
        *out = e.ptr;
        return hipSuccess;
    }
    Entry e{device, stream, nullptr, need};
    hipError_t r = hipMalloc(reinterpret_cast<void**>(&e.ptr), need);
    if (r != hipSuccess) return r;
    pool.push_back(e);
    *out = e.ptr;
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
        ep_encode_opts o = opts ? *opts : ep_encode_opts{EP_MODE_LOSSY_E8, 4.0, 12, 16, 0};
        if (o.prob_bits < 10 || o.prob_bits > 12) return fail(EP_EINVAL, "prob_bits must be 10..12");
        if (o.tile_rows != 16 && o.tile_rows != 32) return fail(EP_EINVAL, "tile_rows must be 16 or 32");
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
        if (K % 8 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(EP_EINVAL, "K must be a multiple of 8");
        if ((reinterpret_cast<uintptr_t>(dev_x) | reinterpret_cast<uintptr_t>(dev_w)) & 15)
            return fail(EP_EINVAL, "X and W must be 16-byte aligned");
        ep::GemmArgs g{static_cast<const uint16_t*>(dev_x), static_cast<const uint16_t*>(dev_w), nullptr,
                       static_cast<uint16_t*>(dev_y), (int)M, (int)N, (int)K, (int)K, (int)K, (int)N};
        hipError_t e = ep::launch_gemm(g, static_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return hip_fail(e, "gemm launch");
        return EP_OK;
    });
}

// Compressed linear forward. The weight is decoded once per call, one slice of output rows at a
// time, into the (device, stream) workspace of at most kSliceBytes, and each slice's GEMM writes
// its columns of Y. A slice is large enough to keep every CU's decode block busy and, with the
// activations, small enough to stay in the 256 MB Infinity Cache between the decode that writes
// it and the GEMM that reads it (128 MiB measured best against 64 and 256 for M = 256 ... 4096).
ep_status ep_linear_forward(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias, void* dev_y,
                            void* hip_stream) {
    return guarded([&]() -> ep_status {
        constexpr size_t kSliceBytes = 128u << 20;
        if (!w) return fail(EP_EINVAL, "null handle");
        if (ep_status st = on_its_device(w); st != EP_OK) return st;
        if (w->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
        const int64_t N = w->view.rows, K = w->view.cols;
        if (M < 0) return fail(EP_EINVAL, "negative M");
        if (M == 0 || N == 0) return EP_OK;
        if (!dev_x || !dev_y) return fail(EP_EINVAL, "null pointer");
        if (K % 8 || M > INT32_MAX) return fail(EP_EINVAL, "in_features must be a multiple of 8");
        if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        if (M <= 4) {
            // a few activation rows: decoding fused with the matrix-vector products, the weight never
            // written out; fp32 accumulation in the workspace, then rounding (+ bias) to BF16
            uint16_t* acc = nullptr;
            int dev = 0;
            hipError_t we = hipGetDevice(&dev);
            if (we == hipSuccess) we = workspace(dev, s, sizeof(float) * (size_t)M * (size_t)N, &acc);
            if (we != hipSuccess) return hip_fail(we, "hipMalloc for the linear forward workspace");
            float* yacc = reinterpret_cast<float*>(acc);
            ep::MatDesc d = desc_for(w, M == 1 ? ep::CT_GEMV1 : M == 2 ? ep::CT_GEMV2 : ep::CT_GEMV4, yacc, nullptr);
            d.gemv_x = static_cast<const uint16_t*>(dev_x);
            d.gemv_m = (uint8_t)M;
            hipError_t e = ep::launch_gemv_zero(yacc, M * N, s);
            if (e == hipSuccess) e = ep::launch_gemv(d, s);
            if (e == hipSuccess)
                e = ep::launch_gemv_finish(yacc, static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y), M, N, s);
            return e == hipSuccess ? EP_OK : hip_fail(e, "fused matrix-vector launch");
        }
        const int tr = w->view.tile_rows;
        int64_t slice = (int64_t)(kSliceBytes / (2 * (size_t)K)) / tr * tr;
        if (slice < tr) slice = tr;
        if (slice > N) slice = (N + tr - 1) / tr * tr;
        const size_t need = (size_t)slice * (size_t)K * 2;
        uint16_t* scratch = nullptr;
        int dev = 0;
        hipError_t we = hipGetDevice(&dev);
        if (we == hipSuccess) we = workspace(dev, s, need, &scratch);
        if (we != hipSuccess) return hip_fail(we, "hipMalloc for the linear forward workspace");
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
            e = ep::launch_gemm(g, s);
            if (e != hipSuccess) return hip_fail(e, "slice gemm launch");
        }
        return EP_OK;
    });
}

ep_status ep_compress_device(const void* dev_w, ep_dtype src, int64_t rows, int64_t cols, const ep_encode_opts* opts,
                             void* hip_stream, uint8_t** out_stream, size_t* out_len, double* actual_bpp) {
    return guarded([&]() -> ep_status {
        if (!out_stream || !out_len) return fail(EP_EINVAL, "null output pointer");
        if (rows < 0 || cols < 0) return fail(EP_EINVAL, "negative shape");
        if (rows * cols > 0 && !dev_w) return fail(EP_EINVAL, "null input");
        if (rows > 0xFFFFFFFFll || cols >= (1ll << 28)) return fail(EP_ERANGE, "shape too large (cols must be < 2^28)");
        ep_encode_opts o = opts ? *opts : ep_encode_opts{EP_MODE_LOSSY_E8, 4.0, 12, 16, 0};
        if (o.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the device encoder codes the lossy mode");
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
        if (K % 16 || M > INT32_MAX || K > INT32_MAX) return fail(EP_EINVAL, "K must be a multiple of 16");
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
        if (K % 16 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(EP_EINVAL, "K must be a multiple of 16");
        if ((reinterpret_cast<uintptr_t>(dev_xq) | reinterpret_cast<uintptr_t>(dev_wq)) & 15)
            return fail(EP_EINVAL, "X and W codes must be 16-byte aligned");
        ep::GemmF8Args g{dev_xq, dev_xs, dev_wq, dev_ws, static_cast<const uint16_t*>(dev_bias), static_cast<uint16_t*>(dev_y),
                         (int)M, (int)N, (int)K, (int)K, (int)K, (int)N};
        hipError_t e = ep::launch_gemm_f8(g, static_cast<hipStream_t>(hip_stream));
        return e == hipSuccess ? EP_OK : hip_fail(e, "fp8 gemm launch");
    });
}

ep_status ep_linear_forward_fp8(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias, void* dev_y,
                                void* hip_stream) {
    return guarded([&]() -> ep_status {
        constexpr size_t kSliceBytes = 128u << 20;
        if (!w) return fail(EP_EINVAL, "null handle");
        if (ep_status st = on_its_device(w); st != EP_OK) return st;
        if (w->view.mode != EP_MODE_LOSSY_E8) return fail(EP_EUNSUPPORTED, "the linear forward takes a lossy stream");
        const int64_t N = w->view.rows, K = w->view.cols;
        if (M < 0) return fail(EP_EINVAL, "negative M");
        if (M == 0 || N == 0) return EP_OK;
        if (!dev_x || !dev_y) return fail(EP_EINVAL, "null pointer");
        if (K % 16 || M > INT32_MAX) return fail(EP_EINVAL, "in_features must be a multiple of 16 for the FP8 forward");
        if (reinterpret_cast<uintptr_t>(dev_x) & 15) return fail(EP_EINVAL, "X must be 16-byte aligned");
        const int tr = w->view.tile_rows;
        int64_t slice = (int64_t)(kSliceBytes / (size_t)K) / tr * tr;
        if (slice < tr) slice = tr;
        if (slice > N) slice = (N + tr - 1) / tr * tr;
        // workspace: X codes [M][K] | X scales [M] | weight codes [slice][K] | weight scales [slice]
        const size_t o_xs = up((size_t)M * (size_t)K, 256), o_wq = up(o_xs + 4 * (size_t)M, 256);
        const size_t o_ws = up(o_wq + (size_t)slice * (size_t)K, 256), need = o_ws + 4 * (size_t)slice;
        hipStream_t s = static_cast<hipStream_t>(hip_stream);
        uint16_t* base = nullptr;
        int dev = 0;
        hipError_t we = hipGetDevice(&dev);
        if (we == hipSuccess) we = workspace(dev, s, need, &base);
        if (we != hipSuccess) return hip_fail(we, "hipMalloc for the linear forward workspace");
        uint8_t* ws8 = reinterpret_cast<uint8_t*>(base);
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
            e = ep::launch_gemm_f8(g, s);
            if (e != hipSuccess) return hip_fail(e, "slice fp8 gemm launch");
        }
        return EP_OK;
    });
}

}  // extern "C"
