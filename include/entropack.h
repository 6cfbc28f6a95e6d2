/*
 * entropack.h — C ABI of the MI355X (gfx950) tile-rANS weight codec.
 *
 * What the library computes. Weights are compressed by row normalization, nearest-point
 * quantization on the E8 lattice, a probability model of the lattice coordinates, a sampled
 * estimate that picks the quantization step for a target bitrate, and entropy coding in tiles
 * that decode independently; on the GPU the symbols are decoded and the weights reconstructed
 * into BF16, FP16, FP8 or INT8 containers in one fused pass ("EntroPack: Fast and Accurate
 * Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract). The calls follow the
 * pages' statement of the interface: compress(tensor, target) returning a stream and its actual
 * bitrate, which includes metadata ("EntroPack PyTorch Guide: Lossless Weights, Bitrates and
 * Memory Checks", sections "Choose a compression contract" and "Start with a tensor round
 * trip"); decompress(stream) returning a tensor; a compressed linear layer whose forward pass
 * consumes the compressed weight (same guide, "Replace one linear layer before a whole model").
 *
 * Conventions for every call:
 *   - Status: every call returns ep_status (0 = EP_OK, negative = error). No C++ exception
 *     crosses the ABI. After an error, ep_last_error() returns a message for the calling thread.
 *   - Matrices are row-major [rows][cols]; for a linear layer rows = out_features.
 *   - "host" pointers are CPU memory; "dev" pointers are device memory of the current HIP
 *     device; hip_stream is a hipStream_t (NULL = the default stream). Device work is queued
 *     on hip_stream and returns without synchronizing unless stated otherwise.
 *   - Ownership: buffers returned by ep_compress belong to the caller and are freed with
 *     ep_free; ep_handle objects belong to the caller and are freed with ep_release; device
 *     outputs are always allocated by the caller.
 *   - Devices: a handle lives on the device that was current at ep_upload; calls that launch
 *     work for it return EP_EINVAL when another device is current.
 *   - Thread safety: distinct handles may be used from distinct threads; a handle is immutable
 *     after ep_upload except for its device error flag. The library's own shared state (per-device
 *     kernel attributes and CU counts, the linear forwards' workspaces) is guarded internally;
 *     each (device, stream) pair has its own workspace, so forwards on distinct streams may run
 *     concurrently, and forwards on one stream are ordered by that stream.
 */
#ifndef ENTROPACK_H
#define ENTROPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_EINVAL = -1,        /* bad argument (null pointer, bad size, bad option) */
    EP_ECORRUPT = -2,      /* stream fails validation, or a decode found it inconsistent */
    EP_EUNSUPPORTED = -3,  /* container / dtype / mode the stream cannot supply (no silent casts) */
    EP_ERANGE = -4,        /* value out of the representable range (non-finite input, too wide) */
    EP_EHIP = -5,          /* a HIP runtime call failed; the message names it */
    EP_ENOMEM = -6,        /* host or device allocation failed */
    EP_EDEVICE = -7        /* a kernel flagged a stream inconsistency (see ep_handle_check) */
} ep_status;

typedef enum { EP_F32 = 0, EP_BF16 = 1, EP_F16 = 2, EP_F8E4M3 = 3, EP_I8 = 4, EP_U8 = 5 } ep_dtype;

typedef enum {
    EP_MODE_LOSSY_E8 = 0,     /* target bitrate, E8 lattice coordinates */
    EP_MODE_LOSSLESS = 1,     /* bit-exact byte-plane coding of any supported dtype */
    EP_MODE_LOSSLESS_EXP = 2  /* bit-exact BF16: the 8-bit exponent coded by tile rANS, sign and
                                 mantissa stored as one uncoded byte per element (the guide's
                                 DFloat11 config for lossless BF16, section "Choose a compression
                                 contract", read after the published DFloat11 split) */
} ep_mode;

/* Encoder options. A NULL pointer means: lossy, target 4.0, prob_bits 12, tile_rows 16, all
 * host threads. */
typedef struct {
    ep_mode mode;
    double target_bpp;     /* lossy only: target payload bits per weight (0 < t <= 32) */
    int prob_bits;         /* probability precision n (10..12); frequencies sum to 2^n */
    int tile_rows;         /* 16 or 32 rows per tile; tiles are tile_rows x 256 */
    int n_threads;         /* host encoder threads, 0 = all hardware threads */
} ep_encode_opts;

/* Stream summary. actual_bpp = 8 * total_bytes / (rows * cols) (0 for an empty matrix).
 * payload_bytes counts the tile payload, plus the raw sign/mantissa plane of an exponent-coded
 * stream; meta_bytes = total_bytes - payload_bytes. */
typedef struct {
    int64_t rows, cols;
    int32_t mode, src_dtype, tile_rows, prob_bits;
    uint32_t n_tiles, n_escapes;
    float step, target_bpp;
    double actual_bpp;
    uint64_t total_bytes, payload_bytes, state_bytes, meta_bytes;
} ep_info;

typedef struct ep_handle ep_handle;   /* device-resident, validated stream */

/* Compress a host matrix.
 *   host_w: [rows][cols] elements of dtype src (lossy: EP_F32, EP_BF16, EP_F16; lossless: any;
 *           exponent-coded lossless: EP_BF16).
 *   *out_stream receives a library-allocated byte buffer (free with ep_free), *out_len its size,
 *   *actual_bpp (optional) the stored bits per weight including all metadata.
 * Errors: EP_EINVAL (null pointers, bad options), EP_EUNSUPPORTED (dtype not allowed for the
 * mode), EP_ERANGE (non-finite lossy input, cols >= 2^28), EP_ENOMEM. */
ep_status ep_compress(const void* host_w, ep_dtype src, int64_t rows, int64_t cols,
                      const ep_encode_opts* opts, uint8_t** out_stream, size_t* out_len,
                      double* actual_bpp);

/* Device encoder of the lossy mode: the same stream as ep_compress, byte for byte, computed on the
 * GPU from a weight already in device memory (row scales, the sampled rate search, the E8
 * quantization, the model and the tile rANS coding all run as kernels; the method's "fast
 * encoding", "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
 * Bitrates", Abstract). dev_w: [rows][cols] elements of src (EP_F32, EP_BF16, EP_F16) on the
 * current device; opts as for ep_compress (mode must be EP_MODE_LOSSY_E8; n_threads is unused).
 * The call synchronizes hip_stream. Device scratch (about 2.3 bytes per weight plus 18 KiB per
 * 16-row tile for the word stacks) is kept per device after the call, grown to the largest
 * matrix encoded, and reused; concurrent calls on one device take turns. *out_stream is
 * library-allocated (free with ep_free). Errors: as ep_compress, plus EP_EHIP / EP_ENOMEM for
 * device failures and EP_EUNSUPPORTED for a lossless mode. */
ep_status ep_compress_device(const void* dev_w, ep_dtype src, int64_t rows, int64_t cols,
                             const ep_encode_opts* opts, void* hip_stream, uint8_t** out_stream,
                             size_t* out_len, double* actual_bpp);

/* Free a buffer returned by ep_compress or ep_compress_device. NULL is allowed. */
void ep_free(void* p);

/* Validate a host stream (magic, format version 2, section bounds, every table summing to 2^n,
 * tile offsets, and three CRC-32s: the payload's, the raw plane's and the metadata's, which
 * covers every other byte, so any single-bit corruption is refused) and summarize it. Host only;
 * no device work. EP_ECORRUPT on any inconsistency. */
ep_status ep_stream_info(const uint8_t* host_stream, size_t len, ep_info* out);

/* Validate a host stream and copy it to the current device together with its decode tables.
 * Synchronizes hip_stream before returning (the host buffer may be freed afterwards).
 * *out receives the handle. Errors: EP_ECORRUPT, EP_ERANGE (a tile payload of 4 GiB or more,
 * beyond the decoder's 32-bit payload addressing: code such a matrix as several streams),
 * EP_ENOMEM, EP_EHIP. */
ep_status ep_upload(const uint8_t* host_stream, size_t len, void* hip_stream, ep_handle** out);

/* Summary of an uploaded stream (same fields as ep_stream_info). */
ep_status ep_handle_info(const ep_handle* h, ep_info* out);

/* Decode a whole matrix into a device container (the "decompress" call).
 *   dev_out: [rows][cols] elements of `container`, row-major, 16-byte aligned when cols % 8 == 0
 *            for the vector-store path (any alignment of the element size is accepted).
 *   dev_row_scale: [rows] fp32 dequantization scales, written for EP_F8E4M3 and EP_I8 (the
 *            weight is value * scale[row]); must be NULL for other containers.
 * Lossy streams accept EP_BF16, EP_F16, EP_F8E4M3, EP_I8; lossless streams accept only their
 * own dtype (EP_EUNSUPPORTED otherwise). Asynchronous on hip_stream. */
ep_status ep_decompress(const ep_handle* h, ep_dtype container, void* dev_out,
                        float* dev_row_scale, void* hip_stream);

/* Decode `count` matrices in one grouped launch. Arrays are host arrays of length count with
 * the same meaning as ep_decompress's arguments; NULL entries in dev_row_scales are allowed
 * where the container needs none. Asynchronous on hip_stream. */
ep_status ep_decompress_many(const ep_handle* const* hs, const ep_dtype* containers,
                             void* const* dev_outs, float* const* dev_row_scales, int count,
                             void* hip_stream);

/* Decode a lossy stream's lattice symbols: dev_q [rows][cols] int16 doubled coordinates
 * q = 2p of the E8 point p (the reconstructed weight is q * step / 2 * row_scale).
 * EP_EUNSUPPORTED for lossless streams. Asynchronous on hip_stream. */
ep_status ep_decode_symbols(const ep_handle* h, int16_t* dev_q, void* hip_stream);

/* Compressed linear layer forward: Y[M][N] = X[M][K] * W^T (+ bias), W = the decoded BF16
 * weight [N][K] of handle w, fp32 accumulation, BF16 output ("EntroPack PyTorch Guide", section
 * "Replace one linear layer before a whole model"). For M <= 4 the decode kernel itself forms the
 * products (the decoded fp32 weights, not rounded to BF16, are multiplied by the activations in
 * registers and summed into an fp32 accumulator in the workspace by atomic additions, whose order
 * varies, so two calls may differ in the last bits; the weight is never written). For larger M
 * the weight is decoded once per call, up to 128 MiB of BF16 rows at a time, into a
 * library-owned workspace that stays in the Infinity Cache, and each slice is multiplied by the
 * BF16 MFMA GEMM (deterministic); no decoded copy of W outlives the call. The workspace belongs
 * to the (device, hip_stream) pair: calls on one stream reuse it in order, calls on different
 * streams get different workspaces; it is allocated on first use
 * (hipMalloc, which may synchronize the device) and kept until the process ends.
 *   dev_x: [M][K] bf16, 16-byte aligned; dev_bias: [N] bf16 or NULL; dev_y: [M][N] bf16.
 * Requires a lossy stream and K % 8 == 0. Asynchronous on hip_stream. */
ep_status ep_linear_forward(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                            void* dev_y, void* hip_stream);

/* Plain BF16 GEMM, the one ep_linear_forward runs on each decoded slice, for overhead
 * comparisons: Y[M][N] = X[M][K] * W^T, X [M][K] bf16, W [N][K] bf16, Y [M][N] bf16, fp32
 * accumulation. Requires K % 8 == 0 and 16-byte aligned X and W. Asynchronous on hip_stream. */
ep_status ep_gemm_bf16(const void* dev_x, const void* dev_w, int64_t M, int64_t N, int64_t K,
                       void* dev_y, void* hip_stream);

/* FP8 variant of ep_linear_forward: Y[M][N] = s_x[m] s_w[n] sum_k x8[m][k] w8[n][k] (+ bias), BF16
 * output. The weight is decoded, slice by slice as in ep_linear_forward, into the FP8 E4M3
 * container with its per-row scale s_w (the FP8 container of "EntroPack: Fast and Accurate
 * Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract), the activations are
 * quantized per row as ep_quantize_rows_fp8 does, and both meet in the gfx950 FP8 MFMA with fp32
 * accumulation. Same workspace rules as ep_linear_forward. dev_x: [M][K] bf16, 16-byte aligned,
 * finite; dev_bias: [N] bf16 or NULL; dev_y: [M][N] bf16. Requires a lossy stream and
 * K % 16 == 0. Asynchronous on hip_stream. */
ep_status ep_linear_forward_fp8(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                                void* dev_y, void* hip_stream);

/* Per-row FP8 E4M3 quantization of BF16 rows, as the FP8 forward applies it to its activations:
 * amax = max |x| over the row (raised to 2^-100 when smaller, unless zero), scale = amax / 448,
 * code = E4M3(x * (448 / amax)) rounded to nearest even and saturated at +-448; a zero row gets
 * scale 0 and codes 0. dev_x: [M][K] bf16 (finite), dev_q: [M][K] codes, dev_scale: [M] fp32;
 * K % 16 == 0, dev_x and dev_q 16-byte aligned. Asynchronous on hip_stream. */
ep_status ep_quantize_rows_fp8(const void* dev_x, int64_t M, int64_t K, uint8_t* dev_q, float* dev_scale,
                               void* hip_stream);

/* Plain FP8 GEMM, the one ep_linear_forward_fp8 runs on each decoded slice, for overhead
 * comparisons: Y[m][n] = xs[m] ws[n] sum_k xq[m][k] wq[n][k] (+ bias[n]); xq [M][K] and wq [N][K]
 * E4M3 codes (16-byte aligned), xs [M] and ws [N] fp32, bias [N] bf16 or NULL, Y [M][N] bf16.
 * Requires K % 16 == 0. Asynchronous on hip_stream. */
ep_status ep_gemm_fp8(const uint8_t* dev_xq, const float* dev_xs, const uint8_t* dev_wq, const float* dev_ws,
                      int64_t M, int64_t N, int64_t K, const void* dev_bias, void* dev_y, void* hip_stream);

/* Synchronize hip_stream and read the handle's device error flag, which kernels set when a
 * tile's words run out or overrun, or a lane's final rANS state differs from its initial
 * value (or, as an internal consistency check, when a decode kernel finds its LDS tables
 * misplaced). EP_EDEVICE if set (the flag is then cleared), else EP_OK. */
ep_status ep_handle_check(ep_handle* h, void* hip_stream);

/* Free a handle and its device memory. NULL is allowed. The caller must ensure no queued
 * work still uses it. */
void ep_release(ep_handle* h);

/* Message for the last failed call on this thread ("" if none). */
const char* ep_last_error(void);

/* Library build string (version, target architecture). */
const char* ep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTROPACK_H */
