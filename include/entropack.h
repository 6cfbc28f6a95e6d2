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
 * host threads, layout 0. */
typedef struct {
    ep_mode mode;
    double target_bpp;     /* lossy only: target payload bits per weight (0 < t <= 32) */
    int prob_bits;         /* probability precision n (10..12); frequencies sum to 2^n */
    int tile_rows;         /* 16 or 32 rows per tile; tiles are tile_rows x 256 */
    int n_threads;         /* host encoder threads, 0 = all hardware threads */
    int layout;            /* lossy tile layout (reading R27; 0 in the lossless modes): which 8-column
                              block of a tile each of its 32 rANS states codes at block step s.
                              0: tile row s, block column l (lane l). 1: tile row l mod tile_rows,
                              block column (32 / tile_rows) s + l / tile_rows, so every block step
                              covers all tile rows; the compressed linear forward multiplies
                              layout-1 weights straight from the decoder's registers. Both layouts
                              decode to the same weights. */
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
    int32_t layout;        /* lossy tile layout (ep_encode_opts.layout) */
} ep_info;

typedef struct ep_handle ep_handle;   /* device-resident, validated stream */

/* Compress a host matrix.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", sections "Choose a compression
 * contract" (a lossless BF16 config, lossless tile ANS across dtypes, a lossy target bitrate) and
 * "Start with a tensor round trip" (the stored size, metadata included, is what counts); the lossy
 * steps follow "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates",
 * Abstract; readings R1-R16 fix what the pages leave open.
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
 * quantization, the model and the tile rANS coding all run as kernels).
 * Source: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract (fast
 * encoding); "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model" (conversion cost kept apart from inference).
 * dev_w: [rows][cols] elements of src (EP_F32, EP_BF16, EP_F16) on the current device; opts as for ep_compress (mode must be EP_MODE_LOSSY_E8; n_threads is unused).
 * The call synchronizes hip_stream. Device scratch (about 2.3 bytes per weight plus 18 KiB per
 * 16-row tile for the word stacks) is kept per device after the call, grown to the largest
 * matrix encoded, and reused; concurrent calls on one device take turns. *out_stream is
 * library-allocated (free with ep_free). Errors: as ep_compress, plus EP_EHIP / EP_ENOMEM for
 * device failures and EP_EUNSUPPORTED for a lossless mode. */
ep_status ep_compress_device(const void* dev_w, ep_dtype src, int64_t rows, int64_t cols,
                             const ep_encode_opts* opts, void* hip_stream, uint8_t** out_stream,
                             size_t* out_len, double* actual_bpp);

/* Free a buffer returned by ep_compress or ep_compress_device. NULL is allowed.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Start with a tensor round trip" (the stored representation ep_compress returns belongs to the
 * caller). */
void ep_free(void* p);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", sections
 * "Start with a tensor round trip" (record the actual stored size and its metadata) and "Diagnose
 * compression failures in the correct order" (the saved object must hold everything the decoder
 * needs); reading R22 (three CRC-32s).
 * Validate a host stream (magic, format version 2, section bounds, every table summing to 2^n,
 * tile offsets, and three CRC-32s: the payload's, the raw plane's and the metadata's, which
 * covers every other byte, so any single-bit corruption is refused) and summarize it. Host only;
 * no device work. EP_ECORRUPT on any inconsistency; EP_ERANGE for an intact stream of 2^28 or more
 * columns (wider than the encoders write and the decoders address). */
ep_status ep_stream_info(const uint8_t* host_stream, size_t len, ep_info* out);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", sections
 * "Diagnose compression failures in the correct order" (a stream is checked before the decoder
 * trusts it) and "Measure memory with clear boundaries" (loading is its own phase, apart from the
 * inference call); reading R22.
 * Validate a host stream and copy it to the current device together with its decode tables.
 * Synchronizes hip_stream before returning (the host buffer may be freed afterwards).
 * *out receives the handle. Errors: EP_ECORRUPT, EP_ERANGE (2^28 or more columns, or a tile
 * payload of 4 GiB or more, beyond the decoder's 32-bit payload addressing: code such a matrix as
 * several streams), EP_ENOMEM, EP_EHIP. */
ep_status ep_upload(const uint8_t* host_stream, size_t len, void* hip_stream, ep_handle** out);

/* Summary of an uploaded stream (same fields as ep_stream_info).
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Start with a tensor round trip" (record the stored size). */
ep_status ep_handle_info(const ep_handle* h, ep_info* out);

/* Decode a whole matrix into a device container (the "decompress" call).
 * Source: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract
 * (fused symbol decoding and weight reconstruction on the GPU into BF16, FP16, FP8 or INT8, the
 * bitrate independent of the container); "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Diagnose compression failures in the correct order" (no silent
 * cast of the restored tensor: a container the stream cannot supply is refused); readings R17-R20.
 *   dev_out: [rows][cols] elements of `container`, row-major, 16-byte aligned when cols % 8 == 0
 *            for the vector-store path (any alignment of the element size is accepted).
 *   dev_row_scale: [rows] fp32 dequantization scales, written for EP_F8E4M3 and EP_I8 (the
 *            weight is value * scale[row]); must be NULL for other containers.
 * Lossy streams accept EP_BF16, EP_F16, EP_F8E4M3, EP_I8; lossless streams accept only their
 * own dtype (EP_EUNSUPPORTED otherwise). Asynchronous on hip_stream. */
ep_status ep_decompress(const ep_handle* h, ep_dtype container, void* dev_out,
                        float* dev_row_scale, void* hip_stream);

/* Decode `count` matrices in one grouped launch.
 * Source: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract
 * (decode time grows with the weight count; diffusion denoising decodes every layer each step);
 * "EntroPack 開源：模型壓縮不必只選 4 位元，如何配合顯示記憶體預算？", section "官方時間要保留原工作範圍"
 * (the timing covers a whole denoise step). Arrays are host arrays of length count with
 * the same meaning as ep_decompress's arguments; NULL entries in dev_row_scales are allowed
 * where the container needs none. Asynchronous on hip_stream. */
ep_status ep_decompress_many(const ep_handle* const* hs, const ep_dtype* containers,
                             void* const* dev_outs, float* const* dev_row_scales, int count,
                             void* hip_stream);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Test saved artifacts and reloads before deployment" (the recovered quantized codes are what a
 * quantize-then-entropy-code package reproduces exactly); readings R4, R7, R10.
 * Decode a lossy stream's lattice symbols: dev_q [rows][cols] int16 doubled coordinates
 * q = 2p of the E8 point p (the reconstructed weight is q * step / 2 * row_scale).
 * EP_EUNSUPPORTED for lossless streams. Asynchronous on hip_stream. */
ep_status ep_decode_symbols(const ep_handle* h, int16_t* dev_q, void* hip_stream);

/* Compressed linear layer forward: Y[M][N] = X[M][K] * W^T (+ bias), W = the decoded BF16
 * weight [N][K] of handle w, fp32 accumulation, BF16 output.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model" (CompressedLinear); "EntroPack: Fast and Accurate
 * Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract (decoding fused into the GPU
 * computation that uses the weight). Paths:
 *   - fused decode + MFMA, for M <= 64 on row-layout streams (ep_encode_opts.layout = 1) and for
 *     5 <= M <= 16 on layout-0 streams: each tile pair is decoded once into the B operand of the
 *     BF16 MFMA (row layout: straight from the decoder's registers; layout 0: transposed through
 *     LDS), the weight never written; fp32 partial sums per tile pair in the workspace, summed in
 *     column order (deterministic);
 *   - M <= 4 on layout-0 streams: the decode kernel forms the products (the decoded weights
 *     rounded to BF16 as the decode stores them, times the activations in registers), one fp32
 *     partial sum per row and tile pair column in the workspace, added in column order
 *     (deterministic);
 *   - otherwise the weight is decoded once per call, up to 128 MiB of BF16 rows at a time, into
 *     the workspace, which stays in the Infinity Cache, and each slice is multiplied by the BF16
 *     MFMA GEMM: hipBLASLt's from 512 rows, above 64 when K <= 4096, from 256 when N <= 4096 (faster
 *     there; its handle is created on the device's first such call), else the library's own; both
 *     deterministic (tested); no decoded copy of W outlives the call.
 * The fused and slice paths multiply the same BF16-rounded weights. The workspace belongs
 * to the (device, hip_stream) pair: calls on one stream reuse it in order, calls on different
 * streams get different workspaces; it is allocated on first use
 * (hipMalloc, which may synchronize the device) and kept until the process ends.
 *   dev_x: [M][K] bf16, 16-byte aligned (may be NULL when K == 0); dev_bias: [N] bf16 or NULL;
 * dev_y: [M][N] bf16. K == 0 gives Y = bias (or zeros). Requires a lossy stream and K % 8 == 0
 * (EP_EINVAL); M and N below 2^31 (EP_ERANGE). Asynchronous on hip_stream. */
ep_status ep_linear_forward(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                            void* dev_y, void* hip_stream);

/* Several compressed linear layers that take the same input: Y_i = X * W_i^T (+ bias_i) for
 * i < count, each Y_i the same bits as ep_linear_forward(w[i], dev_x, M, dev_bias[i], dev_y[i]).
 * When every layer is a row-layout stream (ep_encode_opts.layout = 1) with the same prob_bits and
 * 1 <= M <= 64 (the fused path of ep_linear_forward), one kernel decodes all of their tile pairs
 * into the BF16 MFMA, cost-balanced across the layers, so that a layer whose last round of tile
 * pairs would leave most wave slots idle (e.g. the gate and up projections of a gated FFN, 4800
 * pairs each at 10240 x 3840 for 4096 slots) shares its rounds with the others. Above 64 rows, when
 * every layer's own forward would decode it as one slice (N_i K <= 64 Mi) multiplied by hipBLASLt
 * and the group's slices total at most 192 MiB, one grouped launch decodes all the slices and each
 * is then multiplied as its own forward would. Otherwise the layers run one ep_linear_forward
 * each, in order.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model" (compressed layers inside a model's forward);
 * "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract
 * (decoding fused with the computation that uses the weights). Grouping layers that share an
 * input is this library's scheduling, not a step of the method.
 *   w: count handles, all with the same in_features K; dev_x: [M][K] bf16, 16-byte aligned (may be
 * NULL when K == 0); dev_bias: NULL or count pointers (each [N_i] bf16 or NULL); dev_y: count
 * pointers to [M][N_i] bf16. count in 0 ... 32 (EP_ERANGE otherwise); different in_features or a
 * null handle or output give EP_EINVAL before anything is queued; a lossless stream
 * EP_EUNSUPPORTED. The workspace is the (device, hip_stream) pair's, as for ep_linear_forward.
 * Asynchronous on hip_stream. */
ep_status ep_linear_forward_many(const ep_handle* const* w, int count, const void* dev_x, int64_t M,
                                 const void* const* dev_bias, void* const* dev_y, void* hip_stream);

/* ep_linear_forward_many in FP8: Y_i the same bits as ep_linear_forward_fp8(w[i], dev_x, M,
 * dev_bias[i], dev_y[i]) for every layer. When the layers are row-layout streams with one
 * prob_bits, 1 <= M <= 64 and K % 16 == 0, the activations are quantized once per row to E4M3 for
 * the group and one kernel decodes every layer's tile pairs into E4M3 codes for the FP8 MFMA, each
 * layer finished with its own row scales; otherwise one ep_linear_forward_fp8 per layer, in order.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model"; "EntroPack: Fast and Accurate Entropy-Coded
 * Weight Compression at Arbitrary Bitrates", Abstract (FP8 among the containers the decode fills).
 * Grouping layers that share an input is this library's scheduling, not a step of the method.
 * Arguments, checks and errors as ep_linear_forward_many, plus K % 16 == 0 (EP_EINVAL, from the
 * per-layer forwards). */
ep_status ep_linear_forward_fp8_many(const ep_handle* const* w, int count, const void* dev_x, int64_t M,
                                     const void* const* dev_bias, void* const* dev_y, void* hip_stream);

/* For callers that cannot allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc): ep_linear_forward with its scratch in a static device array
 * of 64 MiB per device instead of the library's workspace pool. It calls no hipMalloc, hipFree or
 * allocating library routine; the array lives from library load until the process ends. Same
 * arguments, results and paths as ep_linear_forward (the same kernels: the fused kernels' partial
 * sums, those of M <= 4 on layout-0 streams, otherwise BF16 weight slices of at
 * most 64 MiB, i.e. 64 MiB / (2 K) rows, always multiplied by the library's own GEMM kernel, so
 * results where ep_linear_forward uses hipBLASLt may differ from it in the fp32 summation
 * order). EP_ERANGE when a call needs more than the array holds
 * (M <= 4 on layout-0 streams with 4 M N ceil(K / 512) > 64 MiB, the fused partials of very wide
 * layers, or K > 2^21 for the slices).
 * Every call on a device shares that device's array: calls that overlap in time on one device
 * (other streams, other threads) race and must be serialized by the caller.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Measure
 * memory with clear boundaries" (temporary buffers of a call are part of its memory). */
ep_status ep_linear_forward_noalloc(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                                    void* dev_y, void* hip_stream);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model" (evaluate the original layer beside the
 * compressed copy on the same input): the uncompressed baseline of the compressed forward.
 * Plain BF16 GEMM, the one ep_linear_forward runs on each decoded slice, for overhead
 * comparisons: Y[M][N] = X[M][K] * W^T, X [M][K] bf16, W [N][K] bf16, Y [M][N] bf16, fp32
 * accumulation. Requires K % 8 == 0 and 16-byte aligned X and W (EP_EINVAL); M, N and K below
 * 2^31 (EP_ERANGE). Asynchronous on hip_stream. */
ep_status ep_gemm_bf16(const void* dev_x, const void* dev_w, int64_t M, int64_t N, int64_t K,
                       void* dev_y, void* hip_stream);

/* Source: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates",
 * Abstract (the FP8 container); "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory
 * Checks", section "Replace one linear layer before a whole model".
 * FP8 variant of ep_linear_forward: Y[M][N] = s_x[m] s_w[n] sum_k x8[m][k] w8[n][k] (+ bias), BF16
 * output. The weight is decoded into the FP8 E4M3 container with its per-row scale s_w (the FP8
 * container of "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
 * Bitrates", Abstract), the activations are quantized per row as ep_quantize_rows_fp8 does, and
 * both meet in the gfx950 FP8 MFMA with fp32 accumulation. For M <= 64 on row-layout streams and
 * M <= 16 on layout-0 streams the codes go straight into the MFMA's B operand (fused, as in
 * ep_linear_forward); otherwise the weight is decoded slice by slice into the workspace and
 * multiplied by the FP8 GEMM. Same workspace rules as ep_linear_forward. dev_x: [M][K] bf16, 16-byte aligned,
 * finite (may be NULL when K == 0); dev_bias: [N] bf16 or NULL; dev_y: [M][N] bf16. K == 0 gives
 * Y = bias (or zeros). Requires a lossy stream and K % 16 == 0 (EP_EINVAL); M and N below 2^31
 * (EP_ERANGE). Asynchronous on hip_stream. */
ep_status ep_linear_forward_fp8(const ep_handle* w, const void* dev_x, int64_t M, const void* dev_bias,
                                void* dev_y, void* hip_stream);

/* Source: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates", Abstract (FP8
 * container); the activation scale rule is a reading (amax / 448 per row, like the weight rows).
 * Per-row FP8 E4M3 quantization of BF16 rows, as the FP8 forward applies it to its activations:
 * amax = max |x| over the row (raised to 2^-100 when smaller, unless zero), scale = amax / 448,
 * code = E4M3(x * (448 / amax)) rounded to nearest even and saturated at +-448; a zero row gets
 * scale 0 and codes 0. dev_x: [M][K] bf16 (finite), dev_q: [M][K] codes, dev_scale: [M] fp32;
 * K % 16 == 0, dev_x and dev_q 16-byte aligned (EP_EINVAL); M and K below 2^31 (EP_ERANGE).
 * Asynchronous on hip_stream. */
ep_status ep_quantize_rows_fp8(const void* dev_x, int64_t M, int64_t K, uint8_t* dev_q, float* dev_scale,
                               void* hip_stream);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section
 * "Replace one linear layer before a whole model" (the uncompressed baseline, here of the FP8
 * forward).
 * Plain FP8 GEMM, the one ep_linear_forward_fp8 runs on each decoded slice, for overhead
 * comparisons: Y[m][n] = xs[m] ws[n] sum_k xq[m][k] wq[n][k] (+ bias[n]); xq [M][K] and wq [N][K]
 * E4M3 codes (16-byte aligned), xs [M] and ws [N] fp32, bias [N] bf16 or NULL, Y [M][N] bf16.
 * hipBLASLt's from 512 rows, above 64 when K <= 4096, from 256 when N <= 4096 (the row scales as its
 * outer-vector scales; 32 MiB of workspace from the (device, hip_stream) pool, see
 * ep_linear_forward), else, or when it offers no algorithm, the library's own kernel; both
 * deterministic. Requires K % 16 == 0 (EP_EINVAL); M, N and K below 2^31 (EP_ERANGE).
 * Asynchronous on hip_stream. */
ep_status ep_gemm_fp8(const uint8_t* dev_xq, const float* dev_xs, const uint8_t* dev_wq, const float* dev_ws,
                      int64_t M, int64_t N, int64_t K, const void* dev_bias, void* dev_y, void* hip_stream);

/* Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Test
 * saved artifacts and reloads before deployment" (a failed step must stop with a clear error);
 * reading R12 (every lane ends at its initial state: a free integrity check).
 * Synchronize hip_stream and read the handle's device error flag, which kernels set when a
 * tile's words run out or overrun, or a lane's final rANS state differs from its initial
 * value (or, as an internal consistency check, when a decode kernel finds its LDS tables
 * misplaced). EP_EDEVICE if set (the flag is then cleared), else EP_OK. */
ep_status ep_handle_check(ep_handle* h, void* hip_stream);

/* Free a handle and its device memory. NULL is allowed. The caller must ensure no queued
 * work still uses it.
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Measure
 * memory with clear boundaries" (the resident compressed weight is one device allocation). */
void ep_release(ep_handle* h);

/* Message for the last failed call on this thread ("" if none).
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Test
 * saved artifacts and reloads before deployment" (stop with a clear error). */
const char* ep_last_error(void);

/* Library build string (version, target architecture).
 * Source: "EntroPack PyTorch Guide: Lossless Weights, Bitrates and Memory Checks", section "Check
 * the installation and hardware combination" (record the library revision and the GPU). */
const char* ep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTROPACK_H */
