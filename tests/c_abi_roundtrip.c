/* The C ABI used from plain C (no Python, no PyTorch): compress on the host, upload, decode on
 * the GPU, read back. Built by __graft_entry__.build() with gcc against include/entropack.h and
 * the HIP runtime; run by tests/test_gpu_c_abi.py.
 *
 *   c_abi_roundtrip <dir>
 *
 * 1. A seeded 300 x 700 fp32 matrix (xorshift64* uniforms through a sum of four, roughly
 *    Gaussian, scale 0.02) is coded lossless and decoded on the GPU back to fp32: the program
 *    itself checks the bits.
 * 2. The same matrix is coded lossy at 4.0 bpp and decoded to BF16 on the GPU; the stream and
 *    the decoded bits are written to <dir>/lossy.epk and <dir>/lossy_bf16.bin for the test to
 *    compare with the oracle.
 * Exit status 0 on success; a message on stderr otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "entropack.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform01(void) {      /* xorshift64* (Vigna), top 53 bits */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static int fail_ep(const char* what, ep_status st) {
    fprintf(stderr, "%s: status %d: %s\n", what, (int)st, ep_last_error());
    return 1;
}

static int fail_hip(const char* what, hipError_t e) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
}

static int write_file(const char* dir, const char* name, const void* p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    size_t w = fwrite(p, 1, n, f);
    fclose(f);
    return w != n;
}

/* Decode a host stream on the GPU into `out` (host, n_bytes). */
static int gpu_decode(const uint8_t* stream, size_t len, ep_dtype container, void* out, size_t n_bytes) {
    ep_handle* h = NULL;
    ep_status st = ep_upload(stream, len, NULL, &h);
    if (st != EP_OK) return fail_ep("ep_upload", st);
    void* dev = NULL;
    hipError_t e = hipMalloc(&dev, n_bytes);
    if (e != hipSuccess) {
        ep_release(h);
        return fail_hip("hipMalloc", e);
    }
    int rc = 0;
    st = ep_decompress(h, container, dev, NULL, NULL);
    if (st == EP_OK) st = ep_handle_check(h, NULL);            /* synchronizes the stream */
    if (st != EP_OK) {
        rc = fail_ep("ep_decompress", st);
    } else if ((e = hipMemcpy(out, dev, n_bytes, hipMemcpyDeviceToHost)) != hipSuccess) {
        rc = fail_hip("hipMemcpy", e);
    }
    (void)hipFree(dev);
    ep_release(h);
    return rc;
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s <output dir>\n", argv[0]);
        return 2;
    }
    const int64_t R = 300, C = 700;
    float* w = (float*)malloc(sizeof(float) * (size_t)(R * C));
    float* back = (float*)malloc(sizeof(float) * (size_t)(R * C));
    uint16_t* bf = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(R * C));
    if (!w || !back || !bf) return 1;
    for (int64_t i = 0; i < R * C; ++i)
        w[i] = (float)(0.02 * (uniform01() + uniform01() + uniform01() + uniform01() - 2.0) * 1.7320508);

    /* 1. lossless round trip, checked here */
    ep_encode_opts lossless = {EP_MODE_LOSSLESS, 0.0, 12, 16, 0};
    uint8_t* s = NULL;
    size_t len = 0;
    double bpp = 0.0;
    ep_status st = ep_compress(w, EP_F32, R, C, &lossless, &s, &len, &bpp);
    if (st != EP_OK) return fail_ep("ep_compress (lossless)", st);
    if (gpu_decode(s, len, EP_F32, back, sizeof(float) * (size_t)(R * C))) return 1;
    ep_free(s);
    if (memcmp(w, back, sizeof(float) * (size_t)(R * C)) != 0) {
        fprintf(stderr, "lossless round trip differs\n");
        return 1;
    }
    printf("lossless fp32 round trip bit-exact at %.4f bpp\n", bpp);

    /* 2. lossy decode to BF16, written out for the oracle comparison */
    ep_encode_opts lossy = {EP_MODE_LOSSY_E8, 4.0, 12, 16, 0};
    st = ep_compress(w, EP_F32, R, C, &lossy, &s, &len, &bpp);
    if (st != EP_OK) return fail_ep("ep_compress (lossy)", st);
    ep_info info;
    st = ep_stream_info(s, len, &info);
    if (st != EP_OK) return fail_ep("ep_stream_info", st);
    if (info.rows != R || info.cols != C || info.actual_bpp != bpp) {
        fprintf(stderr, "stream info disagrees with the compress call\n");
        return 1;
    }
    if (gpu_decode(s, len, EP_BF16, bf, sizeof(uint16_t) * (size_t)(R * C))) return 1;
    if (write_file(argv[1], "lossy.epk", s, len) ||
        write_file(argv[1], "lossy_bf16.bin", bf, sizeof(uint16_t) * (size_t)(R * C))) {
        fprintf(stderr, "writing the outputs failed\n");
        return 1;
    }
    ep_free(s);
    printf("lossy 4.0 bpp target, %.4f bpp actual, decoded to BF16\n", bpp);
    free(w);
    free(back);
    free(bf);
    return 0;
}
