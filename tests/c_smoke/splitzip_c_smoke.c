/*
 * splitzip_c_smoke.c -- drives the SplitZip C ABI from plain C (no Python,
 * no torch): reads n bf16 bit patterns from a file, calibrates, encodes with
 * the given chunk size, decodes with validation and in place, and writes the
 * codebook, metadata, payload and both decoded copies to files for the
 * caller to check.  Exit status 0 only when every call succeeded.
 *
 * usage: splitzip_c_smoke IN N CHUNK OUT_PREFIX
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "splitzip.h"

#define CHECK_HIP(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
            return 2;                                                              \
        }                                                                          \
    } while (0)

#define CHECK_SZ(call)                                                             \
    do {                                                                           \
        int s_ = (call);                                                           \
        if (s_ != SPLITZIP_OK) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, splitzip_status_string(s_)); \
            return 3;                                                              \
        }                                                                          \
    } while (0)

static int write_file(const char *prefix, const char *suffix, const void *p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s.%s", prefix, suffix);
    FILE *f = fopen(path, "wb");
    if (!f) return 1;
    size_t w = bytes ? fwrite(p, 1, bytes, f) : 0;
    fclose(f);
    return w == bytes ? 0 : 1;
}

int main(int argc, char **argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: %s IN N CHUNK OUT_PREFIX\n", argv[0]);
        return 1;
    }
    const uint64_t n = strtoull(argv[2], NULL, 10);
    const uint32_t chunk = (uint32_t)strtoul(argv[3], NULL, 10);
    const char *prefix = argv[4];
    if (splitzip_abi_version() != SPLITZIP_ABI_VERSION) return 4;
    size_t cb_bytes = 0, meta_bytes = 0;
    splitzip_struct_sizes(&cb_bytes, &meta_bytes);
    if (cb_bytes != sizeof(splitzip_codebook) || meta_bytes != sizeof(splitzip_meta)) return 4;

    uint16_t *h_x = (uint16_t *)malloc(n * 2 + 16);
    FILE *f = fopen(argv[1], "rb");
    if (!h_x || !f || fread(h_x, 2, n, f) != n) return 1;
    fclose(f);

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    const uint64_t cap = splitzip_payload_size(n, n);
    const size_t ws_bytes = splitzip_workspace_size(n);
    const size_t slot_bytes = (size_t)(2 * n > cap ? 2 * n : cap) + 16;
    uint16_t *d_x, *d_out;
    uint8_t *d_payload, *d_slot, *d_stash;
    void *d_ws;
    splitzip_codebook *d_cb;
    splitzip_meta *d_meta;
    int32_t *d_status;
    CHECK_HIP(hipMalloc((void **)&d_x, n * 2 + 16));
    CHECK_HIP(hipMalloc((void **)&d_out, n * 2 + 16));
    CHECK_HIP(hipMalloc((void **)&d_payload, cap + 16));
    CHECK_HIP(hipMalloc((void **)&d_slot, slot_bytes));
    CHECK_HIP(hipMalloc((void **)&d_stash, cap + 16));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMalloc((void **)&d_cb, sizeof(splitzip_codebook)));
    CHECK_HIP(hipMalloc((void **)&d_meta, sizeof(splitzip_meta)));
    CHECK_HIP(hipMalloc((void **)&d_status, 4));
    CHECK_HIP(hipMemcpy(d_x, h_x, n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_status, 0, 4));

    CHECK_SZ(splitzip_workspace_init(d_ws, ws_bytes, stream));
    CHECK_SZ(splitzip_calibrate(d_x, n, d_cb, d_ws, ws_bytes, stream));
    CHECK_SZ(splitzip_encode_chunked(d_x, n, d_cb, chunk, d_payload, cap, d_meta, d_ws, ws_bytes,
                                     stream));
    const uint8_t *d_lut = (const uint8_t *)d_cb + offsetof(splitzip_codebook, dec_lut);
    CHECK_SZ(splitzip_decode(d_payload, cap, d_meta, d_lut, d_out, n, d_status, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    splitzip_codebook cb;
    splitzip_meta meta;
    int32_t status = -1;
    CHECK_HIP(hipMemcpy(&cb, d_cb, sizeof cb, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&meta, d_meta, sizeof meta, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
    if (meta.status != SPLITZIP_OK || status != 0) {
        fprintf(stderr, "meta status %d, decode status %d\n", meta.status, status);
        return 5;
    }
    uint8_t *h_payload = (uint8_t *)malloc(meta.comp_bytes + 1);
    uint16_t *h_out = (uint16_t *)malloc(n * 2 + 16);
    uint16_t *h_slot = (uint16_t *)malloc(n * 2 + 16);
    if (!h_payload || !h_out || !h_slot) return 1;
    CHECK_HIP(hipMemcpy(h_payload, d_payload, meta.comp_bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(h_out, d_out, n * 2, hipMemcpyDeviceToHost));

    /* in place: the payload at the head of the slot */
    CHECK_HIP(hipMemcpy(d_slot, d_payload, meta.comp_bytes, hipMemcpyDeviceToDevice));
    CHECK_SZ(splitzip_decode_slot(d_slot, slot_bytes, d_meta, d_lut, n, d_stash, cap + 16, NULL,
                                  stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(h_slot, d_slot, n * 2, hipMemcpyDeviceToHost));

    if (write_file(prefix, "cb", &cb, sizeof cb) || write_file(prefix, "meta", &meta, sizeof meta) ||
        write_file(prefix, "payload", h_payload, meta.comp_bytes) ||
        write_file(prefix, "out", h_out, n * 2) || write_file(prefix, "slot", h_slot, n * 2))
        return 1;
    printf("n=%llu chunk=%u n_esc=%llu comp_bytes=%llu n_codes=%u\n", (unsigned long long)n, chunk,
           (unsigned long long)meta.n_esc, (unsigned long long)meta.comp_bytes, cb.n_codes);

    hipFree(d_x); hipFree(d_out); hipFree(d_payload); hipFree(d_slot); hipFree(d_stash);
    hipFree(d_ws); hipFree(d_cb); hipFree(d_meta); hipFree(d_status);
    hipStreamDestroy(stream);
    free(h_x); free(h_payload); free(h_out); free(h_slot);
    return 0;
}
