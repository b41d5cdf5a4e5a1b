/*
 * A C client of libbsq: the C ABI of include/bsq.h used with the HIP runtime
 * alone (no Python, no torch).  It owns its device memory (hipMalloc) and its
 * stream, quantizes a BF16 matrix read from a file, and writes the codes and
 * scales back to files for the test that runs it to compare with the CPU
 * oracle.  For NVFP4 it first computes the tensor scale on the device with
 * tensor_scale_nvfp4 and reads it back.  It also makes one call with an
 * invalid K and prints the library's message for it.
 *
 *   bsq_c_client <format 0|1|2> <M> <K> <x.bin> <codes.bin> <scales.bin> [tsf.bin]
 *
 * x.bin holds M * K little-endian uint16 BF16 patterns, row-major.  Exit
 * status 0 on success; any failed HIP or library call prints a message and
 * exits with 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bsq.h"

#define HIP_OK(call)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

#define BSQ_OK_OR_DIE(call)                                                               \
    do {                                                                                  \
        int s_ = (call);                                                                  \
        if (s_ != BSQ_OK) {                                                               \
            fprintf(stderr, "%s returned %d: %s\n", #call, s_, bsq_last_error());         \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static void* read_file(const char* path, size_t bytes) {
    FILE* f = fopen(path, "rb");
    if (!f) { perror(path); exit(1); }
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(1); }
    fclose(f);
    return p;
}

static void write_file(const char* path, const void* p, size_t bytes) {
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(1); }
    fclose(f);
}

int main(int argc, char** argv) {
    if (argc < 7) {
        fprintf(stderr, "usage: %s format M K x.bin codes.bin scales.bin [tsf.bin]\n", argv[0]);
        return 2;
    }
    const int format = atoi(argv[1]);
    const int64_t M = atoll(argv[2]), K = atoll(argv[3]);
    if (format < BSQ_MXFP4 || format > BSQ_NVFP4 || M <= 0 || K <= 0) {
        fprintf(stderr, "bad arguments\n");
        return 2;
    }
    const int bs = format == BSQ_NVFP4 ? 16 : 32;
    const int64_t width = format == BSQ_MXFP8 ? K : K / 2;   /* code bytes per row */
    const int64_t nblk = K / bs;

    printf("libbsq %s\n", bsq_version());
    uint16_t* x = (uint16_t*)read_file(argv[4], (size_t)(M * K) * 2);

    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *dx, *dq, *ds;
    float* dtsf;
    HIP_OK(hipMalloc(&dx, (size_t)(M * K) * 2));
    HIP_OK(hipMalloc(&dq, (size_t)(M * width)));
    HIP_OK(hipMalloc(&ds, (size_t)(M * nblk)));
    HIP_OK(hipMalloc((void**)&dtsf, sizeof(float)));
    HIP_OK(hipMemcpyAsync(dx, x, (size_t)(M * K) * 2, hipMemcpyHostToDevice, stream));

    float tsf = 1.0f;
    if (format == BSQ_NVFP4) {
        BSQ_OK_OR_DIE(tensor_scale_nvfp4(dx, M, K, K, dtsf, stream));
        HIP_OK(hipMemcpyAsync(&tsf, dtsf, sizeof(float), hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
        printf("tensor scale %.9g\n", (double)tsf);
    }
    BSQ_OK_OR_DIE(quantize_block_scaled(format, bs, BSQ_SCALES_ROW_MAJOR, dx, M, K, K, dq, width,
                                        ds, nblk, tsf, stream));

    /* an invalid call: K not a multiple of the block, rejected before any launch */
    const int bad = quantize_block_scaled(format, bs, BSQ_SCALES_ROW_MAJOR, dx, M, bs + 8, K, dq,
                                          width, ds, nblk, tsf, stream);
    printf("invalid K: status %d, message: %s\n", bad, bsq_last_error());
    if (bad != BSQ_ERR_INVALID_ARG) return 1;

    uint8_t* q = (uint8_t*)malloc((size_t)(M * width));
    uint8_t* s = (uint8_t*)malloc((size_t)(M * nblk));
    HIP_OK(hipMemcpyAsync(q, dq, (size_t)(M * width), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(s, ds, (size_t)(M * nblk), hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    write_file(argv[5], q, (size_t)(M * width));
    write_file(argv[6], s, (size_t)(M * nblk));
    if (argc > 7) write_file(argv[7], &tsf, sizeof(float));

    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(ds));
    HIP_OK(hipFree(dtsf));
    HIP_OK(hipStreamDestroy(stream));
    free(x);
    free(q);
    free(s);
    printf("ok\n");
    return 0;
}
