/*
 * A C client of libbsq: the C ABI of include/bsq.h used with the HIP runtime
 * alone (no Python, no torch).  It owns its device memory (hipMalloc) and its
 * stream, quantizes a BF16 matrix read from a file, and writes the codes and
 * scales back to files for the test that runs it to compare with the CPU
 * oracle.
 *
 * Dense form: for NVFP4 it first computes the tensor scale on the device with
 * tensor_scale_nvfp4 and reads it back.  It also makes one call with an
 * invalid K and prints the library's message for it.
 *
 *   bsq_c_client <format 0|1|2> <M> <K> <x.bin> <codes.bin> <scales.bin> [tsf.bin]
 *
 * Grouped form: the routing metadata comes from files in <dir>; for NVFP4 the
 * per-expert tensor scales are produced on the device with
 * grouped_tensor_scale_nvfp4 and passed to grouped_quantize_block_scaled as
 * they are (no host round trip), then read back.  The output buffers are
 * filled with 0xA5 first, so bytes the call must not touch stay 0xA5.
 *
 *   bsq_c_client grouped <format> <S> <K> <G> <E> <max_rows> <num_scale_rows> <gather 0|1> <dir>
 *
 * <dir> holds x.bin (S * K uint16), ro.bin and so.bin (G + 1 uint32 each),
 * ids.bin (G int32) and, with gather, ri.bin (max_rows int32); the client
 * writes q.bin ([max_rows, K/2 or K]), s.bin ([num_scale_rows, K/bs]) and, for
 * NVFP4, tsf.bin (E float32) there.
 *
 * Little-endian, row-major throughout.  Exit status 0 on success; any failed
 * HIP or library call prints a message and exits with 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

static char* path_in(const char* dir, const char* name) {
    static char buf[4096];
    snprintf(buf, sizeof(buf), "%s/%s", dir, name);
    return buf;
}

static void* to_device(const void* host, size_t bytes, hipStream_t stream) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (bytes) HIP_OK(hipMemcpyAsync(d, host, bytes, hipMemcpyHostToDevice, stream));
    return d;
}

static int grouped_main(int argc, char** argv) {
    if (argc != 11) {
        fprintf(stderr, "usage: %s grouped format S K G E max_rows num_scale_rows gather dir\n",
                argv[0]);
        return 2;
    }
    const int format = atoi(argv[2]);
    const int64_t S = atoll(argv[3]), K = atoll(argv[4]), G = atoll(argv[5]), E = atoll(argv[6]);
    const int64_t max_rows = atoll(argv[7]), nsr = atoll(argv[8]);
    const int gather = atoi(argv[9]);
    const char* dir = argv[10];
    if (format < BSQ_MXFP4 || format > BSQ_NVFP4 || S <= 0 || K <= 0 || G <= 0 || E <= 0 ||
        max_rows <= 0 || nsr <= 0) {
        fprintf(stderr, "bad arguments\n");
        return 2;
    }
    const int bs = format == BSQ_NVFP4 ? 16 : 32;
    const int64_t width = format == BSQ_MXFP8 ? K : K / 2;
    const int64_t nblk = K / bs;
    const size_t qbytes = (size_t)(max_rows * width), sbytes = (size_t)(nsr * nblk);

    printf("libbsq %s (grouped)\n", bsq_version());
    HIP_OK(hipSetDevice(0));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void* hx = read_file(path_in(dir, "x.bin"), (size_t)(S * K) * 2);
    void* hro = read_file(path_in(dir, "ro.bin"), (size_t)(G + 1) * 4);
    void* hso = read_file(path_in(dir, "so.bin"), (size_t)(G + 1) * 4);
    void* hids = read_file(path_in(dir, "ids.bin"), (size_t)G * 4);
    void* hri = gather ? read_file(path_in(dir, "ri.bin"), (size_t)max_rows * 4) : NULL;
    void* dx = to_device(hx, (size_t)(S * K) * 2, stream);
    uint32_t* dro = (uint32_t*)to_device(hro, (size_t)(G + 1) * 4, stream);
    uint32_t* dso = (uint32_t*)to_device(hso, (size_t)(G + 1) * 4, stream);
    int32_t* dids = (int32_t*)to_device(hids, (size_t)G * 4, stream);
    int32_t* dri = gather ? (int32_t*)to_device(hri, (size_t)max_rows * 4, stream) : NULL;
    void *dq, *ds;
    HIP_OK(hipMalloc(&dq, qbytes));
    HIP_OK(hipMalloc(&ds, sbytes));
    HIP_OK(hipMemsetAsync(dq, 0xA5, qbytes, stream));
    HIP_OK(hipMemsetAsync(ds, 0xA5, sbytes, stream));

    float* dtsf = NULL;
    if (format == BSQ_NVFP4) {
        HIP_OK(hipMalloc((void**)&dtsf, (size_t)E * sizeof(float)));
        BSQ_OK_OR_DIE(grouped_tensor_scale_nvfp4(dx, S, K, K, dri, dro, dids, G, E, max_rows,
                                                 dtsf, stream));
    }
    BSQ_OK_OR_DIE(grouped_quantize_block_scaled(format, bs, BSQ_SCALES_ROW_MAJOR, dx, S, K, K, dri,
                                                dro, dso, dids, dtsf, G, E, max_rows, nsr, dq,
                                                width, ds, nblk, stream));
    /* an invalid call: NVFP4 without per-expert tensor scales, or a bad block size */
    const int bad = grouped_quantize_block_scaled(BSQ_NVFP4, 16, BSQ_SCALES_ROW_MAJOR, dx, S, K, K,
                                                  dri, dro, dso, dids, NULL, G, E, max_rows, nsr,
                                                  dq, K / 2, ds, K / 16, stream);
    printf("NVFP4 without tensor scales: status %d, message: %s\n", bad, bsq_last_error());
    if (bad != BSQ_ERR_INVALID_ARG) return 1;

    uint8_t* q = (uint8_t*)malloc(qbytes);
    uint8_t* sc = (uint8_t*)malloc(sbytes);
    HIP_OK(hipMemcpyAsync(q, dq, qbytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipMemcpyAsync(sc, ds, sbytes, hipMemcpyDeviceToHost, stream));
    float* tsf = NULL;
    if (dtsf) {
        tsf = (float*)malloc((size_t)E * sizeof(float));
        HIP_OK(hipMemcpyAsync(tsf, dtsf, (size_t)E * sizeof(float), hipMemcpyDeviceToHost,
                              stream));
    }
    HIP_OK(hipStreamSynchronize(stream));
    write_file(path_in(dir, "q.bin"), q, qbytes);
    write_file(path_in(dir, "s.bin"), sc, sbytes);
    if (tsf) write_file(path_in(dir, "tsf.bin"), tsf, (size_t)E * sizeof(float));

    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dro));
    HIP_OK(hipFree(dso));
    HIP_OK(hipFree(dids));
    if (dri) HIP_OK(hipFree(dri));
    if (dtsf) HIP_OK(hipFree(dtsf));
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(ds));
    HIP_OK(hipStreamDestroy(stream));
    free(hx);
    free(hro);
    free(hso);
    free(hids);
    free(hri);
    free(q);
    free(sc);
    free(tsf);
    printf("ok\n");
    return 0;
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "grouped") == 0) return grouped_main(argc, argv);
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
