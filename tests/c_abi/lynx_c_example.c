/*
 * A plain C consumer of liblynx: no Python and no torch, only the C ABI of
 * include/lynx.h and the HIP runtime.
 *
 *     lynx_c_example DIR M N K R
 *
 * Reads DIR/X.bin [M][K], DIR/W.bin [N][K], and for R > 0 DIR/LA.bin [N][R]
 * and DIR/LB.bin [R][K] (bf16 bit patterns, little-endian uint16, row-major).
 * It copies them to device buffers from hipMalloc, sizes and allocates the
 * workspace with lynx_workspace_bytes, and runs lynx_linear_sparse_lora (the
 * RT-Lynx layer, Y = s (X~ W^T) + (X LB^T) LA^T) and lynx_linear_dense
 * (Y = X W^T) on one stream. It writes DIR/Y_sparse.bin and DIR/Y_dense.bin
 * ([M][N] bf16 bits).
 *
 * Exit status: 0 on success; 2 for bad arguments; 3 for a file error; 4 for a
 * HIP error; 5 for a status other than LYNX_OK from the library (its
 * lynx_status_string is printed).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lynx.h"

#define HIP_OK(call)                                                                 \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            exit(4);                                                                 \
        }                                                                            \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        exit(3);
    }
    void* buf = malloc(bytes > 0 ? bytes : 1);
    if (!buf || fread(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
        exit(3);
    }
    fclose(f);
    return buf;
}

static void write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(3);
    }
    fclose(f);
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 1));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void lynx_ok(lynx_status st, const char* what) {
    if (st != LYNX_OK) {
        fprintf(stderr, "%s: %s\n", what, lynx_status_string(st));
        exit(5);
    }
}

int main(int argc, char** argv) {
    if (argc != 6) {
        fprintf(stderr, "usage: %s DIR M N K R\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    const int64_t M = atoll(argv[2]), N = atoll(argv[3]), K = atoll(argv[4]), R = atoll(argv[5]);
    if (M <= 0 || N <= 0 || K <= 0 || R < 0) {
        fprintf(stderr, "M, N and K must be positive and R non-negative\n");
        return 2;
    }
    const size_t bx = (size_t)(M * K) * 2, bw = (size_t)(N * K) * 2;
    const size_t bla = (size_t)(N * R) * 2, blb = (size_t)(R * K) * 2, by = (size_t)(M * N) * 2;

    void* hX = read_file(dir, "X.bin", bx);
    void* hW = read_file(dir, "W.bin", bw);
    void* hLA = R > 0 ? read_file(dir, "LA.bin", bla) : NULL;
    void* hLB = R > 0 ? read_file(dir, "LB.bin", blb) : NULL;

    uint16_t* X = (uint16_t*)to_device(hX, bx);
    uint16_t* W = (uint16_t*)to_device(hW, bw);
    uint16_t* LA = R > 0 ? (uint16_t*)to_device(hLA, bla) : NULL;
    uint16_t* LB = R > 0 ? (uint16_t*)to_device(hLB, blb) : NULL;
    uint16_t *Ys = NULL, *Yd = NULL;
    HIP_OK(hipMalloc((void**)&Ys, by));
    HIP_OK(hipMalloc((void**)&Yd, by));

    const size_t ws_bytes = lynx_workspace_bytes(M, K, R);
    if (ws_bytes == 0) {
        fprintf(stderr, "lynx_workspace_bytes: shape not supported\n");
        return 5;
    }
    void* ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    lynx_ok(lynx_linear_sparse_lora(X, W, LA, LB, Ys, M, N, K, R, ws, ws_bytes, (lynx_stream_t)stream),
            "lynx_linear_sparse_lora");
    lynx_ok(lynx_linear_dense(X, W, Yd, M, N, K, (lynx_stream_t)stream), "lynx_linear_dense");
    HIP_OK(hipStreamSynchronize(stream));

    void* h = malloc(by);
    if (!h) return 3;
    HIP_OK(hipMemcpy(h, Ys, by, hipMemcpyDeviceToHost));
    write_file(dir, "Y_sparse.bin", h, by);
    HIP_OK(hipMemcpy(h, Yd, by, hipMemcpyDeviceToHost));
    write_file(dir, "Y_dense.bin", h, by);

    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(Ys));
    HIP_OK(hipFree(Yd));
    HIP_OK(hipFree(X));
    HIP_OK(hipFree(W));
    if (R > 0) {
        HIP_OK(hipFree(LA));
        HIP_OK(hipFree(LB));
    }
    free(h);
    free(hX);
    free(hW);
    free(hLA);
    free(hLB);
    printf("lynx_c_example: M=%lld N=%lld K=%lld R=%lld ok (library version %d)\n", (long long)M,
           (long long)N, (long long)K, (long long)R, lynx_version());
    return 0;
}
