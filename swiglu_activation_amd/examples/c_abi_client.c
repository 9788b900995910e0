/*
 * A plain C client of libswiglu_gateup.so: no Python, no torch. It reads x
 * ([rows, 2n]) and dy ([rows, n]) as raw bf16 bit patterns from two files,
 * copies them to the device, runs the fused forward, the out-of-place
 * backward and the in-place backward on one stream through the C ABI, and
 * writes y, dx and the in-place result to three files. It also checks that
 * bad arguments come back as the documented status codes without a launch.
 *
 *   c_abi_client rows n x.bin dy.bin y.bin dx.bin dx_in_place.bin
 *
 * Exit status 0 on success; any HIP or library error prints a message and
 * exits 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "swiglu_gateup.h"

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
            exit(1);                                                            \
        }                                                                       \
    } while (0)

#define SW_OK(call)                                                                     \
    do {                                                                                \
        swiglu_status s_ = (call);                                                      \
        if (s_ != SWIGLU_OK) {                                                          \
            fprintf(stderr, "%s returned %s\n", #call, swiglu_status_string(s_));       \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

static void* read_file(const char* path, size_t bytes) {
    FILE* f = fopen(path, "rb");
    void* p = malloc(bytes ? bytes : 1);
    if (!f || !p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
        exit(1);
    }
    fclose(f);
    return p;
}

static void write_file(const char* path, const void* p, size_t bytes) {
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot write %s\n", path);
        exit(1);
    }
    fclose(f);
}

static void expect(swiglu_status got, swiglu_status want, const char* what) {
    if (got != want) {
        fprintf(stderr, "%s: got %s, want %s\n", what, swiglu_status_string(got),
                swiglu_status_string(want));
        exit(1);
    }
}

int main(int argc, char** argv) {
    if (argc != 8) {
        fprintf(stderr, "usage: %s rows n x.bin dy.bin y.bin dx.bin dx_in_place.bin\n", argv[0]);
        return 1;
    }
    const int64_t rows = atoll(argv[1]), n = atoll(argv[2]);
    const size_t xb = (size_t)(rows * 2 * n) * 2, yb = (size_t)(rows * n) * 2;
    void* hx = read_file(argv[3], xb);
    void* hdy = read_file(argv[4], yb);

    void *x, *dy, *y, *dx, *xi;
    HIP_OK(hipMalloc(&x, xb));
    HIP_OK(hipMalloc(&dy, yb));
    HIP_OK(hipMalloc(&y, yb));
    HIP_OK(hipMalloc(&dx, xb));
    HIP_OK(hipMalloc(&xi, xb));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    HIP_OK(hipMemcpy(x, hx, xb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(xi, hx, xb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy, hdy, yb, hipMemcpyHostToDevice));

    /* argument errors come back before any launch */
    expect(swiglu_gateup_fwd(x, 2 * n - 1, y, n, rows, n, SWIGLU_DTYPE_BF16, st),
           SWIGLU_ERR_BAD_STRIDE, "x row stride below 2n");
    expect(swiglu_gateup_fwd(x, 2 * n, y, n, rows, n, (swiglu_dtype)7, st),
           SWIGLU_ERR_BAD_DTYPE, "unknown dtype");
    expect(swiglu_gateup_bwd(dy, n, x, 2 * n, x, 2 * n, rows, n, SWIGLU_DTYPE_BF16, 0, st),
           SWIGLU_ERR_ALIASING, "out-of-place dx over x");
    expect(swiglu_gateup_fwd(NULL, 2 * n, y, n, rows, n, SWIGLU_DTYPE_BF16, st),
           SWIGLU_ERR_NULL_POINTER, "NULL x");

    SW_OK(swiglu_gateup_fwd(x, 2 * n, y, n, rows, n, SWIGLU_DTYPE_BF16, st));
    SW_OK(swiglu_gateup_bwd(dy, n, x, 2 * n, dx, 2 * n, rows, n, SWIGLU_DTYPE_BF16, 0, st));
    SW_OK(swiglu_gateup_bwd(dy, n, xi, 2 * n, NULL, 0, rows, n, SWIGLU_DTYPE_BF16, 1, st));
    HIP_OK(hipStreamSynchronize(st));

    void* h = malloc(xb);
    HIP_OK(hipMemcpy(h, y, yb, hipMemcpyDeviceToHost));
    write_file(argv[5], h, yb);
    HIP_OK(hipMemcpy(h, dx, xb, hipMemcpyDeviceToHost));
    write_file(argv[6], h, xb);
    HIP_OK(hipMemcpy(h, xi, xb, hipMemcpyDeviceToHost));
    write_file(argv[7], h, xb);

    HIP_OK(hipStreamDestroy(st));
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(xi));
    free(h);
    free(hx);
    free(hdy);
    printf("c_abi_client: ok\n");
    return 0;
}
