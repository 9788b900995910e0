/*
 * A plain C client of libswiglu_gateup.so: no Python, no torch. Every entry
 * point of swiglu_gateup.h is called through the C ABI on one HIP stream.
 * Inputs are read from files as raw bit patterns (bf16) or fp32, copied to
 * the device, and the outputs are written back to files:
 *
 *   c_abi_client gateup     rows n x dy | y dx dx_in_place
 *       packed forward, out-of-place and in-place backward; also checks that
 *       bad arguments come back as the documented status codes
 *   c_abi_client silu_mul   rows n x dy | y dx dx_in_place
 *       the two-tensor entry points on gate = x[:, :n] and up = x[:, n:]
 *       (row strides 2n); dgate and dup land in the two halves of dx
 *   c_abi_client bias_scale rows n x dy bias scale | y dx dbias dscale
 *       bias [2n] (bf16) and scale [rows] (fp32); the backward writes dx,
 *       dbias and dscale (fp32) with a workspace of the size the library
 *       asks for
 *   c_abi_client fc1        m n k a w | y x_out
 *       y = silu(a wg^T) * (a wu^T) with a [m, k] and w [2n, k], and the
 *       [m, 2n] product
 *
 * (inputs before the bar, outputs after it). Exit status 0 on success; any
 * HIP or library error prints a message and exits 1.
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

/* A device buffer holding the contents of a file. */
static void* upload(const char* path, size_t bytes) {
    void* h = read_file(path, bytes);
    void* d;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    free(h);
    return d;
}

/* Writes a device buffer to a file. */
static void download(const char* path, const void* d, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    if (!h) exit(1);
    HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    write_file(path, h, bytes);
    free(h);
}

static void* dev_alloc(size_t bytes) {
    void* d;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    return d;
}

/* exits unless the two device buffers hold the same bytes */
static void check_equal(const void* d1, const void* d2, size_t bytes, const char* what) {
    unsigned char* h1 = (unsigned char*)malloc(bytes ? bytes : 1);
    unsigned char* h2 = (unsigned char*)malloc(bytes ? bytes : 1);
    if (!h1 || !h2) exit(1);
    HIP_OK(hipMemcpy(h1, d1, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h2, d2, bytes, hipMemcpyDeviceToHost));
    if (memcmp(h1, h2, bytes) != 0) {
        fprintf(stderr, "%s: outputs differ\n", what);
        exit(1);
    }
    free(h1);
    free(h2);
}

static void expect(swiglu_status got, swiglu_status want, const char* what) {
    if (got != want) {
        fprintf(stderr, "%s: got %s, want %s\n", what, swiglu_status_string(got),
                swiglu_status_string(want));
        exit(1);
    }
}

static void usage(const char* prog) {
    fprintf(stderr,
            "usage: %s gateup|silu_mul rows n x dy y dx dx_in_place\n"
            "       %s bias_scale rows n x dy bias scale y dx dbias dscale\n"
            "       %s fc1 m n k a w y x_out\n",
            prog, prog, prog);
    exit(1);
}

static void run_gateup(int two_tensor, char** a, hipStream_t st) {
    const int64_t rows = atoll(a[0]), n = atoll(a[1]);
    const size_t xb = (size_t)(rows * 2 * n) * 2, yb = (size_t)(rows * n) * 2;
    char* x = (char*)upload(a[2], xb);
    char* xi = (char*)upload(a[2], xb);
    void* dy = upload(a[3], yb);
    void* y = dev_alloc(yb);
    char* dx = (char*)dev_alloc(xb);
    const swiglu_dtype bf = SWIGLU_DTYPE_BF16;
    if (!two_tensor) {
        /* argument errors come back before any launch */
        expect(swiglu_gateup_fwd(x, 2 * n - 1, y, n, rows, n, bf, st), SWIGLU_ERR_BAD_STRIDE,
               "x row stride below 2n");
        expect(swiglu_gateup_fwd(x, 2 * n, y, n, rows, n, (swiglu_dtype)7, st),
               SWIGLU_ERR_BAD_DTYPE, "unknown dtype");
        expect(swiglu_gateup_bwd(dy, n, x, 2 * n, x, 2 * n, rows, n, bf, 0, st),
               SWIGLU_ERR_ALIASING, "out-of-place dx over x");
        expect(swiglu_gateup_fwd(NULL, 2 * n, y, n, rows, n, bf, st), SWIGLU_ERR_NULL_POINTER,
               "NULL x");
        SW_OK(swiglu_gateup_fwd(x, 2 * n, y, n, rows, n, bf, st));
        SW_OK(swiglu_gateup_bwd(dy, n, x, 2 * n, dx, 2 * n, rows, n, bf, 0, st));
        SW_OK(swiglu_gateup_bwd(dy, n, xi, 2 * n, NULL, 0, rows, n, bf, 1, st));
    } else {
        /* gate and up are the two halves of x, dgate and dup those of dx */
        const int64_t h = n * 2; /* bytes to the up half */
        expect(swiglu_silu_mul_fwd(x, 2 * n, x + h, 2 * n, x, n, rows, n, bf, st),
               SWIGLU_ERR_ALIASING, "two-tensor y over gate");
        SW_OK(swiglu_silu_mul_fwd(x, 2 * n, x + h, 2 * n, y, n, rows, n, bf, st));
        SW_OK(swiglu_silu_mul_bwd(dy, n, x, 2 * n, x + h, 2 * n, dx, 2 * n, dx + h, 2 * n, rows,
                                  n, bf, 0, st));
        SW_OK(swiglu_silu_mul_bwd(dy, n, xi, 2 * n, xi + h, 2 * n, NULL, 0, NULL, 0, rows, n, bf,
                                  1, st));
    }
    HIP_OK(hipStreamSynchronize(st));
    download(a[4], y, yb);
    download(a[5], dx, xb);
    download(a[6], xi, xb);
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(xi));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(dx));
}

static void run_bias_scale(char** a, hipStream_t st) {
    const int64_t rows = atoll(a[0]), n = atoll(a[1]);
    const size_t xb = (size_t)(rows * 2 * n) * 2, yb = (size_t)(rows * n) * 2;
    void* x = upload(a[2], xb);
    void* dy = upload(a[3], yb);
    void* bias = upload(a[4], (size_t)(2 * n) * 2);
    float* scale = (float*)upload(a[5], (size_t)rows * 4);
    void* y = dev_alloc(yb);
    void* dx = dev_alloc(xb);
    float* dbias = (float*)dev_alloc((size_t)(2 * n) * 4);
    float* dscale = (float*)dev_alloc((size_t)rows * 4);
    const swiglu_dtype bf = SWIGLU_DTYPE_BF16;
    const size_t wsb = swiglu_gateup_bias_scale_workspace_size(rows, n, 1, 1);
    void* ws = dev_alloc(wsb);
    expect(swiglu_gateup_bias_scale_bwd(dy, n, x, 2 * n, bias, scale, 1, dx, 2 * n, dbias, dscale,
                                        1, ws, wsb / 2, rows, n, bf, 0, st),
           SWIGLU_ERR_WORKSPACE, "workspace too small");
    expect(swiglu_gateup_bias_scale_bwd(dy, n, x, 2 * n, NULL, scale, 1, dx, 2 * n, dbias, dscale,
                                        1, ws, wsb, rows, n, bf, 0, st),
           SWIGLU_ERR_NULL_POINTER, "dbias without a bias");
    SW_OK(swiglu_gateup_bias_scale_fwd(x, 2 * n, bias, scale, 1, y, n, rows, n, bf, st));
    SW_OK(swiglu_gateup_bias_scale_bwd(dy, n, x, 2 * n, bias, scale, 1, dx, 2 * n, dbias, dscale,
                                       1, ws, wsb, rows, n, bf, 0, st));
    HIP_OK(hipStreamSynchronize(st));
    download(a[6], y, yb);
    download(a[7], dx, xb);
    download(a[8], dbias, (size_t)(2 * n) * 4);
    download(a[9], dscale, (size_t)rows * 4);
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(bias));
    HIP_OK(hipFree(scale));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dbias));
    HIP_OK(hipFree(dscale));
    HIP_OK(hipFree(ws));
}

static void run_fc1(char** a, hipStream_t st) {
    const int64_t m = atoll(a[0]), n = atoll(a[1]), k = atoll(a[2]);
    const size_t ab = (size_t)(m * k) * 2, wb = (size_t)(2 * n * k) * 2;
    const size_t yb = (size_t)(m * n) * 2, xb = (size_t)(m * 2 * n) * 2;
    void* ad = upload(a[3], ab);
    void* wd = upload(a[4], wb);
    void* y = dev_alloc(yb);
    void* xo = dev_alloc(xb);
    void* y2 = dev_alloc(yb);
    /* the tile-queue workspace: zeroed once, left zeroed by every call */
    void* ws = dev_alloc(swiglu_fc1_workspace_size());
    HIP_OK(hipMemsetAsync(ws, 0, swiglu_fc1_workspace_size(), st));
    expect(swiglu_fc1_fwd(ad, k, wd, k, y, n, NULL, 0, m, n, k, SWIGLU_DTYPE_F32, NULL, st),
           SWIGLU_ERR_BAD_DTYPE, "fc1 in fp32");
    expect(swiglu_fc1_fwd(ad, k, wd, k, y, n, NULL, 0, m, n, k, SWIGLU_DTYPE_BF16,
                          (char*)ws + 8, st),
           SWIGLU_ERR_BAD_STRIDE, "fc1 with a misaligned workspace");
    SW_OK(swiglu_fc1_fwd(ad, k, wd, k, y, n, xo, 2 * n, m, n, k, SWIGLU_DTYPE_BF16, ws, st));
    SW_OK(swiglu_fc1_fwd(ad, k, wd, k, y2, n, NULL, 0, m, n, k, SWIGLU_DTYPE_BF16, NULL, st));
    HIP_OK(hipStreamSynchronize(st));
    check_equal(y, y2, yb, "fc1 with and without a workspace");
    download(a[5], y, yb);
    download(a[6], xo, xb);
    HIP_OK(hipFree(ad));
    HIP_OK(hipFree(wd));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(y2));
    HIP_OK(hipFree(xo));
    HIP_OK(hipFree(ws));
}

int main(int argc, char** argv) {
    if (argc < 2) usage(argv[0]);
    const char* cmd = argv[1];
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    if ((!strcmp(cmd, "gateup") || !strcmp(cmd, "silu_mul")) && argc == 9)
        run_gateup(!strcmp(cmd, "silu_mul"), argv + 2, st);
    else if (!strcmp(cmd, "bias_scale") && argc == 12)
        run_bias_scale(argv + 2, st);
    else if (!strcmp(cmd, "fc1") && argc == 9)
        run_fc1(argv + 2, st);
    else
        usage(argv[0]);
    HIP_OK(hipStreamDestroy(st));
    printf("c_abi_client: ok\n");
    return 0;
}
