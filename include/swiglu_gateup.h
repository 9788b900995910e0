/*
 * swiglu_gateup.h -- C ABI of the fused gate-up SwiGLU for AMD MI355X (gfx950).
 *
 * The operation (Liger-Kernel Megatron SwiGLU page, §Background and
 * §What's added): the fc1 projection of a Megatron-style MLP produces ONE
 * packed tensor x of shape [rows, 2n] -- rows are the flattened leading
 * dimensions (tokens, or sequence x batch), the gate half g is columns [0, n)
 * and the up half u is columns [n, 2n). The fused forward reads both halves of
 * each row through a column offset, with no split, copy or concatenation, and
 * writes y = silu(g) * u of shape [rows, n]; silu(z) = z * sigma(z),
 * sigma(z) = 1 / (1 + exp(-z)). The backward recomputes silu from the saved x
 * and writes dx = [dgate | dup] of shape [rows, 2n] with
 *     dgate = dy * u * sigma(g) * (1 + g * (1 - sigma(g)))
 *     dup   = dy * silu(g)
 * either into a separate buffer or, in place, over x (same page, §Optional
 * in_place). Supported element types are fp32 and bf16 (same page, §Megatron
 * feature compatibility). All arithmetic is fp32 in registers; bf16 results
 * are rounded once, to nearest even.
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers on the current HIP device. The caller owns
 *    every buffer; the library allocates nothing, frees nothing, keeps no
 *    per-call state, and never synchronizes. (The one static buffer, the
 *    scratch of swiglu_gateup_bias_scale_bwd_noalloc, is part of the
 *    library's code object on each GPU, not an allocation made by a call.)
 *  - Row strides are counted in ELEMENTS (not bytes); columns are contiguous
 *    (unit stride). A row stride larger than the row's width is allowed (for
 *    example a view into a wider buffer); the columns past the width are never
 *    read or written.
 *  - Work is enqueued on `stream` (0 = the null stream) and runs
 *    asynchronously; a return of SWIGLU_OK means "validated and launched".
 *  - Every argument check happens on the host before anything is launched. On
 *    an error nothing is written and no HIP call is made.
 *  - rows == 0 or n == 0 is a valid empty problem: SWIGLU_OK, no launch (the
 *    dtype, shape and stride checks still apply).
 *  - n must be below 2^31 (SWIGLU_ERR_BAD_SHAPE otherwise).
 *  - Pointer alignment is never an error: 16-byte vector loads and stores are
 *    used when the base pointers, n and the row strides allow them, narrower
 *    accesses otherwise.
 *  - Results are bitwise deterministic, and the in-place backward produces the
 *    same bits as the out-of-place one.
 *  - Two calls that write the same memory must not run concurrently.
 */
#ifndef SWIGLU_GATEUP_H
#define SWIGLU_GATEUP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x, y, dy and dx (all four share it). */
typedef enum {
    SWIGLU_DTYPE_F32 = 0,   /* IEEE binary32 */
    SWIGLU_DTYPE_BF16 = 1   /* bfloat16: 1 sign, 8 exponent, 7 mantissa bits */
} swiglu_dtype;

typedef enum {
    SWIGLU_OK = 0,
    SWIGLU_ERR_NULL_POINTER = 1,  /* a required pointer is NULL (and the problem is not empty) */
    SWIGLU_ERR_BAD_SHAPE = 2,     /* rows < 0, n < 0, or 2n / rows*stride overflow int64 */
    SWIGLU_ERR_BAD_STRIDE = 3,    /* a row stride is smaller than its row's width */
    SWIGLU_ERR_BAD_DTYPE = 4,     /* dtype is neither SWIGLU_DTYPE_F32 nor SWIGLU_DTYPE_BF16 */
    SWIGLU_ERR_ALIASING = 5,      /* outputs overlap inputs where that is not allowed */
    SWIGLU_ERR_HIP = 6,           /* a HIP runtime call or kernel launch failed */
    SWIGLU_ERR_WORKSPACE = 7,     /* a needed workspace is NULL, too small or not 16-byte aligned */
    SWIGLU_ERR_SCRATCH_LIMIT = 8  /* the problem needs more than the static scratch holds
                                     (swiglu_gateup_bias_scale_bwd_noalloc only) */
} swiglu_status;

/*
 * Forward (Liger-Kernel Megatron SwiGLU page, §Background: input row stride
 * 2n, output row stride n).
 *
 *   x            [rows, 2n] input, read only; row r starts at x + r*x_row_stride.
 *   x_row_stride elements between rows of x; must be >= 2n.
 *   y            [rows, n] output; row r starts at y + r*y_row_stride.
 *   y_row_stride elements between rows of y; must be >= n.
 *   rows, n      problem size; >= 0.
 *   dtype        element type of x and y.
 *   stream       HIP stream the kernel is enqueued on.
 *
 * Errors: SWIGLU_ERR_NULL_POINTER (x or y NULL), SWIGLU_ERR_BAD_SHAPE,
 * SWIGLU_ERR_BAD_STRIDE, SWIGLU_ERR_BAD_DTYPE, SWIGLU_ERR_ALIASING (the
 * memory span of y overlaps that of x), SWIGLU_ERR_HIP (launch failed).
 */
swiglu_status swiglu_gateup_fwd(const void* x, int64_t x_row_stride,
                                void* y, int64_t y_row_stride,
                                int64_t rows, int64_t n,
                                swiglu_dtype dtype, hipStream_t stream);

/*
 * Backward (same page, §What's added: a backward kernel over the [tokens, 2n]
 * layout; §Optional in_place: the gradient may overwrite the fc1 output).
 *
 *   dy            [rows, n] upstream gradient, read only.
 *   dy_row_stride elements between rows of dy; must be >= n.
 *   x             [rows, 2n] saved forward input. Read only when in_place == 0;
 *                 when in_place != 0 it is read and then overwritten, element
 *                 by element, with dx = [dgate | dup].
 *   x_row_stride  elements between rows of x; must be >= 2n.
 *   dx            out of place: [rows, 2n] output buffer, must not overlap x
 *                 or dy. In place: must be NULL or equal to x (x is then the
 *                 output).
 *   dx_row_stride out of place: elements between rows of dx, >= 2n. In place:
 *                 ignored (x_row_stride is used).
 *   rows, n       problem size; >= 0.
 *   dtype         element type of dy, x and dx.
 *   in_place      0 = write dx; nonzero = overwrite x.
 *   stream        HIP stream the kernel is enqueued on.
 *
 * Errors: SWIGLU_ERR_NULL_POINTER (dy or x NULL, or dx NULL out of place),
 * SWIGLU_ERR_BAD_SHAPE, SWIGLU_ERR_BAD_STRIDE, SWIGLU_ERR_BAD_DTYPE,
 * SWIGLU_ERR_ALIASING (out of place: dx overlaps x or dy; in place: dx is
 * neither NULL nor x, or dy overlaps x), SWIGLU_ERR_HIP (launch failed).
 */
swiglu_status swiglu_gateup_bwd(const void* dy, int64_t dy_row_stride,
                                void* x, int64_t x_row_stride,
                                void* dx, int64_t dx_row_stride,
                                int64_t rows, int64_t n,
                                swiglu_dtype dtype, int in_place, hipStream_t stream);

/*
 * Two-tensor forward (Liger-Kernel Megatron SwiGLU page, §Background: Liger's
 * existing SiLU-times-up op takes gate and up as two separate tensors, the
 * layout of models whose gate and up projections are separate GEMMs).
 * Same arithmetic as swiglu_gateup_fwd, on two [rows, n] inputs.
 *
 *   gate, up      [rows, n] inputs, read only; each has its own row stride
 *                 (>= n). They may overlap each other.
 *   y             [rows, n] output, row stride >= n; must not overlap gate or up.
 *   rows, n, dtype, stream: as for swiglu_gateup_fwd.
 *
 * Errors: SWIGLU_ERR_NULL_POINTER, SWIGLU_ERR_BAD_SHAPE, SWIGLU_ERR_BAD_STRIDE,
 * SWIGLU_ERR_BAD_DTYPE, SWIGLU_ERR_ALIASING (y overlaps gate or up),
 * SWIGLU_ERR_HIP.
 */
swiglu_status swiglu_silu_mul_fwd(const void* gate, int64_t gate_row_stride,
                                  const void* up, int64_t up_row_stride,
                                  void* y, int64_t y_row_stride,
                                  int64_t rows, int64_t n,
                                  swiglu_dtype dtype, hipStream_t stream);

/*
 * Two-tensor backward: dgate = dy * up * sigma(gate) * (1 + gate (1 - sigma(gate))),
 * dup = dy * silu(gate), each [rows, n].
 *
 *   dy            [rows, n], read only, row stride >= n.
 *   gate, up      [rows, n] saved forward inputs, row strides >= n. Read only
 *                 when in_place == 0; when in_place != 0 dgate overwrites gate
 *                 and dup overwrites up.
 *   dgate, dup    out of place: [rows, n] outputs with their own row strides;
 *                 they must not overlap each other, dy, gate or up. In place:
 *                 each must be NULL or equal to gate / up respectively (their
 *                 strides are then ignored).
 *   in_place      0 = write dgate, dup; nonzero = overwrite gate and up (which
 *                 must then not overlap each other or dy).
 *
 * Errors: SWIGLU_ERR_NULL_POINTER, SWIGLU_ERR_BAD_SHAPE, SWIGLU_ERR_BAD_STRIDE,
 * SWIGLU_ERR_BAD_DTYPE, SWIGLU_ERR_ALIASING, SWIGLU_ERR_HIP.
 */
swiglu_status swiglu_silu_mul_bwd(const void* dy, int64_t dy_row_stride,
                                  void* gate, int64_t gate_row_stride,
                                  void* up, int64_t up_row_stride,
                                  void* dgate, int64_t dgate_row_stride,
                                  void* dup, int64_t dup_row_stride,
                                  int64_t rows, int64_t n,
                                  swiglu_dtype dtype, int in_place, hipStream_t stream);

/*
 * Bias and per-token scale variants (Liger-Kernel Megatron SwiGLU page,
 * §Scope and §Known issues: Megatron's activation may take a bias on the fc1
 * output, and MoE routed experts use a version weighted by a per-token
 * scale; the page names both and prints no formula). With
 *     z = x + bias                     (bias: [2n], the same for every row)
 *     y[r, c] = s[r] * silu(z[r, c]) * z[r, n + c]
 * and bias = 0 / s = 1 when the pointer is NULL, the backward writes
 *     dx    = dz, the base backward at z with upstream gradient s[r] * dy
 *     dbias = sum over rows of dx                            ([2n], fp32)
 *     ds[r] = sum over c of dy[r, c] * silu(z[r, c]) * z[r, n + c]  ([rows], fp32)
 * The sums are accumulated in fp32 from the fp32 values of dz (before any
 * rounding to bf16) in a fixed order, so results are bitwise deterministic.
 *
 * Forward:
 *   x, x_row_stride, y, y_row_stride, rows, n, dtype, stream: as in
 *                 swiglu_gateup_fwd.
 *   bias          NULL or [2n] elements of dtype (gate part, then up part).
 *   scale         NULL or fp32 per row: s[r] = scale[r * scale_stride];
 *                 scale_stride >= 1 when scale is given.
 * Errors: as swiglu_gateup_fwd; also SWIGLU_ERR_BAD_STRIDE (scale_stride < 1
 * with a scale) and SWIGLU_ERR_ALIASING (y overlaps bias or scale).
 */
swiglu_status swiglu_gateup_bias_scale_fwd(const void* x, int64_t x_row_stride,
                                           const void* bias, const float* scale,
                                           int64_t scale_stride,
                                           void* y, int64_t y_row_stride,
                                           int64_t rows, int64_t n,
                                           swiglu_dtype dtype, hipStream_t stream);

/*
 * Bytes of workspace swiglu_gateup_bias_scale_bwd needs for a problem of
 * this size when dbias (want_dbias != 0) and/or ds (want_dscale != 0) are
 * requested; 0 when neither is, and for empty or invalid sizes. The value
 * does not depend on pointers or dtype.
 */
size_t swiglu_gateup_bias_scale_workspace_size(int64_t rows, int64_t n,
                                               int want_dbias, int want_dscale);

/*
 * Backward of swiglu_gateup_bias_scale_fwd.
 *
 *   dy, x, dx, their strides, rows, n, dtype, in_place, stream: as in
 *                 swiglu_gateup_bwd (dx receives dz; in place it overwrites x).
 *   bias, scale, scale_stride: as in the forward.
 *   dbias         NULL (not wanted) or [2n] fp32 output; needs bias.
 *   dscale        NULL (not wanted) or fp32 per row, at dscale[r * dscale_stride]
 *                 (dscale_stride >= 1); needs scale.
 *   workspace     device memory of at least
 *                 swiglu_gateup_bias_scale_workspace_size(rows, n, dbias != NULL,
 *                 dscale != NULL) bytes, 16-byte aligned; may be NULL when that
 *                 size is 0. Its contents need no initialisation and are
 *                 scratch afterwards; calls that share a workspace must not run
 *                 concurrently.
 * With rows == 0, dbias (if given) is set to zero; with n == 0, ds (if given)
 * is set to zero; nothing else is launched for empty problems.
 * Errors: as swiglu_gateup_bwd; also SWIGLU_ERR_NULL_POINTER (dbias without
 * bias, dscale without scale), SWIGLU_ERR_BAD_STRIDE (scale or dscale stride
 * < 1), SWIGLU_ERR_WORKSPACE, and SWIGLU_ERR_ALIASING when an output (dx,
 * dbias, dscale, workspace) overlaps an input or another output.
 */
swiglu_status swiglu_gateup_bias_scale_bwd(const void* dy, int64_t dy_row_stride,
                                           void* x, int64_t x_row_stride,
                                           const void* bias, const float* scale,
                                           int64_t scale_stride,
                                           void* dx, int64_t dx_row_stride,
                                           float* dbias, float* dscale, int64_t dscale_stride,
                                           void* workspace, size_t workspace_bytes,
                                           int64_t rows, int64_t n,
                                           swiglu_dtype dtype, int in_place, hipStream_t stream);

/*
 * Allocation-free variant of swiglu_gateup_bias_scale_bwd, for callers that
 * cannot allocate device memory or pass a workspace: code recorded under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and bits as swiglu_gateup_bias_scale_bwd, without
 * workspace and workspace_bytes: the partial sums go to a static device array
 * of SWIGLU_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU
 * it runs on until the process ends (its address is looked up once per
 * device, on the first call there). The call allocates and frees nothing.
 *
 *   Limit: swiglu_gateup_bias_scale_workspace_size(rows, n, dbias != NULL,
 *   dscale != NULL) must not exceed SWIGLU_NOALLOC_SCRATCH_BYTES; larger
 *   problems return SWIGLU_ERR_SCRATCH_LIMIT before anything is launched.
 *   (8192 rows of n = 32768 with both sums need 48 MiB.)
 *   Concurrency: every call on one GPU shares that GPU's array, so calls on
 *   one GPU that may overlap in time (different streams, or different host
 *   threads without ordering) race and must not be issued. The array needs
 *   no clearing: every partial is written before it is read.
 *
 * Errors: those of swiglu_gateup_bias_scale_bwd except SWIGLU_ERR_WORKSPACE;
 * also SWIGLU_ERR_SCRATCH_LIMIT, and SWIGLU_ERR_HIP when the array's device
 * address cannot be obtained.
 */
#define SWIGLU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

swiglu_status swiglu_gateup_bias_scale_bwd_noalloc(const void* dy, int64_t dy_row_stride,
                                                   void* x, int64_t x_row_stride,
                                                   const void* bias, const float* scale,
                                                   int64_t scale_stride,
                                                   void* dx, int64_t dx_row_stride,
                                                   float* dbias, float* dscale,
                                                   int64_t dscale_stride,
                                                   int64_t rows, int64_t n,
                                                   swiglu_dtype dtype, int in_place,
                                                   hipStream_t stream);

/*
 * fc1 projection with the SwiGLU as its epilogue (Liger-Kernel Megatron
 * SwiGLU page, §Background: the packed [tokens, 2n] tensor is the output of
 * one fc1 projection; Liger-Kernel test/cute page, §MLP1 numerical reference:
 * fused MLP1-with-activation variants). With W = [Wg; Wu] of shape [2n, k] in
 * the Linear layout (row j holds output feature j),
 *     y = silu(A Wg^T) * (A Wu^T)            ([m, n])
 * is computed without writing the [m, 2n] product, which stays in fp32
 * registers (bf16 inputs, fp32 accumulation on the matrix cores, one
 * nearest-even rounding of y). On request the product itself is also
 * written, rounded to bf16, for a later backward.
 *
 *   a, lda        [m, k] activations (tokens), row stride lda (elements).
 *   w, ldw        [2n, k] weights: rows [0, n) gate, [n, 2n) up; stride ldw.
 *   y, ldy        [m, n] output, row stride ldy.
 *   x_out, ldx    NULL, or [m, 2n] output receiving A W^T (bf16), stride ldx.
 *   m, n, k       sizes: m >= 0; n a multiple of 64 in [0, 2^30]; k a
 *                 positive multiple of 64 (k may be 0 only when m or n is 0).
 *   dtype         must be SWIGLU_DTYPE_BF16.
 *   workspace     NULL, or swiglu_fc1_workspace_size() bytes of device memory,
 *                 owned by the caller, that are all zero on entry. With it,
 *                 a launch of at least 16 output tiles (256 x 128) per CU
 *                 ends on a pool. Its last quarter of tiles is taken by
 *                 workgroups as they start, through counters kept there, so
 *                 those tiles go to whichever XCD has room instead of a
 *                 fixed share each. The call leaves the workspace all zero
 *                 again once it completes, so one workspace serves every
 *                 call on one stream. Calls that use the same workspace must
 *                 not overlap in time (e.g. on two streams). With NULL, every
 *                 tile is its own workgroup. y and x_out are the same bits
 *                 either way.
 *   stream        HIP stream of the launch.
 * All pointers must be 16-byte aligned and all row strides multiples of 8;
 * lda and ldw (hence k) are at most 2^28 elements.
 *
 * Errors: SWIGLU_ERR_BAD_DTYPE (not bf16), SWIGLU_ERR_BAD_SHAPE (n or k not
 * multiples of 64, k == 0 with a non-empty output), SWIGLU_ERR_BAD_STRIDE
 * (strides below the widths or lda / ldw above 2^28, misaligned pointers,
 * workspace or strides),
 * SWIGLU_ERR_NULL_POINTER, SWIGLU_ERR_ALIASING (an output overlaps an input
 * or the other output, or the workspace overlaps any of them), SWIGLU_ERR_HIP.
 */
swiglu_status swiglu_fc1_fwd(const void* a, int64_t lda, const void* w, int64_t ldw,
                             void* y, int64_t ldy, void* x_out, int64_t ldx,
                             int64_t m, int64_t n, int64_t k,
                             swiglu_dtype dtype, void* workspace, hipStream_t stream);

/* Bytes of the workspace that swiglu_fc1_fwd takes (a constant). */
size_t swiglu_fc1_workspace_size(void);

/* Static, human-readable name of a status code (never NULL). */
const char* swiglu_status_string(swiglu_status status);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_GATEUP_H */
