// Fused gate-up SwiGLU forward and backward for AMD MI355X (gfx950), with
// the C ABI declared in include/swiglu_gateup.h.
//
// What is computed (Liger-Kernel Megatron SwiGLU page, §Background,
// §What's added, §Optional in_place): x is one packed [rows, 2n] fc1 output,
// gate g = columns [0, n), up u = columns [n, 2n), read through a column
// offset within the same row. Forward: y = silu(g) * u. Backward: recompute
// silu from x and write dgate = dy * u * sigma(g) * (1 + g (1 - sigma(g))) and
// dup = dy * silu(g), to a separate [rows, 2n] buffer or over x.
//
// Design. The op is elementwise and touches every byte once, so there is no
// reuse for LDS or MFMA to exploit; the kernels are HBM streams.
//  * Each lane owns ONE vector (16 bytes when alignment allows: 8 bf16 or 4
//    fp32 elements) of every stream: it loads the gate, up (and dy) vectors,
//    computes in fp32 registers and stores the result vectors. Consecutive
//    lanes own consecutive vectors, so each wave64 load or store covers 1 KiB
//    of contiguous memory.
//  * The grid is one-shot and 2D: blockIdx.y picks a row (or, for rows
//    narrower than a block, a group of rows), blockIdx.x a 256-vector column
//    tile. Row offsets are uniform per block and live in scalar registers; no
//    lane divides. Enough blocks are in flight that HBM stays saturated
//    (131072 blocks for 8192 x 32768 bf16).
//  * Loads and stores carry the nontemporal hint: nothing is re-read, and
//    keeping the stream out of the caches measured faster on large shapes.
//  * Arithmetic is kept short because at 16 bytes per lane the forward has
//    only ~29 VALU slots per element pair at 8 TB/s: bf16 uses one exp2 and
//    one reciprocal per element with no selects; fp32 (half the elements per
//    lane, same bytes) affords a compensated exponential and a series at the
//    root of silu' for its tighter tolerance. bf16 results are rounded once,
//    nearest-even, by the hardware convert.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "swiglu_gateup.h"
#include "host_logic.h"

#ifndef SWIGLU_NT_LOAD
#define SWIGLU_NT_LOAD 1        // nontemporal hint on loads
#endif
#ifndef SWIGLU_NT_STORE
#define SWIGLU_NT_STORE 1       // nontemporal hint on stores
#endif

namespace {

constexpr int kBlock = 256;                 // threads (4 wave64) and vectors per tile
constexpr uint32_t kMaxGridY = 65535;       // row groups per launch; more rows -> more launches

// ---------------------------------------------------------------------------
// Element access: VEC elements of T as one load/store of VEC*sizeof(T) bytes.
// bf16 is carried as its uint16_t bit pattern.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int BYTES> struct Raw;
template <> struct Raw<16> { typedef u32x4 type; };
template <> struct Raw<8> { typedef u32x2 type; };
template <> struct Raw<4> { typedef uint32_t type; };
template <> struct Raw<2> { typedef uint16_t type; };

template <typename R>
__device__ __forceinline__ R load_raw(const void* p) {
#if SWIGLU_NT_LOAD
    return __builtin_nontemporal_load(reinterpret_cast<const R*>(p));
#else
    return *reinterpret_cast<const R*>(p);
#endif
}

template <typename R>
__device__ __forceinline__ void store_raw(void* p, R v) {
#if SWIGLU_NT_STORE
    __builtin_nontemporal_store(v, reinterpret_cast<R*>(p));
#else
    *reinterpret_cast<R*>(p) = v;
#endif
}

template <typename T, int VEC>
struct Vec {
    static constexpr int kBytes = VEC * (int)sizeof(T);
    typedef typename Raw<kBytes>::type R;

    // Load VEC elements starting at p and widen them to fp32 (exact).
    static __device__ __forceinline__ void load(const T* p, float (&f)[VEC]) {
        R r = load_raw<R>(p);
        if constexpr (sizeof(T) == 4) {
            __builtin_memcpy(f, &r, sizeof(r));
        } else if constexpr (kBytes == 2) {
            f[0] = __uint_as_float((uint32_t)r << 16);
        } else {
            uint32_t w[kBytes / 4];
            __builtin_memcpy(w, &r, sizeof(r));
#pragma unroll
            for (int i = 0; i < kBytes / 4; ++i) {
                f[2 * i] = __uint_as_float(w[i] << 16);         // lower address: low half
                f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }

    // Narrow VEC fp32 values to T (bf16: one nearest-even rounding) and store.
    static __device__ __forceinline__ void store(T* p, const float (&f)[VEC]) {
        R r;
        if constexpr (sizeof(T) == 4) {
            __builtin_memcpy(&r, f, sizeof(r));
        } else if constexpr (kBytes == 2) {
            __bf16 h = (__bf16)f[0];
            r = __builtin_bit_cast(uint16_t, h);
        } else {
            uint32_t w[kBytes / 4];
#pragma unroll
            for (int i = 0; i < kBytes / 4; ++i) {
                f32x2 pr = {f[2 * i], f[2 * i + 1]};
                w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
            }
            __builtin_memcpy(&r, w, sizeof(r));
        }
        store_raw<R>(p, r);
    }
};

// ---------------------------------------------------------------------------
// Math (fp32). Constants are derived from the definitions:
//   log2(e) split into an fp32 head and tail;
//   g0 = -1 - W(1/e), the root of 1 + g + e^g (the minimiser of silu), split
//   into an fp32 head and tail; c = e^{g0} = -(1 + g0).
// ---------------------------------------------------------------------------
constexpr float kLog2eHi = 0x1.715476p+0f;
constexpr float kLog2eLo = 0x1.4ae0c0p-26f;
constexpr float kLn2 = 0x1.62e430p-1f;
constexpr float kG0Hi = -0x1.474974p+0f;
constexpr float kG0Lo = 0x1.bdf6fap-27f;
constexpr float kC = 0x1.1d25d0p-2f;        // e^{g0} = -(1 + g0)

// --- bf16 path: sigma with one exp2 and one reciprocal -----------------------
// With E = e^{-g} 2^-64 and r = 1 / (2^-64 + E):
//   sigma(g) = r 2^-64   and   1 - sigma(g) = e^{-g} sigma(g) = E r.
// The 2^-64 shift keeps E finite for g >= -131 and r a normal number, so
// the hardware exp2 and reciprocal (which do not produce subnormals) are
// never asked for one; the final multiply by 2^-64 rounds correctly into the
// subnormal range. Below g = -131.7, E overflows to inf and r is 0, which is
// sigma(g) there to fp32 precision; 1 - sigma = E r would then be inf * 0,
// so when it is wanted (WANT_OSIG) the exponent is clamped to 126 instead,
// giving r = 2^-126 and E r = 1. Relative error of sigma is a few 1e-6: far
// inside one bf16 step (2^-8).
template <bool WANT_OSIG>
__device__ __forceinline__ void sigmoid_fast(float g, float& sig, float& osig) {
    float a = __builtin_fmaf(-g, kLog2eHi, -64.0f);
    if constexpr (WANT_OSIG) a = __builtin_fminf(a, 126.0f);
    const float E = __builtin_amdgcn_exp2f(a);
    const float r = __builtin_amdgcn_rcpf(0x1p-64f + E);
    sig = r * 0x1p-64f;
    if constexpr (WANT_OSIG) osig = E * r;
}

// --- fp32 path: compensated exponential ---------------------------------------
// e^{-a} for a >= 0 (a = +inf gives 0, a NaN gives NaN). Written as
// 2^{-a log2 e}: the product is split so the exponent keeps ~48 bits, the
// hardware 2^x does the rest, and the tail of the exponent is applied as a
// first-order correction. The hardware 2^x does not return subnormal
// results, so arguments below -126 are lifted by 64 and scaled back by an
// exact multiply, which rounds correctly into the subnormal range.
__device__ __forceinline__ float exp_neg(float a) {
    a = __builtin_fminf(a, 200.0f);         // e^{-200} is 0 in fp32; keeps the
                                            // products below finite
    const float p = -a * kLog2eHi;
    float perr = __builtin_fmaf(-a, kLog2eHi, -p);      // exact product error
    perr = __builtin_fmaf(-a, kLog2eLo, perr);
    const bool tiny = p < -126.0f;
    float r = __builtin_amdgcn_exp2f(tiny ? p + 64.0f : p);
    r = __builtin_fmaf(r, perr * kLn2, r);
    return tiny ? r * 0x1p-64f : r;
}

// sigma(g) and 1 - sigma(g) without cancellation and without forming inf:
// with e = e^{-|g|} and d = 1/(1+e) = sigma(|g|), sigma(g) is d for g >= 0 and
// e*d otherwise, and 1 - sigma(g) = sigma(-g) is the other one.
__device__ __forceinline__ void sigmoid_accurate(float g, float& sig, float& osig) {
    const float e = exp_neg(__builtin_fabsf(g));
    const float d = __builtin_amdgcn_rcpf(1.0f + e);
    const float ed = e * d;
    const bool pos = g >= 0.0f;
    sig = pos ? d : ed;
    osig = pos ? ed : d;
}

// h(g) = 1 + g (1 - sigma(g)), the factor with silu'(g) = sigma(g) h(g).
// h has a simple root at g0 where the direct sum cancels. Since
// h(g) = (1 + g + e^g) sigma(-g) and, with t = g - g0,
// 1 + g + e^g = t + c (e^t - 1) (c = e^{g0}), the Taylor series of that
// bracket in t has no cancellation: t (1 + c) + c (t^2/2! + t^3/3! + ...).
// It is used for |t| < 1/4 (series truncated after t^7: relative error below
// 1e-9); the direct form elsewhere, where |h| > 0.24.
__device__ __forceinline__ float h_root_series(float g, float osig) {
    const float direct = __builtin_fmaf(g, osig, 1.0f);
    const float t = (g - kG0Hi) - kG0Lo;   // g - kG0Hi is exact near g0
    float q = kC * (1.0f / 5040.0f);
    q = __builtin_fmaf(q, t, kC * (1.0f / 720.0f));
    q = __builtin_fmaf(q, t, kC * (1.0f / 120.0f));
    q = __builtin_fmaf(q, t, kC * (1.0f / 24.0f));
    q = __builtin_fmaf(q, t, kC * (1.0f / 6.0f));
    q = __builtin_fmaf(q, t, kC * 0.5f);
    q = __builtin_fmaf(q, t, 1.0f + kC);
    const float series = (q * t) * osig;
    return __builtin_fabsf(t) < 0.25f ? series : direct;
}

// Per-dtype choice. bf16 needs 2 ulp of an 8-bit significand: the bracket
// 1 + g(1 - sigma) never comes closer to 0 than 0.0028 on the bf16 grid, so
// the direct sum (absolute error ~1e-7) is far inside that. fp32 needs 1e-5
// relative everywhere, including next to g0.
template <typename T, bool WANT_OSIG>
__device__ __forceinline__ void sigmoid_pair(float g, float& sig, float& osig) {
    if constexpr (sizeof(T) == 2) sigmoid_fast<WANT_OSIG>(g, sig, osig);
    else sigmoid_accurate(g, sig, osig);
}

template <typename T>
__device__ __forceinline__ float h_factor(float g, float osig) {
    if constexpr (sizeof(T) == 2) return __builtin_fmaf(g, osig, 1.0f);
    else return h_root_series(g, osig);
}

// ---------------------------------------------------------------------------
// Launch geometry. WIDE (n/VEC >= kBlock): block (x, y) owns vectors
// [x*kBlock, (x+1)*kBlock) of row y. Narrow: block y owns rpb whole rows;
// lane t takes row t / nv, vector t % nv, computed once in fp32 (exact: both
// operands are below 256 and the quotient is never within 1/512 of an
// integer).
// ---------------------------------------------------------------------------
struct Geom {
    int64_t rows;     // rows covered by this launch
    uint32_t nv;      // vectors per half row (n / VEC)
    uint32_t rpb;     // rows per block (1 when WIDE)
    float inv_nv;     // 1 / nv (narrow mode)
};

template <bool WIDE>
__device__ __forceinline__ bool locate(const Geom& G, int64_t& row, uint32_t& col) {
    if constexpr (WIDE) {
        row = blockIdx.y;
        col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
        return col < G.nv;
    } else {
        const uint32_t t = threadIdx.x;
        const uint32_t q = (uint32_t)(((float)t + 0.5f) * G.inv_nv);
        col = t - q * G.nv;
        row = (int64_t)blockIdx.y * G.rpb + q;
        return q < G.rpb && row < G.rows;
    }
}

// ---------------------------------------------------------------------------
// Kernels. The gate and up operands are two [rows, n] views with their own
// base pointers and row strides: the packed layout is the case up = x + n
// with both strides equal to x's, and the two-tensor layout passes two
// tensors. Row offsets are uniform per block, so the extra base costs no
// lane arithmetic.
// ---------------------------------------------------------------------------
template <typename T, int VEC, bool WIDE>
__global__ __launch_bounds__(kBlock) void swiglu_fwd_kernel(
    const T* __restrict__ gp, int64_t gs, const T* __restrict__ up, int64_t us,
    T* __restrict__ y, int64_t ys, Geom G) {
    int64_t row;
    uint32_t col;
    if (!locate<WIDE>(G, row, col)) return;
    const int64_t c = (int64_t)col * VEC;
    float g[VEC], u[VEC], out[VEC];
    Vec<T, VEC>::load(gp + row * gs + c, g);
    Vec<T, VEC>::load(up + row * us + c, u);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig;
        sigmoid_pair<T, false>(g[i], sig, osig);
        out[i] = (g[i] * sig) * u[i];
    }
    Vec<T, VEC>::store(y + row * ys + c, out);
}

// IN_PLACE: dgate over gate and dup over up (no restrict: the same addresses
// are read, then written by the same lane; no other lane touches them).
template <typename T, int VEC, bool WIDE, bool IN_PLACE>
__global__ __launch_bounds__(kBlock) void swiglu_bwd_kernel(
    const T* dyp, int64_t dys, T* gp, int64_t gs, T* up, int64_t us,
    T* dgp, int64_t dgs, T* dup, int64_t dus, Geom G) {
    if constexpr (IN_PLACE) {
        dgp = gp;
        dgs = gs;
        dup = up;
        dus = us;
    }
    int64_t row;
    uint32_t col;
    if (!locate<WIDE>(G, row, col)) return;
    const int64_t c = (int64_t)col * VEC;
    float g[VEC], u[VEC], d[VEC], dg[VEC], du[VEC];
    Vec<T, VEC>::load(gp + row * gs + c, g);
    Vec<T, VEC>::load(up + row * us + c, u);
    Vec<T, VEC>::load(dyp + row * dys + c, d);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig;
        sigmoid_pair<T, true>(g[i], sig, osig);
        const float h = h_factor<T>(g[i], osig);
        du[i] = d[i] * (g[i] * sig);
        dg[i] = ((d[i] * u[i]) * sig) * h;
    }
    Vec<T, VEC>::store(dgp + row * dgs + c, dg);
    Vec<T, VEC>::store(dup + row * dus + c, du);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
using swiglu_host::Operand;
using swiglu_host::Plan;
using swiglu_host::vec_bytes;
using swiglu_host::views_overlap;

swiglu_status check_shape(int64_t rows, int64_t n, swiglu_dtype dtype) {
    if (dtype != SWIGLU_DTYPE_F32 && dtype != SWIGLU_DTYPE_BF16) return SWIGLU_ERR_BAD_DTYPE;
    if (rows < 0 || n < 0) return SWIGLU_ERR_BAD_SHAPE;
    if (n > (int64_t)INT32_MAX) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

// One [rows, width] operand with the given row stride (elements).
swiglu_status check_operand(int64_t rows, int64_t stride, int64_t width, int64_t esz) {
    if (stride < width) return SWIGLU_ERR_BAD_STRIDE;
    // ((rows - 1) * stride + width) * esz must fit in int64.
    // (stride == 0 only when width == 0: the empty problem, nothing to bound.)
    const int64_t lim = INT64_MAX / esz - width;
    if (rows > 1 && stride > 0 && (rows - 1) > lim / stride) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

Plan make_plan(int64_t n, int vec) {
    return swiglu_host::make_plan(n, vec, (uint32_t)kBlock, kMaxGridY);
}

// Launch `kernel` over rows [0, rows) in chunks. The argument array holds, in
// order, (pointer, stride) pairs for each operand followed by the Geom; each
// chunk advances every pointer by r0 rows.
template <typename T, int NOPS>
swiglu_status launch_chunks(const void* kernel, const Plan& P, int64_t rows, const Operand* ops,
                            hipStream_t stream) {
    T* ptr[NOPS];
    int64_t stride[NOPS];
    Geom G;
    void* args[2 * NOPS + 1];
    for (int i = 0; i < NOPS; ++i) {
        stride[i] = ops[i].stride;
        args[2 * i] = &ptr[i];
        args[2 * i + 1] = &stride[i];
    }
    args[2 * NOPS] = &G;
    G.nv = P.nv;
    G.rpb = P.rpb;
    G.inv_nv = 1.0f / (float)P.nv;
    for (int64_t r0 = 0; r0 < rows; r0 += P.rows_per_launch) {
        const int64_t rc = rows - r0 < P.rows_per_launch ? rows - r0 : P.rows_per_launch;
        for (int i = 0; i < NOPS; ++i)
            ptr[i] = const_cast<T*>(static_cast<const T*>(ops[i].p)) + r0 * ops[i].stride;
        G.rows = rc;
        const uint32_t groups = (uint32_t)((rc + P.rpb - 1) / P.rpb);
        const hipError_t e =
            hipLaunchKernel(kernel, dim3(P.tiles, groups), dim3(kBlock), args, 0, stream);
        if (e != hipSuccess) return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

// ops: gate, up, y.
template <typename T, int VEC>
swiglu_status fwd_launch(const Operand* ops, int64_t rows, int64_t n, hipStream_t stream) {
    const Plan P = make_plan(n, VEC);
    const void* k = P.wide ? reinterpret_cast<const void*>(&swiglu_fwd_kernel<T, VEC, true>)
                           : reinterpret_cast<const void*>(&swiglu_fwd_kernel<T, VEC, false>);
    return launch_chunks<T, 3>(k, P, rows, ops, stream);
}

// ops: dy, gate, up, dgate, dup.
template <typename T, int VEC>
swiglu_status bwd_launch(const Operand* ops, int64_t rows, int64_t n, bool in_place,
                         hipStream_t stream) {
    const Plan P = make_plan(n, VEC);
    const void* k;
    if (P.wide)
        k = in_place ? reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, true, true>)
                     : reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, true, false>);
    else
        k = in_place ? reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, false, true>)
                     : reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, false, false>);
    return launch_chunks<T, 5>(k, P, rows, ops, stream);
}

// Validated forward on [rows, n] views: gate, up -> y.
swiglu_status run_fwd(Operand gate, Operand up, Operand y, int64_t rows, int64_t n,
                      swiglu_dtype dtype, hipStream_t stream) {
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    const Operand ops[3] = {gate, up, y};
    const int vb = vec_bytes((int)esz, ops, 3);
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return fwd_launch<uint16_t, 8>(ops, rows, n, stream);
            case 8: return fwd_launch<uint16_t, 4>(ops, rows, n, stream);
            case 4: return fwd_launch<uint16_t, 2>(ops, rows, n, stream);
            default: return fwd_launch<uint16_t, 1>(ops, rows, n, stream);
        }
    }
    switch (vb) {
        case 16: return fwd_launch<float, 4>(ops, rows, n, stream);
        case 8: return fwd_launch<float, 2>(ops, rows, n, stream);
        default: return fwd_launch<float, 1>(ops, rows, n, stream);
    }
}

// Validated backward on [rows, n] views: dy, gate, up -> dgate, dup.
swiglu_status run_bwd(Operand dy, Operand gate, Operand up, Operand dgate, Operand dup,
                      int64_t rows, int64_t n, swiglu_dtype dtype, bool in_place,
                      hipStream_t stream) {
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    const Operand ops[5] = {dy, gate, up, dgate, dup};
    const int vb = vec_bytes((int)esz, ops, 5);
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return bwd_launch<uint16_t, 8>(ops, rows, n, in_place, stream);
            case 8: return bwd_launch<uint16_t, 4>(ops, rows, n, in_place, stream);
            case 4: return bwd_launch<uint16_t, 2>(ops, rows, n, in_place, stream);
            default: return bwd_launch<uint16_t, 1>(ops, rows, n, in_place, stream);
        }
    }
    switch (vb) {
        case 16: return bwd_launch<float, 4>(ops, rows, n, in_place, stream);
        case 8: return bwd_launch<float, 2>(ops, rows, n, in_place, stream);
        default: return bwd_launch<float, 1>(ops, rows, n, in_place, stream);
    }
}

const void* offset(const void* p, int64_t elems, int64_t esz) {
    return p ? static_cast<const char*>(p) + elems * esz : nullptr;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) const char* swiglu_status_string(swiglu_status s) {
    switch (s) {
        case SWIGLU_OK: return "SWIGLU_OK";
        case SWIGLU_ERR_NULL_POINTER: return "SWIGLU_ERR_NULL_POINTER: a required pointer is NULL";
        case SWIGLU_ERR_BAD_SHAPE: return "SWIGLU_ERR_BAD_SHAPE: rows or n out of range";
        case SWIGLU_ERR_BAD_STRIDE: return "SWIGLU_ERR_BAD_STRIDE: a row stride is below the row width";
        case SWIGLU_ERR_BAD_DTYPE: return "SWIGLU_ERR_BAD_DTYPE: dtype must be F32 or BF16";
        case SWIGLU_ERR_ALIASING: return "SWIGLU_ERR_ALIASING: output overlaps an input";
        case SWIGLU_ERR_HIP: return "SWIGLU_ERR_HIP: HIP runtime or launch failure";
    }
    return "SWIGLU_ERR_UNKNOWN: not a swiglu_status value";
}

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_fwd(
    const void* x, int64_t x_row_stride, void* y, int64_t y_row_stride, int64_t rows, int64_t n,
    swiglu_dtype dtype, hipStream_t stream) {
    swiglu_status st = check_shape(rows, n, dtype);
    if (st != SWIGLU_OK) return st;
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    if ((st = check_operand(rows, x_row_stride, 2 * n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, y_row_stride, n, esz)) != SWIGLU_OK) return st;
    if (rows == 0 || n == 0) return SWIGLU_OK;
    if (!x || !y) return SWIGLU_ERR_NULL_POINTER;
    const Operand ox{x, x_row_stride}, oy{y, y_row_stride};
    if (views_overlap(ox, 2 * n, oy, n, rows, esz)) return SWIGLU_ERR_ALIASING;
    return run_fwd(ox, Operand{offset(x, n, esz), x_row_stride}, oy, rows, n, dtype, stream);
}

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_bwd(
    const void* dy, int64_t dy_row_stride, void* x, int64_t x_row_stride, void* dx,
    int64_t dx_row_stride, int64_t rows, int64_t n, swiglu_dtype dtype, int in_place,
    hipStream_t stream) {
    swiglu_status st = check_shape(rows, n, dtype);
    if (st != SWIGLU_OK) return st;
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    const bool ip = in_place != 0;
    if (ip) {
        if (dx != nullptr && dx != x) return SWIGLU_ERR_ALIASING;
        dx = x;
        dx_row_stride = x_row_stride;
    }
    if ((st = check_operand(rows, dy_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, x_row_stride, 2 * n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, dx_row_stride, 2 * n, esz)) != SWIGLU_OK) return st;
    if (rows == 0 || n == 0) return SWIGLU_OK;
    if (!dy || !x || !dx) return SWIGLU_ERR_NULL_POINTER;
    const Operand ody{dy, dy_row_stride}, ox{x, x_row_stride}, odx{dx, dx_row_stride};
    if (views_overlap(ody, n, ox, 2 * n, rows, esz)) return SWIGLU_ERR_ALIASING;
    if (!ip && (views_overlap(odx, 2 * n, ox, 2 * n, rows, esz) ||
                views_overlap(odx, 2 * n, ody, n, rows, esz)))
        return SWIGLU_ERR_ALIASING;
    return run_bwd(ody, ox, Operand{offset(x, n, esz), x_row_stride}, odx,
                   Operand{offset(dx, n, esz), dx_row_stride}, rows, n, dtype, ip, stream);
}

__attribute__((visibility("default"))) swiglu_status swiglu_silu_mul_fwd(
    const void* gate, int64_t gate_row_stride, const void* up, int64_t up_row_stride, void* y,
    int64_t y_row_stride, int64_t rows, int64_t n, swiglu_dtype dtype, hipStream_t stream) {
    swiglu_status st = check_shape(rows, n, dtype);
    if (st != SWIGLU_OK) return st;
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    if ((st = check_operand(rows, gate_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, up_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, y_row_stride, n, esz)) != SWIGLU_OK) return st;
    if (rows == 0 || n == 0) return SWIGLU_OK;
    if (!gate || !up || !y) return SWIGLU_ERR_NULL_POINTER;
    const Operand og{gate, gate_row_stride}, ou{up, up_row_stride}, oy{y, y_row_stride};
    if (views_overlap(oy, n, og, n, rows, esz) || views_overlap(oy, n, ou, n, rows, esz))
        return SWIGLU_ERR_ALIASING;
    return run_fwd(og, ou, oy, rows, n, dtype, stream);
}

__attribute__((visibility("default"))) swiglu_status swiglu_silu_mul_bwd(
    const void* dy, int64_t dy_row_stride, void* gate, int64_t gate_row_stride, void* up,
    int64_t up_row_stride, void* dgate, int64_t dgate_row_stride, void* dup,
    int64_t dup_row_stride, int64_t rows, int64_t n, swiglu_dtype dtype, int in_place,
    hipStream_t stream) {
    swiglu_status st = check_shape(rows, n, dtype);
    if (st != SWIGLU_OK) return st;
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    const bool ip = in_place != 0;
    if (ip) {
        if ((dgate != nullptr && dgate != gate) || (dup != nullptr && dup != up))
            return SWIGLU_ERR_ALIASING;
        dgate = gate;
        dgate_row_stride = gate_row_stride;
        dup = up;
        dup_row_stride = up_row_stride;
    }
    if ((st = check_operand(rows, dy_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, gate_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, up_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, dgate_row_stride, n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, dup_row_stride, n, esz)) != SWIGLU_OK) return st;
    if (rows == 0 || n == 0) return SWIGLU_OK;
    if (!dy || !gate || !up || !dgate || !dup) return SWIGLU_ERR_NULL_POINTER;
    const Operand ody{dy, dy_row_stride}, og{gate, gate_row_stride}, ou{up, up_row_stride},
        odg{dgate, dgate_row_stride}, odu{dup, dup_row_stride};
    if (ip) {
        // both inputs are written: they must not overlap each other or dy
        if (views_overlap(og, n, ou, n, rows, esz) || views_overlap(ody, n, og, n, rows, esz) ||
            views_overlap(ody, n, ou, n, rows, esz))
            return SWIGLU_ERR_ALIASING;
    } else {
        if (views_overlap(odg, n, odu, n, rows, esz)) return SWIGLU_ERR_ALIASING;
        for (const Operand& o : {odg, odu})
            if (views_overlap(o, n, ody, n, rows, esz) || views_overlap(o, n, og, n, rows, esz) ||
                views_overlap(o, n, ou, n, rows, esz))
                return SWIGLU_ERR_ALIASING;
    }
    return run_bwd(ody, og, ou, odg, odu, rows, n, dtype, ip, stream);
}

}  // extern "C"
