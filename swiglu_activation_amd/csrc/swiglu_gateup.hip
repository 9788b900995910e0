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
// Design: the op is elementwise and streams every byte exactly once, so it is
// bound by HBM bandwidth, not by MFMA or LDS (there is no reuse to stage).
// Each lane owns 16-byte vectors (8 bf16 or 4 fp32 elements) and keeps
// UNROLL of them in flight per stream before touching any result; the
// (row, vector) space is flattened so narrow rows leave no idle lanes; the
// grid is a fixed multiple of the CU count and strides over that space.
// All arithmetic is fp32 in registers; bf16 results are rounded once,
// nearest-even, by the hardware convert.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "swiglu_gateup.h"

#ifndef SWIGLU_BLOCK
#define SWIGLU_BLOCK 256        // threads per workgroup (4 wave64)
#endif
#ifndef SWIGLU_UNROLL
#define SWIGLU_UNROLL 4         // 16-byte vectors in flight per lane and stream
#endif
#ifndef SWIGLU_BLOCKS_PER_CU
#define SWIGLU_BLOCKS_PER_CU 8  // grid cap = CUs * this
#endif
#ifndef SWIGLU_NT_LOAD
#define SWIGLU_NT_LOAD 0        // nontemporal hint on loads
#endif
#ifndef SWIGLU_NT_STORE
#define SWIGLU_NT_STORE 0       // nontemporal hint on stores
#endif
#ifndef SWIGLU_ROOT_SERIES_BF16
#define SWIGLU_ROOT_SERIES_BF16 1   // also use the root series for bf16
#endif

namespace {

constexpr int kBlock = SWIGLU_BLOCK;
constexpr int kUnroll = SWIGLU_UNROLL;

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

    // Load VEC elements starting at p and widen them to fp32.
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

// e^{-a} for a >= 0 (a = +inf gives 0, a NaN gives NaN). Written as
// 2^{-a log2 e}: the product is split so the exponent keeps ~48 bits, the
// hardware 2^x (v_exp_f32) does the rest, and the tail of the exponent is
// applied as a first-order correction. v_exp_f32 does not return subnormal
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
__device__ __forceinline__ void sigmoid_pair(float g, float& sig, float& osig) {
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
template <bool ROOT_SERIES>
__device__ __forceinline__ float h_factor(float g, float osig) {
    const float direct = __builtin_fmaf(g, osig, 1.0f);
    if constexpr (!ROOT_SERIES) {
        return direct;
    } else {
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
}

template <typename T>
constexpr bool root_series() {
    return sizeof(T) == 4 || SWIGLU_ROOT_SERIES_BF16;
}

// ---------------------------------------------------------------------------
// Index walk over the flattened (row, vector) space. Slot k of a lane starts
// at flat index blockIdx.x*kBlock*kUnroll + k*kBlock + threadIdx.x and
// advances by the grid's span S = dq*nv + dr each iteration; row and column
// are carried incrementally so the loop needs no division.
// ---------------------------------------------------------------------------
struct Walk {
    int64_t rows;
    uint32_t nv;     // vectors per half row (n / VEC)
    uint32_t dq;     // S / nv
    uint32_t dr;     // S % nv
};

struct Slot {
    int64_t row;
    uint32_t col;
};

__device__ __forceinline__ void slot_init(Slot& s, uint32_t idx, const Walk& w) {
    const uint32_t q = idx / w.nv;
    s.row = q;
    s.col = idx - q * w.nv;
}

__device__ __forceinline__ void slot_step(Slot& s, const Walk& w) {
    s.row += w.dq;
    s.col += w.dr;
    if (s.col >= w.nv) {
        s.col -= w.nv;
        s.row += 1;
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__device__ __forceinline__ void fwd_one(const T* __restrict__ x, int64_t xs, T* __restrict__ y,
                                        int64_t ys, int64_t n, const Slot& s,
                                        float (&g)[VEC], float (&u)[VEC]) {
    (void)x; (void)xs; (void)n;
    float out[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig;
        sigmoid_pair(g[i], sig, osig);
        out[i] = (g[i] * sig) * u[i];
    }
    Vec<T, VEC>::store(y + s.row * ys + (int64_t)s.col * VEC, out);
}

template <typename T, int VEC>
__global__ __launch_bounds__(kBlock) void swiglu_fwd_kernel(
    const T* __restrict__ x, int64_t xs, T* __restrict__ y, int64_t ys, int64_t n, Walk w) {
    Slot s[kUnroll];
    const uint32_t base = blockIdx.x * (uint32_t)(kBlock * kUnroll) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) slot_init(s[k], base + k * kBlock, w);

    // Full iterations: the last slot has the largest flat index, so if it is
    // in range all are.
    while (s[kUnroll - 1].row < w.rows) {
        float g[kUnroll][VEC], u[kUnroll][VEC];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const T* xr = x + s[k].row * xs + (int64_t)s[k].col * VEC;
            Vec<T, VEC>::load(xr, g[k]);
            Vec<T, VEC>::load(xr + n, u[k]);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            fwd_one<T, VEC>(x, xs, y, ys, n, s[k], g[k], u[k]);
            slot_step(s[k], w);
        }
    }
    // Last, partial iteration.
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        if (s[k].row < w.rows) {
            float g[VEC], u[VEC];
            const T* xr = x + s[k].row * xs + (int64_t)s[k].col * VEC;
            Vec<T, VEC>::load(xr, g);
            Vec<T, VEC>::load(xr + n, u);
            fwd_one<T, VEC>(x, xs, y, ys, n, s[k], g, u);
        }
    }
}

// One vector of the backward. Reads g, u, dy; writes dgate at dxr and dup at
// dxr + n. In place, dxr is the same address the gate was read from; every
// element is read and written by this one lane only, reads first.
template <typename T, int VEC>
__device__ __forceinline__ void bwd_one(T* dxr, int64_t n, const float (&g)[VEC],
                                        const float (&u)[VEC], const float (&dy)[VEC]) {
    float dg[VEC], du[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig;
        sigmoid_pair(g[i], sig, osig);
        const float h = h_factor<root_series<T>()>(g[i], osig);
        du[i] = dy[i] * (g[i] * sig);
        dg[i] = ((dy[i] * u[i]) * sig) * h;
    }
    Vec<T, VEC>::store(dxr, dg);
    Vec<T, VEC>::store(dxr + n, du);
}

// IN_PLACE: dx == x (no restrict: the same addresses are read then written).
template <typename T, int VEC, bool IN_PLACE>
__global__ __launch_bounds__(kBlock) void swiglu_bwd_kernel(
    const T* dy, int64_t dys, T* x, int64_t xs, T* dx, int64_t dxs, int64_t n, Walk w) {
    if constexpr (IN_PLACE) { dx = x; dxs = xs; }
    Slot s[kUnroll];
    const uint32_t base = blockIdx.x * (uint32_t)(kBlock * kUnroll) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) slot_init(s[k], base + k * kBlock, w);

    while (s[kUnroll - 1].row < w.rows) {
        float g[kUnroll][VEC], u[kUnroll][VEC], d[kUnroll][VEC];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t c = (int64_t)s[k].col * VEC;
            const T* xr = x + s[k].row * xs + c;
            Vec<T, VEC>::load(xr, g[k]);
            Vec<T, VEC>::load(xr + n, u[k]);
            Vec<T, VEC>::load(dy + s[k].row * dys + c, d[k]);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t c = (int64_t)s[k].col * VEC;
            bwd_one<T, VEC>(dx + s[k].row * dxs + c, n, g[k], u[k], d[k]);
            slot_step(s[k], w);
        }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
        if (s[k].row < w.rows) {
            float g[VEC], u[VEC], d[VEC];
            const int64_t c = (int64_t)s[k].col * VEC;
            const T* xr = x + s[k].row * xs + c;
            Vec<T, VEC>::load(xr, g);
            Vec<T, VEC>::load(xr + n, u);
            Vec<T, VEC>::load(dy + s[k].row * dys + c, d);
            bwd_one<T, VEC>(dx + s[k].row * dxs + c, n, g, u, d);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];   // 0 = not yet queried; racing writers store the same value

hipError_t cu_count(int* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices && g_cu_count[dev] > 0) {
        *out = g_cu_count[dev];
        return hipSuccess;
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus <= 0) cus = 1;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev] = cus;
    *out = cus;
    return hipSuccess;
}

struct Span {
    uintptr_t lo, hi;   // [lo, hi) in bytes
};

Span span_of(const void* p, int64_t rows, int64_t stride, int64_t width, int64_t esz) {
    const uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)(((rows - 1) * stride + width) * esz)};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Largest per-lane access (16, 8, 4 or 2 bytes; at least one element) that
// every base pointer, the up-half offset and every row stride are aligned to.
int vec_bytes(int esz, int64_t n, const uintptr_t* ptrs, int nptr, const int64_t* strides,
              int nstr) {
    int b = 16;
    for (; b > esz; b >>= 1) {
        bool ok = ((n * esz) % b) == 0;
        for (int i = 0; i < nptr; ++i) ok = ok && (ptrs[i] % (uintptr_t)b) == 0;
        for (int i = 0; i < nstr; ++i) ok = ok && ((strides[i] * esz) % b) == 0;
        if (ok) break;
    }
    return b;
}

// Checks shared by both directions. n is the half width; each (ptr, stride,
// width) triple describes one [rows, width] operand.
swiglu_status check_shape(int64_t rows, int64_t n, swiglu_dtype dtype) {
    if (dtype != SWIGLU_DTYPE_F32 && dtype != SWIGLU_DTYPE_BF16) return SWIGLU_ERR_BAD_DTYPE;
    if (rows < 0 || n < 0) return SWIGLU_ERR_BAD_SHAPE;
    if (n > (int64_t)INT32_MAX) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

swiglu_status check_operand(int64_t rows, int64_t stride, int64_t width, int64_t esz) {
    if (stride < width) return SWIGLU_ERR_BAD_STRIDE;
    // ((rows - 1) * stride + width) * esz must fit in int64.
    // (stride == 0 only when width == 0: the empty problem, nothing to bound.)
    const int64_t lim = INT64_MAX / esz - width;
    if (rows > 1 && stride > 0 && (rows - 1) > lim / stride) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

struct Launch {
    uint32_t blocks;
    Walk walk;
};

hipError_t plan(int64_t rows, int64_t n, int vec, Launch* L) {
    int cus = 0;
    hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    const uint64_t nv = (uint64_t)(n / vec);
    const uint64_t total = (uint64_t)rows * nv;
    const uint64_t per_block = (uint64_t)kBlock * kUnroll;
    uint64_t blocks = (total + per_block - 1) / per_block;
    const uint64_t cap = (uint64_t)cus * SWIGLU_BLOCKS_PER_CU;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const uint64_t S = blocks * per_block;
    L->blocks = (uint32_t)blocks;
    L->walk.rows = rows;
    L->walk.nv = (uint32_t)nv;
    L->walk.dq = (uint32_t)(S / nv);
    L->walk.dr = (uint32_t)(S % nv);
    return hipSuccess;
}

swiglu_status launch(const void* kernel, const Launch& L, void** args, hipStream_t stream) {
    hipError_t e = hipLaunchKernel(kernel, dim3(L.blocks), dim3(kBlock), args, 0, stream);
    return e == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_HIP;
}

template <typename T, int VEC>
swiglu_status fwd_launch(const void* x, int64_t xs, void* y, int64_t ys, int64_t rows, int64_t n,
                         hipStream_t stream) {
    Launch L;
    if (plan(rows, n, VEC, &L) != hipSuccess) return SWIGLU_ERR_HIP;
    const T* xp = static_cast<const T*>(x);
    T* yp = static_cast<T*>(y);
    void* args[] = {&xp, &xs, &yp, &ys, &n, &L.walk};
    return launch(reinterpret_cast<const void*>(&swiglu_fwd_kernel<T, VEC>), L, args, stream);
}

template <typename T, int VEC>
swiglu_status bwd_launch(const void* dy, int64_t dys, void* x, int64_t xs, void* dx, int64_t dxs,
                         int64_t rows, int64_t n, bool in_place, hipStream_t stream) {
    Launch L;
    if (plan(rows, n, VEC, &L) != hipSuccess) return SWIGLU_ERR_HIP;
    const T* dyp = static_cast<const T*>(dy);
    T* xp = static_cast<T*>(x);
    T* dxp = static_cast<T*>(dx);
    void* args[] = {&dyp, &dys, &xp, &xs, &dxp, &dxs, &n, &L.walk};
    const void* k = in_place ? reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, true>)
                             : reinterpret_cast<const void*>(&swiglu_bwd_kernel<T, VEC, false>);
    return launch(k, L, args, stream);
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
    if (overlaps(span_of(x, rows, x_row_stride, 2 * n, esz), span_of(y, rows, y_row_stride, n, esz)))
        return SWIGLU_ERR_ALIASING;

    const uintptr_t ptrs[] = {(uintptr_t)x, (uintptr_t)y};
    const int64_t strides[] = {x_row_stride, y_row_stride};
    const int vb = vec_bytes((int)esz, n, ptrs, 2, strides, 2);
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return fwd_launch<uint16_t, 8>(x, x_row_stride, y, y_row_stride, rows, n, stream);
            case 8: return fwd_launch<uint16_t, 4>(x, x_row_stride, y, y_row_stride, rows, n, stream);
            case 4: return fwd_launch<uint16_t, 2>(x, x_row_stride, y, y_row_stride, rows, n, stream);
            default: return fwd_launch<uint16_t, 1>(x, x_row_stride, y, y_row_stride, rows, n, stream);
        }
    }
    switch (vb) {
        case 16: return fwd_launch<float, 4>(x, x_row_stride, y, y_row_stride, rows, n, stream);
        case 8: return fwd_launch<float, 2>(x, x_row_stride, y, y_row_stride, rows, n, stream);
        default: return fwd_launch<float, 1>(x, x_row_stride, y, y_row_stride, rows, n, stream);
    }
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
    const Span sdy = span_of(dy, rows, dy_row_stride, n, esz);
    const Span sx = span_of(x, rows, x_row_stride, 2 * n, esz);
    if (ip) {
        if (overlaps(sdy, sx)) return SWIGLU_ERR_ALIASING;
    } else {
        const Span sdx = span_of(dx, rows, dx_row_stride, 2 * n, esz);
        if (overlaps(sdx, sx) || overlaps(sdx, sdy)) return SWIGLU_ERR_ALIASING;
    }

    const uintptr_t ptrs[] = {(uintptr_t)dy, (uintptr_t)x, (uintptr_t)dx};
    const int64_t strides[] = {dy_row_stride, x_row_stride, dx_row_stride};
    const int vb = vec_bytes((int)esz, n, ptrs, 3, strides, 3);
#define SWIGLU_BWD(T, V) \
    bwd_launch<T, V>(dy, dy_row_stride, x, x_row_stride, dx, dx_row_stride, rows, n, ip, stream)
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return SWIGLU_BWD(uint16_t, 8);
            case 8: return SWIGLU_BWD(uint16_t, 4);
            case 4: return SWIGLU_BWD(uint16_t, 2);
            default: return SWIGLU_BWD(uint16_t, 1);
        }
    }
    switch (vb) {
        case 16: return SWIGLU_BWD(float, 4);
        case 8: return SWIGLU_BWD(float, 2);
        default: return SWIGLU_BWD(float, 1);
    }
#undef SWIGLU_BWD
}

}  // extern "C"
