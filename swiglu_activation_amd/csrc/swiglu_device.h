// Device-side building blocks shared by the SwiGLU kernels (gfx950): vector
// access of bf16 / fp32 rows, the sigmoid and silu' arithmetic, the launch
// geometry, and the host-side argument checks common to every entry point.
// Included by swiglu_gateup.hip and swiglu_bias_scale.hip.
#ifndef SWIGLU_DEVICE_H
#define SWIGLU_DEVICE_H

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

namespace swiglu_impl {


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
    // CACHED: plain load for data that other rows re-read (the bias).
    template <bool CACHED = false>
    static __device__ __forceinline__ void load(const T* p, float (&f)[VEC]) {
        R r;
        if constexpr (CACHED) r = *reinterpret_cast<const R*>(p);
        else r = load_raw<R>(p);
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
// results, so for arguments below -126 the exponent is lifted by 64 (exact)
// and the result is returned as e^{-a} 2^64 with `tiny` set: the caller
// scales it back by an exact multiply wherever that rounds best.
__device__ __forceinline__ float exp_neg_scaled(float a, bool& tiny) {
    a = __builtin_fminf(a, 200.0f);         // e^{-200} is 0 in fp32; keeps the
                                            // products below finite
    const float p = -a * kLog2eHi;
    float perr = __builtin_fmaf(-a, kLog2eHi, -p);      // exact product error
    perr = __builtin_fmaf(-a, kLog2eLo, perr);
    tiny = p < -126.0f;
    const float r = __builtin_amdgcn_exp2f(tiny ? p + 64.0f : p);
    return __builtin_fmaf(r, perr * kLn2, r);
}

// sigma(g) and 1 - sigma(g) without cancellation and without forming inf:
// with e = e^{-|g|} and d = 1/(1+e) = sigma(|g|), sigma(g) is d for g >= 0 and
// e*d otherwise, and 1 - sigma(g) = sigma(-g) is the other one.
// sigma(g) comes back times 1/scl: for g below about -87.3, where e^g is
// under the normal range, sigma is kept as sigma 2^64 (a normal number with
// all 24 bits) and scl = 2^-64, so that each output formed from it is
// scaled back by one final multiply -- exact when the output is normal, a
// single rounding when it is subnormal. Elsewhere scl = 1.
__device__ __forceinline__ void sigmoid_accurate(float g, float& sig, float& osig, float& scl) {
    bool tiny;
    const float e = exp_neg_scaled(__builtin_fabsf(g), tiny);   // e^{-|g|} (x 2^64 if tiny)
    const float d = __builtin_amdgcn_rcpf(1.0f + (tiny ? 0.0f : e));
    const float ed = e * d;
    const bool pos = g >= 0.0f;
    sig = pos ? d : ed;
    osig = pos ? (tiny ? ed * 0x1p-64f : ed) : d;
    scl = !pos && tiny ? 0x1p-64f : 1.0f;
}

// h(g) = 1 + g (1 - sigma(g)), the factor with silu'(g) = sigma(g) h(g).
// h has a simple root at g0 where the direct sum cancels. Since
// h(g) = (1 + g + e^g) sigma(-g) and, with t = g - g0,
// 1 + g + e^g = t + c (e^t - 1) (c = e^{g0}), the Taylor series of that
// bracket in t has no cancellation: t (1 + c) + c (t^2/2! + t^3/3! + ...).
// It is used for |t| < 1/4 (series truncated after t^7: relative error below
// 1e-9); the direct form elsewhere, where |h| > 0.24.
// With HAS_LO the argument is the unevaluated sum g + glo (glo well below one
// ulp of g): only the root series needs the low part, as t = g - g0 is then
// the cancellation-free difference of an exact head and two small tails.
template <bool HAS_LO>
__device__ __forceinline__ float h_root_series(float g, float glo, float osig) {
    const float direct = __builtin_fmaf(g, osig, 1.0f);
    float t = g - kG0Hi;                   // exact near g0
    if constexpr (HAS_LO) t += glo;
    t -= kG0Lo;
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
// relative everywhere, including next to g0 and where sigma(g) is below the
// normal range. Every output that sigma enters is multiplied by scl last
// (1 for bf16, where the multiply folds away; see sigmoid_accurate).
template <typename T, bool WANT_OSIG>
__device__ __forceinline__ void sigmoid_pair(float g, float& sig, float& osig, float& scl) {
    if constexpr (sizeof(T) == 2) {
        sigmoid_fast<WANT_OSIG>(g, sig, osig);
        scl = 1.0f;
    } else {
        sigmoid_accurate(g, sig, osig, scl);
    }
}

template <typename T>
__device__ __forceinline__ float h_factor(float g, float osig) {
    if constexpr (sizeof(T) == 2) return __builtin_fmaf(g, osig, 1.0f);
    else return h_root_series<false>(g, 0.0f, osig);
}

// h at the unevaluated sum z + zlo (a biased gate formed in fp32).
template <typename T>
__device__ __forceinline__ float h_factor_lo(float z, float zlo, float osig) {
    if constexpr (sizeof(T) == 2) return __builtin_fmaf(z, osig, 1.0f);
    else return h_root_series<true>(z, zlo, osig);
}

// ---------------------------------------------------------------------------
// Launch geometry (the mapping is described at locate() below).
// ---------------------------------------------------------------------------
struct Geom {
    int64_t rows;     // rows covered by this launch
    uint32_t nv;      // vectors per half row (n / VEC)
    double inv_nv;    // 1 / nv (narrow mode)
};

// The (row, vector) a lane owns. WIDE: block (x, y) owns vectors
// [256 x, 256 x + 256) of row y. Narrow: lane L = 256 blockIdx.x + t of the
// flat launch owns row L / nv, vector L % nv. The quotient is taken as
// floor((L + 1/2) * fp64(1/nv)): for L < 2^31 and nv < 256 the product is
// within 2^-21 of (L + 1/2) / nv, whose distance to the nearest integer is at
// least 1/(2 nv) > 2^-9, so the floor is exact.
template <bool WIDE>
__device__ __forceinline__ bool locate(const Geom& G, int64_t& row, uint32_t& col) {
    if constexpr (WIDE) {
        row = blockIdx.y;
        col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
        return col < G.nv;
    } else {
        const uint32_t L = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
        const uint32_t q = (uint32_t)(((double)L + 0.5) * G.inv_nv);
        col = L - q * G.nv;
        row = q;
        return (int64_t)q < G.rows;
    }
}

// ---------------------------------------------------------------------------
// Host-side checks shared by every entry point
// ---------------------------------------------------------------------------
using swiglu_host::Operand;
using swiglu_host::Plan;
using swiglu_host::vec_bytes;
using swiglu_host::views_overlap;

inline swiglu_status check_shape(int64_t rows, int64_t n, swiglu_dtype dtype) {
    if (dtype != SWIGLU_DTYPE_F32 && dtype != SWIGLU_DTYPE_BF16) return SWIGLU_ERR_BAD_DTYPE;
    if (rows < 0 || n < 0) return SWIGLU_ERR_BAD_SHAPE;
    if (n > (int64_t)INT32_MAX) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

// One [rows, width] operand with the given row stride (elements).
inline swiglu_status check_operand(int64_t rows, int64_t stride, int64_t width, int64_t esz) {
    if (stride < width) return SWIGLU_ERR_BAD_STRIDE;
    // ((rows - 1) * stride + width) * esz must fit in int64.
    // (stride == 0 only when width == 0: the empty problem, nothing to bound.)
    const int64_t lim = INT64_MAX / esz - width;
    if (rows > 1 && stride > 0 && (rows - 1) > lim / stride) return SWIGLU_ERR_BAD_SHAPE;
    return SWIGLU_OK;
}

inline Plan make_plan(int64_t n, int vec) {
    return swiglu_host::make_plan(n, vec, (uint32_t)kBlock, kMaxGridY);
}

inline const void* offset(const void* p, int64_t elems, int64_t esz) {
    return p ? static_cast<const char*>(p) + elems * esz : nullptr;
}

}  // namespace swiglu_impl

#endif  // SWIGLU_DEVICE_H
