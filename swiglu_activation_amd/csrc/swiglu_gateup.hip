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
// relative everywhere, including next to g0.
template <typename T, bool WANT_OSIG>
__device__ __forceinline__ void sigmoid_pair(float g, float& sig, float& osig) {
    if constexpr (sizeof(T) == 2) sigmoid_fast<WANT_OSIG>(g, sig, osig);
    else sigmoid_accurate(g, sig, osig);
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
// Bias and per-token scale variants. With z = x + bias (bias: [2n], added to
// every row) and a per-row scale s (fp32):
//   forward   y = s * silu(z_gate) * z_up
//   backward  dz = the base backward at z with upstream gradient s * dy,
//             dx = dz, dbias = sum over rows of dz, ds = sum over columns of
//             dy * silu(z_gate) * z_up.
// bias and s are optional (NULL = 0 and 1).
// ---------------------------------------------------------------------------
#ifndef SWIGLU_BS_ROWS_PER_GROUP
#define SWIGLU_BS_ROWS_PER_GROUP 128   // rows reduced in registers per block (backward)
#endif
#ifndef SWIGLU_BS_UNROLL
#define SWIGLU_BS_UNROLL 4             // rows in flight per iteration (backward)
#endif
constexpr int kBsRows = SWIGLU_BS_ROWS_PER_GROUP;
constexpr int kBsUnroll = SWIGLU_BS_UNROLL;
static_assert(kBsRows % kBsUnroll == 0, "rows per group must be a multiple of the unroll");

// Exact sum of two fp32 values as head + tail (Knuth's two-sum).
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

template <typename T, int VEC, bool WIDE>
__global__ __launch_bounds__(kBlock) void swiglu_fwd_bs_kernel(
    const T* __restrict__ gp, int64_t gs, const T* __restrict__ up, int64_t us,
    T* __restrict__ y, int64_t ys, const T* __restrict__ bg, const T* __restrict__ bu,
    const float* __restrict__ sc, int64_t scs, Geom G) {
    int64_t row;
    uint32_t col;
    if (!locate<WIDE>(G, row, col)) return;
    const int64_t c = (int64_t)col * VEC;
    float g[VEC], u[VEC], out[VEC];
    Vec<T, VEC>::load(gp + row * gs + c, g);
    Vec<T, VEC>::load(up + row * us + c, u);
    if (bg != nullptr) {
        float b[VEC], d[VEC];
        Vec<T, VEC>::load(bg + c, b);
        Vec<T, VEC>::load(bu + c, d);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            g[i] += b[i];
            u[i] += d[i];
        }
    }
    const float s = sc != nullptr ? sc[row * scs] : 1.0f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig;
        sigmoid_pair<T, false>(g[i], sig, osig);
        out[i] = ((g[i] * sig) * u[i]) * s;
    }
    Vec<T, VEC>::store(y + row * ys + c, out);
}

// Partial sums of a backward over rows [row0 + y*R, row0 + (y+1)*R) for the
// column tile x. Writes dz for every element; part_db[group][k] gets this
// group's column sums (k in [0, 2n): gate columns, then up columns) and
// part_ds[row][x] this tile's share of each row's ds. Fixed summation order
// throughout: each lane adds its rows in order, each row's tile share is a
// fixed butterfly over the wave and then the four waves in order.
struct BsGeom {
    int64_t rows;       // rows in this launch
    int64_t n;          // half width (elements)
    int64_t group0;     // global index of this launch's first row group
    int64_t row0;       // global index of this launch's first row
    uint32_t nv;        // vectors per half row
    uint32_t tiles;     // column tiles per row (= gridDim.x)
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <typename T, int VEC, bool IN_PLACE>
__global__ __launch_bounds__(kBlock) void swiglu_bwd_bs_kernel(
    const T* dyp, int64_t dys, T* gp, int64_t gs, T* up, int64_t us, T* dgp, int64_t dgs,
    T* dup, int64_t dus, const T* bg, const T* bu, const float* sc, int64_t scs,
    float* part_db, float* part_ds, BsGeom G) {
    if constexpr (IN_PLACE) {
        dgp = gp;
        dgs = gs;
        dup = up;
        dus = us;
    }
    __shared__ float red[kBsUnroll][kBlock / 64];
    const uint32_t col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
    const bool active = col < G.nv;
    const int64_t c = (int64_t)col * VEC;
    const int64_t r_begin = (int64_t)blockIdx.y * kBsRows;
    const int64_t r_end = r_begin + kBsRows < G.rows ? r_begin + kBsRows : G.rows;
    const bool has_bias = bg != nullptr;
    float bgv[VEC], buv[VEC], acc_g[VEC], acc_u[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        bgv[i] = buv[i] = 0.0f;
        acc_g[i] = acc_u[i] = 0.0f;
    }
    if (has_bias && active) {
        Vec<T, VEC>::load(bg + c, bgv);
        Vec<T, VEC>::load(bu + c, buv);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t r = r_begin; r < r_end; r += kBsUnroll) {
        float g[kBsUnroll][VEC], u[kBsUnroll][VEC], d[kBsUnroll][VEC];
#pragma unroll
        for (int k = 0; k < kBsUnroll; ++k) {
            const int64_t row = r + k;
            if (active && row < r_end) {
                Vec<T, VEC>::load(gp + row * gs + c, g[k]);
                Vec<T, VEC>::load(up + row * us + c, u[k]);
                Vec<T, VEC>::load(dyp + row * dys + c, d[k]);
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i) g[k][i] = u[k][i] = d[k][i] = 0.0f;
            }
        }
        float pds[kBsUnroll];
#pragma unroll
        for (int k = 0; k < kBsUnroll; ++k) {
            const int64_t row = r + k;
            const bool live = active && row < r_end;
            const float s = (sc != nullptr && row < r_end) ? sc[row * scs] : 1.0f;
            float dg[VEC], du[VEC], p = 0.0f;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                float zg, zlo, zu = u[k][i] + buv[i];
                two_sum(g[k][i], bgv[i], zg, zlo);
                float sig, osig;
                sigmoid_pair<T, true>(zg, sig, osig);
                const float h = h_factor_lo<T>(zg, zlo, osig);
                const float silu = zg * sig;
                const float ds_ = d[k][i] * s;
                du[i] = ds_ * silu;
                dg[i] = ((ds_ * zu) * sig) * h;
                p = __builtin_fmaf(d[k][i] * silu, zu, p);
                if (live) {
                    acc_g[i] += dg[i];
                    acc_u[i] += du[i];
                }
            }
            pds[k] = live ? p : 0.0f;
            if (live) {
                Vec<T, VEC>::store(dgp + row * dgs + c, dg);
                Vec<T, VEC>::store(dup + row * dus + c, du);
            }
        }
        if (part_ds != nullptr) {
#pragma unroll
            for (int k = 0; k < kBsUnroll; ++k) {
                const float w = wave_sum(pds[k]);
                if (lane == 0) red[k][wave] = w;
            }
            __syncthreads();
            if (threadIdx.x < kBsUnroll) {
                const int k = threadIdx.x;
                const int64_t row = r + k;
                if (row < r_end) {
                    float t = red[k][0];
#pragma unroll
                    for (int wv = 1; wv < kBlock / 64; ++wv) t += red[k][wv];
                    part_ds[(G.row0 + row) * G.tiles + blockIdx.x] = t;
                }
            }
            __syncthreads();
        }
    }
    if (part_db != nullptr && active) {
        float* pg = part_db + (G.group0 + blockIdx.y) * (2 * G.n) + c;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            pg[i] = acc_g[i];
            pg[G.n + i] = acc_u[i];
        }
    }
}

// out[k * out_stride] = sum over j < count of part[j * jstride + k * kstride],
// j in order, for k < width.
__global__ __launch_bounds__(kBlock) void swiglu_sum_partials_kernel(
    const float* __restrict__ part, int64_t count, int64_t jstride, int64_t kstride,
    int64_t width, float* __restrict__ out, int64_t out_stride) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k >= width) return;
    const float* p = part + k * kstride;
    float acc = 0.0f;
    for (int64_t j = 0; j < count; ++j) acc += p[j * jstride];
    out[k * out_stride] = acc;
}

__global__ __launch_bounds__(kBlock) void swiglu_zero_kernel(float* p, int64_t count,
                                                             int64_t stride) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k < count) p[k * stride] = 0.0f;
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


// ---- bias / scale variants ---------------------------------------------------
struct BsArgs {
    const void* bias;        // [2n] of T or NULL
    const float* scale;      // [rows] with stride scale_stride, or NULL
    int64_t scale_stride;
};

template <typename T, int VEC>
swiglu_status fwd_bs_launch(const Operand* ops, const BsArgs& A, int64_t rows, int64_t n,
                            hipStream_t stream) {
    const Plan P = make_plan(n, VEC);
    const void* k = P.wide ? reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, true>)
                           : reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, false>);
    const T* g;
    const T* u;
    T* y;
    int64_t gs = ops[0].stride, us = ops[1].stride, ys = ops[2].stride, scs = A.scale_stride;
    const T* bg = static_cast<const T*>(A.bias);
    const T* bu = bg != nullptr ? bg + n : nullptr;
    const float* sc;
    Geom G;
    G.nv = P.nv;
    G.rpb = P.rpb;
    G.inv_nv = 1.0f / (float)P.nv;
    void* args[] = {&g, &gs, &u, &us, &y, &ys, &bg, &bu, &sc, &scs, &G};
    for (int64_t r0 = 0; r0 < rows; r0 += P.rows_per_launch) {
        const int64_t rc = rows - r0 < P.rows_per_launch ? rows - r0 : P.rows_per_launch;
        g = static_cast<const T*>(ops[0].p) + r0 * gs;
        u = static_cast<const T*>(ops[1].p) + r0 * us;
        y = const_cast<T*>(static_cast<const T*>(ops[2].p)) + r0 * ys;
        sc = A.scale != nullptr ? A.scale + r0 * scs : nullptr;
        G.rows = rc;
        const uint32_t groups = (uint32_t)((rc + P.rpb - 1) / P.rpb);
        if (hipLaunchKernel(k, dim3(P.tiles, groups), dim3(kBlock), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

// Workspace layout of the backward: [part_db: groups x 2n fp32][part_ds: rows x tiles fp32],
// each part starting on a 256-byte boundary. tiles is bounded by the
// single-element access width, so the size does not depend on alignment.
int64_t bs_groups(int64_t rows) { return (rows + kBsRows - 1) / kBsRows; }
int64_t bs_max_tiles(int64_t n) { return (n + kBlock - 1) / kBlock; }
int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

size_t bs_workspace_bytes(int64_t rows, int64_t n, bool want_db, bool want_ds) {
    int64_t b = 0;
    if (want_db) b += round256(bs_groups(rows) * 2 * n * 4);
    if (want_ds) b += round256(rows * bs_max_tiles(n) * 4);
    return (size_t)b;
}

swiglu_status zero_fill(float* p, int64_t count, int64_t stride, hipStream_t stream) {
    if (count <= 0) return SWIGLU_OK;
    void* args[] = {&p, &count, &stride};
    const uint32_t blocks = (uint32_t)((count + kBlock - 1) / kBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_zero_kernel), dim3(blocks),
                           dim3(kBlock), args, 0, stream) == hipSuccess
               ? SWIGLU_OK
               : SWIGLU_ERR_HIP;
}

swiglu_status sum_partials(const float* part, int64_t count, int64_t jstride, int64_t kstride,
                           int64_t width, float* out, int64_t out_stride, hipStream_t stream) {
    void* args[] = {&part, &count, &jstride, &kstride, &width, &out, &out_stride};
    const uint32_t blocks = (uint32_t)((width + kBlock - 1) / kBlock);
    return hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_sum_partials_kernel),
                           dim3(blocks), dim3(kBlock), args, 0, stream) == hipSuccess
               ? SWIGLU_OK
               : SWIGLU_ERR_HIP;
}

// ops: dy, gate, up, dgate, dup.
template <typename T, int VEC>
swiglu_status bwd_bs_launch(const Operand* ops, const BsArgs& A, int64_t rows, int64_t n,
                            bool in_place, float* dbias, float* dscale, int64_t dscale_stride,
                            void* workspace, hipStream_t stream) {
    const uint32_t nv = (uint32_t)(n / VEC);
    const uint32_t tiles = (nv + kBlock - 1) / kBlock;
    const int64_t groups = bs_groups(rows);
    float* part_db = nullptr;
    float* part_ds = nullptr;
    char* ws = static_cast<char*>(workspace);
    if (dbias != nullptr) {
        part_db = reinterpret_cast<float*>(ws);
        ws += round256(groups * 2 * n * 4);
    }
    if (dscale != nullptr) part_ds = reinterpret_cast<float*>(ws);

    const void* k = in_place ? reinterpret_cast<const void*>(&swiglu_bwd_bs_kernel<T, VEC, true>)
                             : reinterpret_cast<const void*>(&swiglu_bwd_bs_kernel<T, VEC, false>);
    const T *dyp, *bg = static_cast<const T*>(A.bias), *bu;
    T *gp, *upp, *dgp, *dup;
    int64_t dys = ops[0].stride, gs = ops[1].stride, us = ops[2].stride, dgs = ops[3].stride,
            dus = ops[4].stride, scs = A.scale_stride;
    bu = bg != nullptr ? bg + n : nullptr;
    const float* sc;
    BsGeom G;
    G.n = n;
    G.nv = nv;
    G.tiles = tiles;
    void* args[] = {&dyp, &dys, &gp, &gs, &upp, &us, &dgp, &dgs, &dup, &dus,
                    &bg, &bu, &sc, &scs, &part_db, &part_ds, &G};
    const int64_t rows_per_launch = (int64_t)kMaxGridY * kBsRows;
    for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
        const int64_t rc = rows - r0 < rows_per_launch ? rows - r0 : rows_per_launch;
        dyp = static_cast<const T*>(ops[0].p) + r0 * dys;
        gp = const_cast<T*>(static_cast<const T*>(ops[1].p)) + r0 * gs;
        upp = const_cast<T*>(static_cast<const T*>(ops[2].p)) + r0 * us;
        dgp = const_cast<T*>(static_cast<const T*>(ops[3].p)) + r0 * dgs;
        dup = const_cast<T*>(static_cast<const T*>(ops[4].p)) + r0 * dus;
        sc = A.scale != nullptr ? A.scale + r0 * scs : nullptr;
        G.rows = rc;
        G.row0 = r0;
        G.group0 = r0 / kBsRows;
        const uint32_t gy = (uint32_t)bs_groups(rc);
        if (hipLaunchKernel(k, dim3(tiles, gy), dim3(kBlock), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    swiglu_status st = SWIGLU_OK;
    if (dbias != nullptr)
        st = sum_partials(part_db, groups, 2 * n, 1, 2 * n, dbias, 1, stream);
    if (st == SWIGLU_OK && dscale != nullptr)
        st = sum_partials(part_ds, tiles, 1, tiles, rows, dscale, dscale_stride, stream);
    return st;
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
        case SWIGLU_ERR_WORKSPACE: return "SWIGLU_ERR_WORKSPACE: workspace missing, too small or misaligned";
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

__attribute__((visibility("default"))) size_t swiglu_gateup_bias_scale_workspace_size(
    int64_t rows, int64_t n, int want_dbias, int want_dscale) {
    if (rows <= 0 || n <= 0 || n > (int64_t)INT32_MAX) return 0;
    return bs_workspace_bytes(rows, n, want_dbias != 0, want_dscale != 0);
}

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_bias_scale_fwd(
    const void* x, int64_t x_row_stride, const void* bias, const float* scale,
    int64_t scale_stride, void* y, int64_t y_row_stride, int64_t rows, int64_t n,
    swiglu_dtype dtype, hipStream_t stream) {
    swiglu_status st = check_shape(rows, n, dtype);
    if (st != SWIGLU_OK) return st;
    const int64_t esz = dtype == SWIGLU_DTYPE_F32 ? 4 : 2;
    if ((st = check_operand(rows, x_row_stride, 2 * n, esz)) != SWIGLU_OK) return st;
    if ((st = check_operand(rows, y_row_stride, n, esz)) != SWIGLU_OK) return st;
    if (scale != nullptr && (st = check_operand(rows, scale_stride, 1, 4)) != SWIGLU_OK) return st;
    if (rows == 0 || n == 0) return SWIGLU_OK;
    if (!x || !y) return SWIGLU_ERR_NULL_POINTER;
    const Operand ox{x, x_row_stride}, oy{y, y_row_stride};
    if (views_overlap(ox, 2 * n, oy, n, rows, esz)) return SWIGLU_ERR_ALIASING;
    const swiglu_host::Span sy = swiglu_host::span_of(oy, rows, n, esz);
    if (bias != nullptr &&
        swiglu_host::spans_overlap(sy, swiglu_host::span_of(Operand{bias, 2 * n}, 1, 2 * n, esz)))
        return SWIGLU_ERR_ALIASING;
    if (scale != nullptr &&
        swiglu_host::spans_overlap(sy, swiglu_host::span_of(Operand{scale, scale_stride}, rows, 1, 4)))
        return SWIGLU_ERR_ALIASING;

    const BsArgs A{bias, scale, scale_stride};
    const Operand ops[5] = {ox, Operand{offset(x, n, esz), x_row_stride}, oy,
                            Operand{bias, 0}, Operand{offset(bias, n, esz), 0}};
    const int vb = vec_bytes((int)esz, ops, bias != nullptr ? 5 : 3);
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return fwd_bs_launch<uint16_t, 8>(ops, A, rows, n, stream);
            case 8: return fwd_bs_launch<uint16_t, 4>(ops, A, rows, n, stream);
            case 4: return fwd_bs_launch<uint16_t, 2>(ops, A, rows, n, stream);
            default: return fwd_bs_launch<uint16_t, 1>(ops, A, rows, n, stream);
        }
    }
    switch (vb) {
        case 16: return fwd_bs_launch<float, 4>(ops, A, rows, n, stream);
        case 8: return fwd_bs_launch<float, 2>(ops, A, rows, n, stream);
        default: return fwd_bs_launch<float, 1>(ops, A, rows, n, stream);
    }
}

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_bias_scale_bwd(
    const void* dy, int64_t dy_row_stride, void* x, int64_t x_row_stride, const void* bias,
    const float* scale, int64_t scale_stride, void* dx, int64_t dx_row_stride, float* dbias,
    float* dscale, int64_t dscale_stride, void* workspace, size_t workspace_bytes, int64_t rows,
    int64_t n, swiglu_dtype dtype, int in_place, hipStream_t stream) {
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
    if (scale != nullptr && (st = check_operand(rows, scale_stride, 1, 4)) != SWIGLU_OK) return st;
    if (dscale != nullptr && (st = check_operand(rows, dscale_stride, 1, 4)) != SWIGLU_OK) return st;
    if ((dbias != nullptr && bias == nullptr) || (dscale != nullptr && scale == nullptr))
        return SWIGLU_ERR_NULL_POINTER;
    if (rows == 0 || n == 0) {
        // Sums over nothing: dbias is 0 when there are no rows, each ds is 0
        // when rows are empty of columns.
        if (rows == 0 && n > 0 && dbias != nullptr) return zero_fill(dbias, 2 * n, 1, stream);
        if (n == 0 && rows > 0 && dscale != nullptr)
            return zero_fill(dscale, rows, dscale_stride, stream);
        return SWIGLU_OK;
    }
    if (!dy || !x || !dx) return SWIGLU_ERR_NULL_POINTER;
    const size_t need = bs_workspace_bytes(rows, n, dbias != nullptr, dscale != nullptr);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || (uintptr_t)workspace % 16))
        return SWIGLU_ERR_WORKSPACE;

    const Operand ody{dy, dy_row_stride}, ox{x, x_row_stride}, odx{dx, dx_row_stride};
    if (views_overlap(ody, n, ox, 2 * n, rows, esz)) return SWIGLU_ERR_ALIASING;
    if (!ip && (views_overlap(odx, 2 * n, ox, 2 * n, rows, esz) ||
                views_overlap(odx, 2 * n, ody, n, rows, esz)))
        return SWIGLU_ERR_ALIASING;
    // Every other pair: outputs (dx, dbias, dscale, workspace) against
    // everything else, by memory span.
    using swiglu_host::Span;
    using swiglu_host::span_of;
    using swiglu_host::spans_overlap;
    Span ins[4];
    int nin = 0;
    ins[nin++] = span_of(ody, rows, n, esz);
    if (!ip) ins[nin++] = span_of(ox, rows, 2 * n, esz);
    if (bias != nullptr) ins[nin++] = span_of(Operand{bias, 2 * n}, 1, 2 * n, esz);
    if (scale != nullptr) ins[nin++] = span_of(Operand{scale, scale_stride}, rows, 1, 4);
    Span outs[4];
    int nout = 0;
    outs[nout++] = span_of(odx, rows, 2 * n, esz);
    if (dbias != nullptr) outs[nout++] = span_of(Operand{dbias, 2 * n}, 1, 2 * n, 4);
    if (dscale != nullptr) outs[nout++] = span_of(Operand{dscale, dscale_stride}, rows, 1, 4);
    if (need > 0) outs[nout++] = Span{(uintptr_t)workspace, (uintptr_t)workspace + need};
    for (int i = 0; i < nout; ++i) {
        for (int j = (i == 0 ? 2 - (ip ? 1 : 0) : 0); j < nin; ++j)   // dx vs dy/x: checked above
            if (spans_overlap(outs[i], ins[j])) return SWIGLU_ERR_ALIASING;
        for (int j = i + 1; j < nout; ++j)
            if (spans_overlap(outs[i], outs[j])) return SWIGLU_ERR_ALIASING;
    }

    const BsArgs A{bias, scale, scale_stride};
    const Operand ops[7] = {ody, ox, Operand{offset(x, n, esz), x_row_stride}, odx,
                            Operand{offset(dx, n, esz), dx_row_stride}, Operand{bias, 0},
                            Operand{offset(bias, n, esz), 0}};
    const int vb = vec_bytes((int)esz, ops, bias != nullptr ? 7 : 5);
#define SWIGLU_BWD_BS(T, V)                                                                  \
    bwd_bs_launch<T, V>(ops, A, rows, n, ip, dbias, dscale, dscale_stride, workspace, stream)
    if (dtype == SWIGLU_DTYPE_BF16) {
        switch (vb) {
            case 16: return SWIGLU_BWD_BS(uint16_t, 8);
            case 8: return SWIGLU_BWD_BS(uint16_t, 4);
            case 4: return SWIGLU_BWD_BS(uint16_t, 2);
            default: return SWIGLU_BWD_BS(uint16_t, 1);
        }
    }
    switch (vb) {
        case 16: return SWIGLU_BWD_BS(float, 4);
        case 8: return SWIGLU_BWD_BS(float, 2);
        default: return SWIGLU_BWD_BS(float, 1);
    }
#undef SWIGLU_BWD_BS
}

}  // extern "C"
