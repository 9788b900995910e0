// fc1 projection with the SwiGLU as its epilogue, for AMD MI355X (gfx950):
//     y = silu(A Wg^T) * (A Wu^T),   W = [Wg; Wu] in the Linear layout [2n, k]
// (Liger-Kernel Megatron SwiGLU page, §Background: the packed [tokens, 2n]
// tensor is one fc1 projection's output; the Liger-Kernel test/cute page's
// §MLP1 numerical reference describes fused MLP1-with-activation variants).
// The [tokens, 2n] product is kept in registers and only y (and, on request,
// the product itself for a later backward) is written.
//
// Design (bf16 in, fp32 accumulate, MFMA 32x32x16):
//  * Both operands are k-contiguous, so every MFMA fragment is one 16-byte
//    vector per lane. The roles are swapped relative to y: the MFMA's row
//    operand is a weight row (an output feature) and its column operand a
//    token, so each lane ends up holding four consecutive features of one
//    token and writes y with 8-byte stores.
//  * A workgroup of 4 waves computes 128 features x 128 tokens of y; each
//    wave 64 x 64, i.e. 2 x 2 MFMA tiles for the gate and 2 x 2 for the up
//    projection (128 fp32 accumulators per lane).
//  * k is walked in 64-wide tiles through a double-buffered LDS stage
//    (A: 128 x 64, W: 256 x 64 bf16, rows padded by 16 bytes); the next
//    tile's global loads are in flight while the current one feeds the
//    MFMAs, and one barrier per tile separates the stages.
//  * Rows past m (tokens) or n (features) load zeros and store nothing.
#include "swiglu_device.h"

namespace {

using namespace swiglu_impl;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kFcThreads = 256;            // 4 waves
constexpr int kFcTileF = 128;              // features per workgroup
constexpr int kFcTileT = 128;              // tokens per workgroup
constexpr int kFcTileK = 64;               // k per stage
constexpr int kFcPitch = kFcTileK + 8;     // LDS row pitch in bf16 (16-byte pad)
constexpr int kFcRowsA = kFcTileT;         // token rows per stage
constexpr int kFcRowsW = 2 * kFcTileF;     // gate rows, then up rows
constexpr int kFcStage = (kFcRowsA + kFcRowsW) * kFcPitch;   // bf16 per stage
// 16-byte vectors per thread per stage
constexpr int kFcVecA = kFcRowsA * (kFcTileK / 8) / kFcThreads;   // 4
constexpr int kFcVecW = kFcRowsW * (kFcTileK / 8) / kFcThreads;   // 8
static_assert(kFcVecA * kFcThreads == kFcRowsA * kFcTileK / 8, "A tile split");
static_assert(kFcVecW * kFcThreads == kFcRowsW * kFcTileK / 8, "W tile split");

struct Fc1Args {
    const uint16_t* a;   // [m, k] tokens, row stride lda
    const uint16_t* w;   // [2n, k] weights, row stride ldw
    uint16_t* y;         // [m, n], row stride ldy
    uint16_t* x;         // NULL or [m, 2n], row stride ldx
    int64_t lda, ldw, ldy, ldx;
    int64_t m, n, k;
};

// Global -> registers for one stage. Thread t loads, for vector v, row
// (v * 256 + t) / 8 and 16-byte column (t % 8) of the A and W tiles.
struct Stage {
    u32x4 a[kFcVecA];
    u32x4 w[kFcVecW];
};

__device__ __forceinline__ void load_stage(const Fc1Args& P, int64_t t0, int64_t f0, int64_t k0,
                                           Stage& s) {
    const int t = threadIdx.x;
    const int cv = t % 8;
#pragma unroll
    for (int v = 0; v < kFcVecA; ++v) {
        const int r = (v * kFcThreads + t) / 8;
        const int64_t tok = t0 + r;
        if (tok < P.m)
            s.a[v] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(P.a + tok * P.lda + k0 + cv * 8));
        else
            s.a[v] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int v = 0; v < kFcVecW; ++v) {
        const int r = (v * kFcThreads + t) / 8;       // 0..255: gate rows then up rows
        const int64_t f = f0 + (r % kFcTileF);
        const int64_t wrow = (r < kFcTileF ? 0 : P.n) + f;
        if (f < P.n)
            s.w[v] = *reinterpret_cast<const u32x4*>(P.w + wrow * P.ldw + k0 + cv * 8);
        else
            s.w[v] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ void store_stage(uint16_t* lds, const Stage& s) {
    const int t = threadIdx.x;
    const int cv = t % 8;
    uint16_t* la = lds;
    uint16_t* lw = lds + kFcRowsA * kFcPitch;
#pragma unroll
    for (int v = 0; v < kFcVecA; ++v) {
        const int r = (v * kFcThreads + t) / 8;
        *reinterpret_cast<u32x4*>(la + r * kFcPitch + cv * 8) = s.a[v];
    }
#pragma unroll
    for (int v = 0; v < kFcVecW; ++v) {
        const int r = (v * kFcThreads + t) / 8;
        *reinterpret_cast<u32x4*>(lw + r * kFcPitch + cv * 8) = s.w[v];
    }
}

__device__ __forceinline__ bf16x8 frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__global__ __launch_bounds__(kFcThreads) void swiglu_fc1_kernel(Fc1Args P) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kFcStage];   // 2 stages, 108 KiB
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wf = (wave & 1) * 64;                // wave's feature offset in the tile
    const int wt = (wave >> 1) * 64;               // wave's token offset in the tile
    const int64_t f0 = (int64_t)blockIdx.x * kFcTileF;
    const int64_t t0 = (int64_t)blockIdx.y * kFcTileT;

    f32x16 acc_g[2][2], acc_u[2][2];               // [feature tile][token tile]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc_g[i][j] = f32x16{};
            acc_u[i][j] = f32x16{};
        }

    const int kt_count = (int)(P.k / kFcTileK);
    Stage st;
    load_stage(P, t0, f0, 0, st);
    store_stage(lds, st);
    __syncthreads();

    const int frow = lane % 32;                    // fragment row within a 32-tile
    const int fk = 8 * (lane / 32);                // fragment k offset within a 16-step
    for (int kt = 0; kt < kt_count; ++kt) {
        if (kt + 1 < kt_count) load_stage(P, t0, f0, (int64_t)(kt + 1) * kFcTileK, st);
        const uint16_t* la = lds + (kt & 1) * kFcStage;
        const uint16_t* lw = la + kFcRowsA * kFcPitch;
#pragma unroll
        for (int ks = 0; ks < kFcTileK; ks += 16) {
            bf16x8 fa[2], fg[2], fu[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fa[j] = frag(la + (wt + 32 * j + frow) * kFcPitch + ks + fk);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fg[i] = frag(lw + (wf + 32 * i + frow) * kFcPitch + ks + fk);
                fu[i] = frag(lw + (kFcTileF + wf + 32 * i + frow) * kFcPitch + ks + fk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc_g[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fg[i], fa[j],
                                                                        acc_g[i][j], 0, 0, 0);
                    acc_u[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fu[i], fa[j],
                                                                        acc_u[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < kt_count) store_stage(lds + ((kt + 1) & 1) * kFcStage, st);
        __syncthreads();
    }

    // Epilogue. Register v of a 32x32 tile holds feature
    // (v % 4) + 8 (v / 4) + 4 (lane / 32) and token lane % 32, so each group
    // of four registers is four consecutive features of one token.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t tok = t0 + wt + 32 * j + lane % 32;
            if (tok >= P.m) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t f = f0 + wf + 32 * i + 8 * q + 4 * (lane / 32);
                if (f >= P.n) continue;                 // n is a multiple of 4
                float yv[4], gv[4], uv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    gv[r] = acc_g[i][j][4 * q + r];
                    uv[r] = acc_u[i][j][4 * q + r];
                    float sig, osig;
                    sigmoid_pair<uint16_t, false>(gv[r], sig, osig);
                    yv[r] = (gv[r] * sig) * uv[r];
                }
                Vec<uint16_t, 4>::store(P.y + tok * P.ldy + f, yv);
                if (P.x != nullptr) {
                    Vec<uint16_t, 4>::store(P.x + tok * P.ldx + f, gv);
                    Vec<uint16_t, 4>::store(P.x + tok * P.ldx + P.n + f, uv);
                }
            }
        }
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) swiglu_status swiglu_fc1_fwd(
    const void* a, int64_t lda, const void* w, int64_t ldw, void* y, int64_t ldy, void* x_out,
    int64_t ldx, int64_t m, int64_t n, int64_t k, swiglu_dtype dtype, hipStream_t stream) {
    if (dtype != SWIGLU_DTYPE_BF16) return SWIGLU_ERR_BAD_DTYPE;
    if (m < 0 || n < 0 || k < 0 || n > (int64_t)INT32_MAX || k > (int64_t)INT32_MAX)
        return SWIGLU_ERR_BAD_SHAPE;
    if (n % 64 != 0 || k % kFcTileK != 0) return SWIGLU_ERR_BAD_SHAPE;
    swiglu_status st;
    if ((st = check_operand(m, lda, k, 2)) != SWIGLU_OK) return st;
    if ((st = check_operand(2 * n, ldw, k, 2)) != SWIGLU_OK) return st;
    if ((st = check_operand(m, ldy, n, 2)) != SWIGLU_OK) return st;
    if (x_out != nullptr && (st = check_operand(m, ldx, 2 * n, 2)) != SWIGLU_OK) return st;
    if (m == 0 || n == 0) return SWIGLU_OK;
    if (k == 0) return SWIGLU_ERR_BAD_SHAPE;       // an empty sum: y would be silu(0)*0 = 0
    if (!a || !w || !y) return SWIGLU_ERR_NULL_POINTER;
    // 16-byte rows for the vector loads and stores
    const uintptr_t ptr_or = (uintptr_t)a | (uintptr_t)w | (uintptr_t)y | (uintptr_t)x_out;
    if (ptr_or % 16 != 0 || lda % 8 || ldw % 8 || ldy % 8 || (x_out && ldx % 8))
        return SWIGLU_ERR_BAD_STRIDE;
    const Operand oa{a, lda}, ow{w, ldw}, oy{y, ldy}, ox{x_out, ldx};
    if (views_overlap(oy, n, oa, k, m, 2)) return SWIGLU_ERR_ALIASING;
    if (swiglu_host::spans_overlap(swiglu_host::span_of(oy, m, n, 2),
                                   swiglu_host::span_of(ow, 2 * n, k, 2)))
        return SWIGLU_ERR_ALIASING;
    if (x_out != nullptr) {
        if (views_overlap(ox, 2 * n, oa, k, m, 2) || views_overlap(ox, 2 * n, oy, n, m, 2) ||
            swiglu_host::spans_overlap(swiglu_host::span_of(ox, m, 2 * n, 2),
                                       swiglu_host::span_of(ow, 2 * n, k, 2)))
            return SWIGLU_ERR_ALIASING;
    }

    Fc1Args P;
    P.a = static_cast<const uint16_t*>(a);
    P.w = static_cast<const uint16_t*>(w);
    P.y = static_cast<uint16_t*>(y);
    P.x = static_cast<uint16_t*>(x_out);
    P.lda = lda;
    P.ldw = ldw;
    P.ldy = ldy;
    P.ldx = ldx;
    P.n = n;
    P.k = k;
    const int64_t f_tiles = (n + kFcTileF - 1) / kFcTileF;
    const int64_t rows_per_launch = (int64_t)kMaxGridY * kFcTileT;
    void* args[] = {&P};
    for (int64_t r0 = 0; r0 < m; r0 += rows_per_launch) {
        const int64_t mc = m - r0 < rows_per_launch ? m - r0 : rows_per_launch;
        P.a = static_cast<const uint16_t*>(a) + r0 * lda;
        P.y = static_cast<uint16_t*>(y) + r0 * ldy;
        P.x = x_out ? static_cast<uint16_t*>(x_out) + r0 * ldx : nullptr;
        P.m = mc;
        const uint32_t t_tiles = (uint32_t)((mc + kFcTileT - 1) / kFcTileT);
        if (hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_fc1_kernel),
                            dim3((uint32_t)f_tiles, t_tiles), dim3(kFcThreads), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

}  // extern "C"
