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
//  * A workgroup of 4 waves computes 256 tokens x 128 features of y; each
//    wave 128 tokens x 64 features, i.e. 4 x 2 MFMA tiles for the gate and
//    4 x 2 for the up projection (256 fp32 accumulators per lane, in the
//    accumulation registers). Per 16-wide k step a wave reads 8 fragments
//    from LDS for 16 MFMAs: 1/64 byte of LDS traffic per flop.
//  * k is walked in 64-wide tiles through a double-buffered LDS stage
//    (A: 256 x 64, W: 256 x 64 bf16, rows padded by 16 bytes, 144 KiB);
//    the next tile's global loads are in flight while the current one feeds
//    the MFMAs, the next k step's fragments are read while the current
//    step's MFMAs run, and one barrier per tile separates the stages.
//  * Rows past m (tokens) or n (features) load zeros and store nothing.
#include "swiglu_device.h"

namespace {

using namespace swiglu_impl;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef SWIGLU_FC_WAVE_T
#define SWIGLU_FC_WAVE_T 128    // tokens per wave (multiple of 32)
#endif
#ifndef SWIGLU_FC_WAVE_F
#define SWIGLU_FC_WAVE_F 64     // output features per wave (multiple of 32)
#endif
#ifndef SWIGLU_FC_WAVES_T
#define SWIGLU_FC_WAVES_T 2     // waves along tokens
#endif
#ifndef SWIGLU_FC_WAVES_F
#define SWIGLU_FC_WAVES_F 2     // waves along features
#endif
#ifndef SWIGLU_FC_TILE_K
#define SWIGLU_FC_TILE_K 64     // k per LDS stage
#endif
#ifndef SWIGLU_FC_GROUP
#define SWIGLU_FC_GROUP 16      // token tiles that share a weight tile in the launch order
#endif
#ifndef SWIGLU_FC_SPLIT_STORE
#define SWIGLU_FC_SPLIT_STORE 0 // write the next stage to LDS between k steps
#endif
#ifndef SWIGLU_FC_FRAG_DB
#define SWIGLU_FC_FRAG_DB 1     // read the next k step's fragments during the MFMAs
#endif

constexpr int kFcMT = SWIGLU_FC_WAVE_T / 32;         // 32x32 tiles per wave along tokens
constexpr int kFcMF = SWIGLU_FC_WAVE_F / 32;         // ... along features (each: gate + up)
constexpr int kFcThreads = 64 * SWIGLU_FC_WAVES_T * SWIGLU_FC_WAVES_F;
constexpr int kFcTileT = SWIGLU_FC_WAVE_T * SWIGLU_FC_WAVES_T;   // tokens per workgroup
constexpr int kFcTileF = SWIGLU_FC_WAVE_F * SWIGLU_FC_WAVES_F;   // features per workgroup
constexpr int kFcTileK = SWIGLU_FC_TILE_K;
constexpr int kFcPitch = kFcTileK + 8;               // LDS row pitch in bf16 (16-byte pad)
constexpr int kFcRowsA = kFcTileT;                   // token rows per stage
constexpr int kFcRowsW = 2 * kFcTileF;               // gate rows, then up rows
constexpr int kFcStage = (kFcRowsA + kFcRowsW) * kFcPitch;   // bf16 per stage
constexpr int kFcVecRow = kFcTileK / 8;              // 16-byte vectors per row
constexpr int kFcVecA = kFcRowsA * kFcVecRow / kFcThreads;
constexpr int kFcVecW = kFcRowsW * kFcVecRow / kFcThreads;
static_assert(kFcVecA * kFcThreads == kFcRowsA * kFcVecRow, "A tile split");
static_assert(kFcVecW * kFcThreads == kFcRowsW * kFcVecRow, "W tile split");
static_assert(2 * kFcStage * 2 <= 160 * 1024, "two stages must fit in LDS");

struct Fc1Args {
    const uint16_t* a;   // [m, k] tokens, row stride lda
    const uint16_t* w;   // [2n, k] weights, row stride ldw
    uint16_t* y;         // [m, n], row stride ldy
    uint16_t* x;         // NULL or [m, 2n], row stride ldx
    int64_t lda, ldw, ldy, ldx;
    int64_t m, n, k;
};

// Global -> registers for one stage. Thread t loads, for vector v, row
// (v * threads + t) / kFcVecRow and 16-byte column t % kFcVecRow of the A
// tile and of the W tile (gate rows, then up rows).
struct Stage {
    u32x4 a[kFcVecA];
    u32x4 w[kFcVecW];
};

__device__ __forceinline__ void load_stage(const Fc1Args& P, int64_t t0, int64_t f0, int64_t k0,
                                           Stage& s) {
    const int t = threadIdx.x;
    const int cv = t % kFcVecRow;
#pragma unroll
    for (int v = 0; v < kFcVecA; ++v) {
        const int r = (v * kFcThreads + t) / kFcVecRow;
        const int64_t tok = t0 + r;
        if (tok < P.m)
            s.a[v] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(P.a + tok * P.lda + k0 + cv * 8));
        else
            s.a[v] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int v = 0; v < kFcVecW; ++v) {
        const int r = (v * kFcThreads + t) / kFcVecRow;
        const int64_t f = f0 + (r % kFcTileF);
        const int64_t wrow = (r < kFcTileF ? 0 : P.n) + f;
        if (f < P.n)
            s.w[v] = *reinterpret_cast<const u32x4*>(P.w + wrow * P.ldw + k0 + cv * 8);
        else
            s.w[v] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Writes part `part` of `parts` of the staged vectors to LDS.
template <int PART, int PARTS>
__device__ __forceinline__ void store_stage_part(uint16_t* lds, const Stage& s) {
    const int t = threadIdx.x;
    const int cv = t % kFcVecRow;
    uint16_t* la = lds;
    uint16_t* lw = lds + kFcRowsA * kFcPitch;
    constexpr int nA = kFcVecA / PARTS, nW = kFcVecW / PARTS;
    static_assert(nA * PARTS == kFcVecA && nW * PARTS == kFcVecW, "even split");
#pragma unroll
    for (int v = PART * nA; v < (PART + 1) * nA; ++v) {
        const int r = (v * kFcThreads + t) / kFcVecRow;
        *reinterpret_cast<u32x4*>(la + r * kFcPitch + cv * 8) = s.a[v];
    }
#pragma unroll
    for (int v = PART * nW; v < (PART + 1) * nW; ++v) {
        const int r = (v * kFcThreads + t) / kFcVecRow;
        *reinterpret_cast<u32x4*>(lw + r * kFcPitch + cv * 8) = s.w[v];
    }
}

__device__ __forceinline__ void store_stage(uint16_t* lds, const Stage& s) {
    store_stage_part<0, 1>(lds, s);
}

// Store part s of the next stage after k step s (all parts by the last step).
template <int S>
__device__ __forceinline__ void store_after_step(uint16_t* lds, const Stage& st) {
    constexpr int steps = kFcTileK / 16;
    store_stage_part<S, steps>(lds, st);
}

__device__ __forceinline__ bf16x8 frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// The fragments one wave needs for one 16-wide k step.
struct Frags {
    bf16x8 a[kFcMT], g[kFcMF], u[kFcMF];
};

__device__ __forceinline__ void load_frags(const uint16_t* la, const uint16_t* lw, int wt, int wf,
                                           int frow, int kk, Frags& F) {
#pragma unroll
    for (int j = 0; j < kFcMT; ++j) F.a[j] = frag(la + (wt + 32 * j + frow) * kFcPitch + kk);
#pragma unroll
    for (int i = 0; i < kFcMF; ++i) {
        F.g[i] = frag(lw + (wf + 32 * i + frow) * kFcPitch + kk);
        F.u[i] = frag(lw + (kFcTileF + wf + 32 * i + frow) * kFcPitch + kk);
    }
}

// Launch order of the output tiles: consecutive workgroups take GROUP token
// tiles of one feature column of tiles before moving to the next feature
// tile, so each weight tile is fetched from HBM once per GROUP token tiles
// and the workgroups in flight share a working set that stays in the
// Infinity Cache.
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t f_tiles, uint32_t t_tiles,
                                        uint32_t& ft, uint32_t& tt) {
    const uint32_t per_group = SWIGLU_FC_GROUP * f_tiles;
    const uint32_t g = b / per_group, in = b % per_group;
    const uint32_t first_t = g * SWIGLU_FC_GROUP;
    const uint32_t gs = t_tiles - first_t < SWIGLU_FC_GROUP ? t_tiles - first_t : SWIGLU_FC_GROUP;
    tt = first_t + in % gs;
    ft = in / gs;
}

__global__ __launch_bounds__(kFcThreads) void swiglu_fc1_kernel(Fc1Args P, uint32_t f_tiles,
                                                                uint32_t t_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kFcStage];   // 2 stages
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wf = (wave % SWIGLU_FC_WAVES_F) * SWIGLU_FC_WAVE_F;   // wave's feature offset
    const int wt = (wave / SWIGLU_FC_WAVES_F) * SWIGLU_FC_WAVE_T;   // wave's token offset
    uint32_t ft, tt;
    tile_of(blockIdx.x, f_tiles, t_tiles, ft, tt);
    const int64_t f0 = (int64_t)ft * kFcTileF;
    const int64_t t0 = (int64_t)tt * kFcTileT;

    f32x16 acc_g[kFcMF][kFcMT], acc_u[kFcMF][kFcMT];   // [feature tile][token tile]
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j) {
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
#if SWIGLU_FC_FRAG_DB
        // Fragments for step s + 1 are read while the MFMAs of step s run.
        Frags F[2];
        load_frags(la, lw, wt, wf, frow, fk, F[0]);
#endif
#pragma unroll
        for (int s = 0; s < kFcTileK / 16; ++s) {
#if SWIGLU_FC_FRAG_DB
            if (s + 1 < kFcTileK / 16)
                load_frags(la, lw, wt, wf, frow, 16 * (s + 1) + fk, F[(s + 1) & 1]);
            const Frags& C = F[s & 1];
#else
            Frags C;
            load_frags(la, lw, wt, wf, frow, 16 * s + fk, C);
#endif
#pragma unroll
            for (int i = 0; i < kFcMF; ++i)
#pragma unroll
                for (int j = 0; j < kFcMT; ++j) {
                    acc_g[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.g[i], C.a[j],
                                                                        acc_g[i][j], 0, 0, 0);
                    acc_u[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.u[i], C.a[j],
                                                                        acc_u[i][j], 0, 0, 0);
                }
#if SWIGLU_FC_SPLIT_STORE
            if (kt + 1 < kt_count) {
                uint16_t* nxt = lds + ((kt + 1) & 1) * kFcStage;
                if (s == 0) store_after_step<0>(nxt, st);
                if constexpr (kFcTileK / 16 > 1) if (s == 1) store_after_step<1>(nxt, st);
                if constexpr (kFcTileK / 16 > 2) if (s == 2) store_after_step<2>(nxt, st);
                if constexpr (kFcTileK / 16 > 3) if (s == 3) store_after_step<3>(nxt, st);
            }
#endif
        }
#if !SWIGLU_FC_SPLIT_STORE
        if (kt + 1 < kt_count) store_stage(lds + ((kt + 1) & 1) * kFcStage, st);
#endif
        __syncthreads();
    }

    // Epilogue. Register v of a 32x32 tile holds feature
    // (v % 4) + 8 (v / 4) + 4 (lane / 32) and token lane % 32, so each group
    // of four registers is four consecutive features of one token.
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j) {
            const int64_t tok = t0 + wt + 32 * j + lane % 32;
            if (tok >= P.m) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t f = f0 + wf + 32 * i + 8 * q + 4 * (lane / 32);
                if (f >= P.n) continue;                 // n is a multiple of 64
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
    // 2n weight rows and k fit in 31 bits, so the feature-tile count fits
    // one launch dimension with room to spare
    if (m < 0 || n < 0 || k < 0 || n > ((int64_t)1 << 30) || k > (int64_t)INT32_MAX)
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
    const uint32_t f_tiles = (uint32_t)((n + kFcTileF - 1) / kFcTileF);
    // One launch covers at most 2^24 - 1 workgroups (its work-item count must
    // stay below 2^32) and 65535 token tiles.
    const int64_t max_wg = ((int64_t)1 << 24) - 1;
    int64_t tiles_per_launch = max_wg / f_tiles;
    if (tiles_per_launch > kMaxGridY) tiles_per_launch = kMaxGridY;
    const int64_t rows_per_launch = tiles_per_launch * kFcTileT;
    uint32_t t_tiles = 0;
    void* args[] = {&P, const_cast<uint32_t*>(&f_tiles), &t_tiles};
    for (int64_t r0 = 0; r0 < m; r0 += rows_per_launch) {
        const int64_t mc = m - r0 < rows_per_launch ? m - r0 : rows_per_launch;
        P.a = static_cast<const uint16_t*>(a) + r0 * lda;
        P.y = static_cast<uint16_t*>(y) + r0 * ldy;
        P.x = x_out ? static_cast<uint16_t*>(x_out) + r0 * ldx : nullptr;
        P.m = mc;
        t_tiles = (uint32_t)((mc + kFcTileT - 1) / kFcTileT);
        if (hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_fc1_kernel),
                            dim3(f_tiles * t_tiles), dim3(kFcThreads), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

}  // extern "C"
