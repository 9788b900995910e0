// Bias and per-token-scale variants of the fused gate-up SwiGLU for AMD
// MI355X (gfx950), with their C ABI (include/swiglu_gateup.h).
//
// What is computed (Liger-Kernel Megatron SwiGLU page, §Scope and §Known
// issues name a bias on the fc1 output and a per-token-scale-aware version
// for MoE routed experts, without a formula): z = x + bias, y = s * silu(z_g)
// * z_u; the backward writes dx and the fp32 sums dbias (over rows) and
// ds (over columns). The elementwise part streams like the base kernels; the
// sums go through fixed-order partials in a caller-provided workspace, so
// results are bitwise deterministic.
#include "swiglu_device.h"

#include <mutex>

namespace {

using namespace swiglu_impl;
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
#ifndef SWIGLU_BS_PREFETCH
#define SWIGLU_BS_PREFETCH 2           // rows loaded ahead of the one computed (backward): 0, 1 or 2
#endif
#ifndef SWIGLU_BS_ONE_SHOT
#define SWIGLU_BS_ONE_SHOT 1           // backward without dbias on wide rows: one-shot grid
#endif
#ifndef SWIGLU_BS_TILE
#define SWIGLU_BS_TILE 1               // backward with dbias on wide rows: one-shot tile kernel
#endif
#ifndef SWIGLU_BS_TILE_WAVES
#define SWIGLU_BS_TILE_WAVES 16        // waves per tile block, each on its own rows
#endif
#ifndef SWIGLU_BS_TILE_RPL
#define SWIGLU_BS_TILE_RPL 2           // rows per lane and phase in the tile kernel
#endif
#ifndef SWIGLU_BS_TILE_PHASES
#define SWIGLU_BS_TILE_PHASES 2        // phases of the tile kernel (rows per lane = RPL x PHASES)
#endif
#ifndef SWIGLU_BS_TILE_MIN_BLOCKS
#define SWIGLU_BS_TILE_MIN_BLOCKS 1    // tile blocks per CU the register budget must allow
#endif
#ifndef SWIGLU_BS_INTERLEAVE
#define SWIGLU_BS_INTERLEAVE 1         // group y takes rows y, y+G, y+2G, ... (else a band)
#endif
constexpr int kBsRows = SWIGLU_BS_ROWS_PER_GROUP;
constexpr int kWaves = kBlock / 64;
constexpr int kTileWaves = SWIGLU_BS_TILE_WAVES;
constexpr int kTileRpl = SWIGLU_BS_TILE_RPL;
constexpr int kTilePhases = SWIGLU_BS_TILE_PHASES;
constexpr int kTileRows = kTileWaves * kTileRpl * kTilePhases;   // rows per tile block (one partial)
constexpr int kTileThreads = 64 * kTileWaves;
// Rows per dbias partial, at most: the workspace is sized for the smaller group.
constexpr int kMinGroupRows = kTileRows < kBsRows ? kTileRows : kBsRows;

// Exact sum of two fp32 values as head + tail (Knuth's two-sum).
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// Widens VEC elements of T held as raw bits (as Vec<T, VEC>::load does
// after its load).
template <typename T, int VEC>
__device__ __forceinline__ void widen_bits(typename Vec<T, VEC>::R r, float (&f)[VEC]) {
    constexpr int kBytes = Vec<T, VEC>::kBytes;
    if constexpr (sizeof(T) == 4) {
        __builtin_memcpy(f, &r, sizeof(r));
    } else if constexpr (kBytes == 2) {
        f[0] = __uint_as_float((uint32_t)r << 16);
    } else {
        uint32_t w[kBytes / 4];
        __builtin_memcpy(w, &r, sizeof(r));
#pragma unroll
        for (int i = 0; i < kBytes / 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);           // lower address: low half
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

#ifndef SWIGLU_BS_BIAS_ROWS
#define SWIGLU_BS_BIAS_ROWS 2    // rows per lane with a bias: wide forward, one-shot backward (1 or 2)
#endif
constexpr int kBiasRows = SWIGLU_BS_BIAS_ROWS;
static_assert(kBiasRows == 1 || kBiasRows == 2, "rows per lane");

template <typename T, int VEC, bool WIDE, bool HAS_BIAS, bool HAS_SCALE>
__global__ __launch_bounds__(kBlock) void swiglu_fwd_bs_kernel(
    const T* __restrict__ gp, int64_t gs, const T* __restrict__ up, int64_t us,
    T* __restrict__ y, int64_t ys, const T* __restrict__ bg, const T* __restrict__ bu,
    const float* __restrict__ sc, int64_t scs, Geom G) {
    if constexpr (WIDE && HAS_BIAS && kBiasRows == 2) {
        // Block (x, y) takes vectors [256 x, 256 x + 256) of rows 2y and
        // 2y + 1; each lane loads its bias vectors once for both rows.
        const uint32_t col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
        if (col >= G.nv) return;
        const int64_t r0 = 2 * (int64_t)blockIdx.y;
        const bool two = r0 + 1 < G.rows;                  // uniform
        const int64_t c = (int64_t)col * VEC;
        typedef typename Vec<T, VEC>::R R;
        const R g0 = load_raw<R>(gp + r0 * gs + c);
        const R u0 = load_raw<R>(up + r0 * us + c);
        R g1{}, u1{};
        if (two) {
            g1 = load_raw<R>(gp + (r0 + 1) * gs + c);
            u1 = load_raw<R>(up + (r0 + 1) * us + c);
        }
        const R bgr = *reinterpret_cast<const R*>(bg + c);
        const R bur = *reinterpret_cast<const R*>(bu + c);
        const float s0 = HAS_SCALE ? sc[r0 * scs] : 1.0f;
        const float s1 = HAS_SCALE && two ? sc[(r0 + 1) * scs] : 1.0f;
        float b[VEC], d[VEC];
        widen_bits<T, VEC>(bgr, b);
        widen_bits<T, VEC>(bur, d);
        auto one_row = [&](const R& gr, const R& ur, float s, T* dst) {
            float g[VEC], u[VEC], out[VEC];
            widen_bits<T, VEC>(gr, g);
            widen_bits<T, VEC>(ur, u);
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                g[i] += b[i];
                u[i] += d[i];
                float sig, osig, scl;
                sigmoid_pair<T, false>(g[i], sig, osig, scl);
                out[i] = HAS_SCALE ? ((g[i] * sig) * (u[i] * s)) * scl : ((g[i] * sig) * u[i]) * scl;
            }
            Vec<T, VEC>::store(dst, out);
        };
        one_row(g0, u0, s0, y + r0 * ys + c);
        if (two) one_row(g1, u1, s1, y + (r0 + 1) * ys + c);
        return;
    }
    int64_t row;
    uint32_t col;
    if (!locate<WIDE>(G, row, col)) return;
    const int64_t c = (int64_t)col * VEC;
    // Every load is issued before any is used (bias and scale are compile-
    // time options, so there is no branch between them).
    typedef typename Vec<T, VEC>::R R;
    const R gr = load_raw<R>(gp + row * gs + c);
    const R ur = load_raw<R>(up + row * us + c);
    R bgr{}, bur{};
    if constexpr (HAS_BIAS) {
        bgr = *reinterpret_cast<const R*>(bg + c);     // re-read by every row: cached
        bur = *reinterpret_cast<const R*>(bu + c);
    }
    const float s = HAS_SCALE ? sc[row * scs] : 1.0f;
    float g[VEC], u[VEC], out[VEC];
    widen_bits<T, VEC>(gr, g);
    widen_bits<T, VEC>(ur, u);
    if constexpr (HAS_BIAS) {
        float b[VEC], d[VEC];
        widen_bits<T, VEC>(bgr, b);
        widen_bits<T, VEC>(bur, d);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            g[i] += b[i];
            u[i] += d[i];
        }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        float sig, osig, scl;
        sigmoid_pair<T, false>(g[i], sig, osig, scl);
        out[i] = HAS_SCALE ? ((g[i] * sig) * (u[i] * s)) * scl : ((g[i] * sig) * u[i]) * scl;
    }
    Vec<T, VEC>::store(y + row * ys + c, out);
}

// Partial sums of a backward over rows [row0 + y*R, row0 + (y+1)*R) for the
// column tile x. Writes dz for every element; part_db[group][k] gets this
// group's column sums (k in [0, 2n): gate columns, then up columns) and
// part_ds[x][w][row] wave w's share of each row's ds. Fixed summation order
// throughout: each lane adds its rows in order, each wave's share is a fixed
// butterfly, and the second pass adds tiles and waves in order.
struct BsGeom {
    int64_t rows;       // rows in this launch
    int64_t n;          // half width (elements)
    int64_t group0;     // global index of this launch's first row group
    int64_t row0;       // global index of this launch's first row
    int64_t total_rows; // rows of the whole problem (the stride of part_ds)
    uint32_t nv;        // vectors per half row
    uint32_t tiles;     // column tiles per row (= gridDim.x)
};

// Sum of v over the 64 lanes of a wave, in a fixed order, through DPP lane
// permutes (no LDS): pairs, quads, 8-lane and 16-lane mirrors, then the
// row broadcasts that fold the four 16-lane rows into lane 63. Every lane
// of the wave must be active. Returns the total (read from lane 63).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141, 0xF>(v);   // row_half_mirror
    v += dpp_f<0x140, 0xF>(v);   // row_mirror
    v += dpp_f<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One element of the backward: z = x + bias (the gate carried as a two-sum,
// so the root series sees the sum's rounding error), dz for gate and up, and
// the element's term dy * silu(z_g) * z_u added to p (for dscale). Shared by
// the row-loop, tile and one-shot kernels so that all give the same bits.
template <typename T>
__device__ __forceinline__ void bwd_bs_elem(float g, float u, float d, float bg, float bu, float s,
                                            float& dg, float& du, float& p) {
    float zg, zlo;
    two_sum(g, bg, zg, zlo);
    const float zu = u + bu;
    float sig, osig, scl;
    sigmoid_pair<T, true>(zg, sig, osig, scl);
    const float h = h_factor_lo<T>(zg, zlo, osig);
    const float silu = zg * sig;                    // times 1/scl, as sig
    const float ds_ = d * s;
    du = (ds_ * silu) * scl;
    dg = ((ds_ * zu) * (sig * h)) * scl;           // sigma h = silu'(z) first: |.| <= 1.1
    p = __builtin_fmaf((d * silu) * scl, zu, p);
}

template <typename T, int VEC, bool IN_PLACE>
__global__ __launch_bounds__(kBlock) void swiglu_bwd_bs_kernel(
    const T* dyp, int64_t dys, T* gp, int64_t gs, T* up, int64_t us, T* dgp, int64_t dgs,
    T* dup, int64_t dus, const T* __restrict__ bg, const T* __restrict__ bu,
    const float* __restrict__ sc, int64_t scs, float* part_db, float* part_ds, BsGeom G) {
    if constexpr (IN_PLACE) {
        dgp = gp;
        dgs = gs;
        dup = up;
        dus = us;
    }
    const uint32_t col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
    const bool active = col < G.nv;
    const int64_t c = (int64_t)col * VEC;
    // Rows of this group, in the order they are summed: with INTERLEAVE the
    // G = gridDim.y groups advance through the tensor together (row
    // blockIdx.y + j*G at step j), so the rows in flight across the grid form
    // one contiguous band, as in a one-shot grid; otherwise group y owns the
    // band [y*R, (y+1)*R).
#if SWIGLU_BS_INTERLEAVE
    const int64_t r_first = blockIdx.y, r_step = gridDim.y;
#else
    const int64_t r_first = (int64_t)blockIdx.y * kBsRows, r_step = 1;
#endif
    float bgv[VEC], buv[VEC], acc_g[VEC], acc_u[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        bgv[i] = buv[i] = 0.0f;
        acc_g[i] = acc_u[i] = 0.0f;
    }
    if (bg != nullptr && active) {
        Vec<T, VEC>::template load<true>(bg + c, bgv);
        Vec<T, VEC>::template load<true>(bu + c, buv);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // The row's math and stores; p collects dy * silu(z_g) * z_u for dscale.
    auto row_step = [&](int64_t row, float s, const float (&g)[VEC], const float (&u)[VEC],
                        const float (&d)[VEC]) {
        float p = 0.0f;
        if (active) {
            float dg[VEC], du[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                bwd_bs_elem<T>(g[i], u[i], d[i], bgv[i], buv[i], s, dg[i], du[i], p);
                acc_g[i] += dg[i];
                acc_u[i] += du[i];
            }
            Vec<T, VEC>::store(dgp + row * dgs + c, dg);
            Vec<T, VEC>::store(dup + row * dus + c, du);
        }
        if (part_ds != nullptr) {
            // One partial per (row, tile, wave); the second pass adds the
            // tiles and waves of a row in order.
            const float w = wave_sum(p);
            if (lane == 0)
                part_ds[((int64_t)blockIdx.x * kWaves + wave) * G.total_rows + G.row0 + row] = w;
        }
    };
#if SWIGLU_BS_PREFETCH == 2
    // Rows j + 1 and j + 2 are loaded (as raw bits) while row j is computed.
    typedef typename Vec<T, VEC>::R R;
    R g0{}, u0{}, d0{}, g1{}, u1{}, d1{};
    float s0 = 1.0f, s1 = 1.0f;
    auto load_row2 = [&](int j, R& gg, R& uu, R& dd, float& ss) {
        const int64_t rr = r_first + j * r_step;
        if (j < kBsRows && rr < G.rows) {             // uniform
            if (active) {
                gg = load_raw<R>(gp + rr * gs + c);
                uu = load_raw<R>(up + rr * us + c);
                dd = load_raw<R>(dyp + rr * dys + c);
            }
            if (sc != nullptr) ss = sc[rr * scs];
        }
    };
    load_row2(0, g0, u0, d0, s0);
    load_row2(1, g1, u1, d1, s1);
    for (int j = 0; j < kBsRows; ++j) {
        const int64_t row = r_first + j * r_step;
        if (row >= G.rows) break;                     // uniform
        R g2{}, u2{}, d2{};
        float s2 = 1.0f;
        load_row2(j + 2, g2, u2, d2, s2);
        float g[VEC], u[VEC], d[VEC];
        widen_bits<T, VEC>(g0, g);
        widen_bits<T, VEC>(u0, u);
        widen_bits<T, VEC>(d0, d);
        row_step(row, s0, g, u, d);
        g0 = g1; u0 = u1; d0 = d1; s0 = s1;
        g1 = g2; u1 = u2; d1 = d2; s1 = s2;
    }
#elif SWIGLU_BS_PREFETCH
    // Row j + 1 is loaded (as raw bits) while row j is computed, so two rows
    // of loads are in flight per wave.
    typedef typename Vec<T, VEC>::R R;
    R gr{}, ur{}, dr{};
    auto load_row = [&](int64_t row, R& gg, R& uu, R& dd) {
        if (active) {
            gg = load_raw<R>(gp + row * gs + c);
            uu = load_raw<R>(up + row * us + c);
            dd = load_raw<R>(dyp + row * dys + c);
        }
    };
    float s = 1.0f;                                   // the row's scale, also one row ahead
    if (r_first < G.rows) {
        load_row(r_first, gr, ur, dr);
        if (sc != nullptr) s = sc[r_first * scs];
    }
    for (int j = 0; j < kBsRows; ++j) {
        const int64_t row = r_first + j * r_step;
        if (row >= G.rows) break;                     // uniform
        const int64_t nrow = row + r_step;
        R gn{}, un{}, dn{};
        float sn = 1.0f;
        const bool more = j + 1 < kBsRows && nrow < G.rows;   // uniform
        if (more) {
            load_row(nrow, gn, un, dn);
            if (sc != nullptr) sn = sc[nrow * scs];
        }
        float g[VEC], u[VEC], d[VEC];
        widen_bits<T, VEC>(gr, g);
        widen_bits<T, VEC>(ur, u);
        widen_bits<T, VEC>(dr, d);
        row_step(row, s, g, u, d);
        gr = gn;
        ur = un;
        dr = dn;
        s = sn;
    }
#else
    for (int j = 0; j < kBsRows; ++j) {
        const int64_t row = r_first + j * r_step;
        if (row >= G.rows) break;                     // uniform
        const float s = sc != nullptr ? sc[row * scs] : 1.0f;
        float g[VEC], u[VEC], d[VEC];
        if (active) {
            Vec<T, VEC>::load(gp + row * gs + c, g);
            Vec<T, VEC>::load(up + row * us + c, u);
            Vec<T, VEC>::load(dyp + row * dys + c, d);
        }
        row_step(row, s, g, u, d);
    }
#endif
    if (part_db != nullptr && active) {
        float* pg = part_db + (G.group0 + blockIdx.y) * (2 * G.n) + c;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            pg[i] = acc_g[i];
            pg[G.n + i] = acc_u[i];
        }
    }
}

// The backward without dbias on wide rows (at least 256 vectors per half
// row): a one-shot grid like the base backward, block (x, y) = column tile x
// of row y. dscale partials, when wanted, are written exactly as the row-loop
// kernel writes them (same lanes, same wave sums), so the results are the
// same bits either way.
template <typename T, int VEC, bool IN_PLACE, bool HAS_BIAS, bool HAS_SCALE, bool WANT_DS>
__global__ __launch_bounds__(kBlock) void swiglu_bwd_bs1_kernel(
    const T* dyp, int64_t dys, T* gp, int64_t gs, T* up, int64_t us, T* dgp, int64_t dgs,
    T* dup, int64_t dus, const T* __restrict__ bg, const T* __restrict__ bu,
    const float* __restrict__ sc, int64_t scs, float* part_ds, BsGeom G) {
    if constexpr (IN_PLACE) {
        dgp = gp;
        dgs = gs;
        dup = up;
        dus = us;
    }
    if constexpr (HAS_BIAS && kBiasRows == 2) {
        // As in the forward: block (x, y) takes rows 2y and 2y + 1, and each
        // lane loads its bias vectors once for both.
        const int64_t r0 = 2 * (int64_t)blockIdx.y;
        const bool two = r0 + 1 < G.rows;                  // uniform
        const uint32_t col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
        const bool active = col < G.nv;
        if (!WANT_DS && !active) return;
        const int64_t c = (int64_t)col * VEC;
        typedef typename Vec<T, VEC>::R R;
        R g0{}, u0{}, d0{}, g1{}, u1{}, d1{}, bgr{}, bur{};
        if (active) {
            g0 = load_raw<R>(gp + r0 * gs + c);
            u0 = load_raw<R>(up + r0 * us + c);
            d0 = load_raw<R>(dyp + r0 * dys + c);
            if (two) {
                g1 = load_raw<R>(gp + (r0 + 1) * gs + c);
                u1 = load_raw<R>(up + (r0 + 1) * us + c);
                d1 = load_raw<R>(dyp + (r0 + 1) * dys + c);
            }
            bgr = *reinterpret_cast<const R*>(bg + c);
            bur = *reinterpret_cast<const R*>(bu + c);
        }
        const float s0 = HAS_SCALE ? sc[r0 * scs] : 1.0f;
        const float s1 = HAS_SCALE && two ? sc[(r0 + 1) * scs] : 1.0f;
        float b[VEC], e[VEC];
        widen_bits<T, VEC>(bgr, b);
        widen_bits<T, VEC>(bur, e);
        auto one_row = [&](int64_t row, const R& gr, const R& ur, const R& dr, float s) {
            float p = 0.0f;
            if (active) {
                float g[VEC], u[VEC], d[VEC], dg[VEC], du[VEC];
                widen_bits<T, VEC>(gr, g);
                widen_bits<T, VEC>(ur, u);
                widen_bits<T, VEC>(dr, d);
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    bwd_bs_elem<T>(g[i], u[i], d[i], b[i], e[i], s, dg[i], du[i], p);
                Vec<T, VEC>::store(dgp + row * dgs + c, dg);
                Vec<T, VEC>::store(dup + row * dus + c, du);
            }
            if constexpr (WANT_DS) {
                const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
                const float w = wave_sum(p);
                if (lane == 0)
                    part_ds[((int64_t)blockIdx.x * kWaves + wave) * G.total_rows + G.row0 + row] = w;
            }
        };
        one_row(r0, g0, u0, d0, s0);
        if (two) one_row(r0 + 1, g1, u1, d1, s1);
        return;
    }
    const int64_t row = blockIdx.y;
    const uint32_t col = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
    const bool active = col < G.nv;
    if (!WANT_DS && !active) return;
    const int64_t c = (int64_t)col * VEC;
    typedef typename Vec<T, VEC>::R R;
    R gr{}, ur{}, dr{}, bgr{}, bur{};
    if (active) {
        gr = load_raw<R>(gp + row * gs + c);
        ur = load_raw<R>(up + row * us + c);
        dr = load_raw<R>(dyp + row * dys + c);
        if constexpr (HAS_BIAS) {
            bgr = *reinterpret_cast<const R*>(bg + c);   // re-read by every row: cached
            bur = *reinterpret_cast<const R*>(bu + c);
        }
    }
    const float s = HAS_SCALE ? sc[row * scs] : 1.0f;
    float p = 0.0f;
    if (active) {
        float g[VEC], u[VEC], d[VEC], b[VEC], e[VEC], dg[VEC], du[VEC];
        widen_bits<T, VEC>(gr, g);
        widen_bits<T, VEC>(ur, u);
        widen_bits<T, VEC>(dr, d);
        widen_bits<T, VEC>(bgr, b);                     // zero bits when there is no bias
        widen_bits<T, VEC>(bur, e);
#pragma unroll
        for (int i = 0; i < VEC; ++i) bwd_bs_elem<T>(g[i], u[i], d[i], b[i], e[i], s, dg[i], du[i], p);
        Vec<T, VEC>::store(dgp + row * dgs + c, dg);
        Vec<T, VEC>::store(dup + row * dus + c, du);
    }
    if constexpr (WANT_DS) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const float w = wave_sum(p);
        if (lane == 0)
            part_ds[((int64_t)blockIdx.x * kWaves + wave) * G.total_rows + G.row0 + row] = w;
    }
}

// The backward with dbias on wide rows of 16-byte vectors, as a one-shot
// grid. Block (x, y) owns vectors [64 x, 64 x + 64) of the kTileRows rows
// [y R, (y + 1) R), R = W * kTileRpl * kTilePhases with W = kTileWaves: wave
// w takes rows y R + k W + w for k < kTileRpl * kTilePhases, each wave on its
// own rows. The rows come in kTilePhases phases of kTileRpl rows, and every
// lane issues all loads of a phase before the first is used. Each lane adds
// its rows' dz in row order; the waves' sums then go through LDS and are
// added in wave order, one thread per column, into this block's dbias
// partial part_db[group][k], written with consecutive threads on
// consecutive columns. The dscale partial of each (row, 64-vector chunk) is
// the chunk's wave sum, stored where the row-loop kernel stores it (chunk x
// of this grid is wave x % 4 of the row loop's tile x / 4), so dscale is the
// same bits either way. Fixed summation order throughout.
template <typename T, int VEC, bool IN_PLACE, bool HAS_BIAS, bool HAS_SCALE, bool WANT_DS>
__global__ __launch_bounds__(kTileThreads, SWIGLU_BS_TILE_MIN_BLOCKS) void swiglu_bwd_bs_tile_kernel(
    const T* dyp, int64_t dys, T* gp, int64_t gs, T* up, int64_t us, T* dgp, int64_t dgs,
    T* dup, int64_t dus, const T* __restrict__ bg, const T* __restrict__ bu,
    const float* __restrict__ sc, int64_t scs, float* part_db, float* part_ds, BsGeom G) {
    if constexpr (IN_PLACE) {
        dgp = gp;
        dgs = gs;
        dup = up;
        dus = us;
    }
    constexpr int kVals = 2 * VEC;                      // dz values per lane and row
    constexpr int kPad = kVals + 1;                     // LDS words per lane (odd: no conflicts)
    __shared__ float lds[kTileWaves * 64 * kPad];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t col = blockIdx.x * 64u + (uint32_t)lane;
    const bool active = col < G.nv;
    const int64_t c = (int64_t)col * VEC;
    const int64_t rbase = (int64_t)blockIdx.y * kTileRows + wave;
    typedef typename Vec<T, VEC>::R R;
    R bgr{}, bur{};
    if (HAS_BIAS && active) {
        bgr = *reinterpret_cast<const R*>(bg + c);      // re-read by every row: cached
        bur = *reinterpret_cast<const R*>(bu + c);
    }
    float acc[kVals];
#pragma unroll
    for (int i = 0; i < kVals; ++i) acc[i] = 0.0f;
    for (int ph = 0; ph < kTilePhases; ++ph) {
        R gr[kTileRpl], ur[kTileRpl], dr[kTileRpl];
        float s[kTileRpl];
#pragma unroll
        for (int k = 0; k < kTileRpl; ++k) {
            const int64_t row = rbase + (int64_t)(ph * kTileRpl + k) * kTileWaves;
            gr[k] = ur[k] = dr[k] = R{};
            if (active && row < G.rows) {
                gr[k] = load_raw<R>(gp + row * gs + c);
                ur[k] = load_raw<R>(up + row * us + c);
                dr[k] = load_raw<R>(dyp + row * dys + c);
            }
            s[k] = HAS_SCALE && row < G.rows ? sc[row * scs] : 1.0f;
        }
        float b[VEC], e[VEC];
        widen_bits<T, VEC>(bgr, b);                     // zero bits when there is no bias
        widen_bits<T, VEC>(bur, e);
#pragma unroll
        for (int k = 0; k < kTileRpl; ++k) {
            const int64_t row = rbase + (int64_t)(ph * kTileRpl + k) * kTileWaves;
            if (row >= G.rows) break;                   // uniform
            float p = 0.0f;
            if (active) {
                float g[VEC], u[VEC], d[VEC], dg[VEC], du[VEC];
                widen_bits<T, VEC>(gr[k], g);
                widen_bits<T, VEC>(ur[k], u);
                widen_bits<T, VEC>(dr[k], d);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    bwd_bs_elem<T>(g[i], u[i], d[i], b[i], e[i], s[k], dg[i], du[i], p);
                    acc[i] += dg[i];
                    acc[VEC + i] += du[i];
                }
                Vec<T, VEC>::store(dgp + row * dgs + c, dg);
                Vec<T, VEC>::store(dup + row * dus + c, du);
            }
            if constexpr (WANT_DS) {
                const float w = wave_sum(p);
                if (lane == 0) part_ds[(int64_t)blockIdx.x * G.total_rows + G.row0 + row] = w;
            }
        }
    }
    float* mine = lds + (wave * 64 + lane) * kPad;
#pragma unroll
    for (int i = 0; i < kVals; ++i) mine[i] = acc[i];
    __syncthreads();
    // thread t: column k = t % (64 VEC) of half t / (64 VEC) of this block
    for (int t = threadIdx.x; t < 64 * kVals; t += kTileThreads) {
        const int half = t / (64 * VEC), k = t % (64 * VEC);
        const int l = k / VEC, j = k % VEC;
        if (blockIdx.x * 64u + (uint32_t)l < G.nv) {
            const float* src = lds + l * kPad + half * VEC + j;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kTileWaves; ++w) sum += src[w * 64 * kPad];
            part_db[(G.group0 + blockIdx.y) * (2 * G.n) + half * G.n +
                    (int64_t)blockIdx.x * 64 * VEC + k] = sum;
        }
    }
}

// One fixed-order column of partial sums: out[k * out_stride] = sum over
// j < count of part[j * jstride + k * kstride], j in order.
struct PartialSum {
    const float* part;
    int64_t count, jstride, kstride, width;
    float* out;
    int64_t out_stride;
    int64_t blocks;     // blocks of kBlock threads over width
};

__device__ __forceinline__ void sum_one(const PartialSum& S, int64_t k) {
    if (k >= S.width) return;
    const float* p = S.part + k * S.kstride;
    float acc = 0.0f;
    int64_t j = 0;
    // 32 loads in flight, added in the same order as the plain loop
    for (; j + 32 <= S.count; j += 32) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = p[(j + i) * S.jstride];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc += v[i];
    }
    for (; j < S.count; ++j) acc += p[j * S.jstride];
    S.out[k * S.out_stride] = acc;
}

// Both second passes of the backward in one launch: blocks [0, A.blocks)
// sum A, the rest sum B (B.blocks may be 0).
__global__ __launch_bounds__(kBlock) void swiglu_sum_partials_kernel(PartialSum A, PartialSum B) {
    const int64_t bx = blockIdx.x;
    if (bx < A.blocks) sum_one(A, bx * kBlock + threadIdx.x);
    else sum_one(B, (bx - A.blocks) * kBlock + threadIdx.x);
}

__global__ __launch_bounds__(kBlock) void swiglu_zero_kernel(float* p, int64_t count,
                                                             int64_t stride) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k < count) p[k * stride] = 0.0f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// ---- bias / scale variants ---------------------------------------------------
struct BsArgs {
    const void* bias;        // [2n] of T or NULL
    const float* scale;      // [rows] with stride scale_stride, or NULL
    int64_t scale_stride;
};

template <typename T, int VEC, bool WIDE>
const void* fwd_bs_kernel_for(bool has_bias, bool has_scale) {
    if (has_bias)
        return has_scale
                   ? reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, WIDE, true, true>)
                   : reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, WIDE, true, false>);
    return has_scale
               ? reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, WIDE, false, true>)
               : reinterpret_cast<const void*>(&swiglu_fwd_bs_kernel<T, VEC, WIDE, false, false>);
}

template <typename T, int VEC>
swiglu_status fwd_bs_launch(const Operand* ops, const BsArgs& A, int64_t rows, int64_t n,
                            hipStream_t stream) {
    const Plan P = make_plan(n, VEC);
    const bool hb = A.bias != nullptr, hs = A.scale != nullptr;
    const void* k = P.wide ? fwd_bs_kernel_for<T, VEC, true>(hb, hs)
                           : fwd_bs_kernel_for<T, VEC, false>(hb, hs);
    const T* g;
    const T* u;
    T* y;
    int64_t gs = ops[0].stride, us = ops[1].stride, ys = ops[2].stride, scs = A.scale_stride;
    const T* bg = static_cast<const T*>(A.bias);
    const T* bu = bg != nullptr ? bg + n : nullptr;
    const float* sc;
    Geom G;
    G.nv = P.nv;
    G.inv_nv = 1.0 / (double)P.nv;
    void* args[] = {&g, &gs, &u, &us, &y, &ys, &bg, &bu, &sc, &scs, &G};
    if (P.rows_per_launch <= 0) return SWIGLU_ERR_BAD_SHAPE;   // n == 0 is never planned
    for (int64_t r0 = 0; r0 < rows; r0 += P.rows_per_launch) {
        const int64_t rc = rows - r0 < P.rows_per_launch ? rows - r0 : P.rows_per_launch;
        g = static_cast<const T*>(ops[0].p) + r0 * gs;
        u = static_cast<const T*>(ops[1].p) + r0 * us;
        y = const_cast<T*>(static_cast<const T*>(ops[2].p)) + r0 * ys;
        sc = A.scale != nullptr ? A.scale + r0 * scs : nullptr;
        G.rows = rc;
        const uint32_t gy = (uint32_t)(hb && kBiasRows == 2 ? (rc + 1) / 2 : rc);
        const dim3 grid = P.wide ? dim3(P.tiles, gy)
                                 : dim3(swiglu_host::flat_blocks(rc, P.nv, kBlock), 1);
        if (hipLaunchKernel(k, grid, dim3(kBlock), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

// Workspace layout of the backward: [part_db: groups x 2n fp32]
// [part_ds: tiles x waves x rows fp32],
// each part starting on a 256-byte boundary. tiles is bounded by the
// single-element access width, so the size does not depend on alignment.
int64_t bs_groups(int64_t rows, int64_t rows_per_group = kBsRows) {
    return (rows + rows_per_group - 1) / rows_per_group;
}
int64_t bs_max_tiles(int64_t n) { return (n + kBlock - 1) / kBlock; }
int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

size_t bs_workspace_bytes(int64_t rows, int64_t n, bool want_db, bool want_ds) {
    int64_t b = 0;
    if (want_db) b += round256(bs_groups(rows, kMinGroupRows) * 2 * n * 4);
    if (want_ds) b += round256(rows * bs_max_tiles(n) * kWaves * 4);
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

PartialSum partial_sum(const float* part, int64_t count, int64_t jstride, int64_t kstride,
                       int64_t width, float* out, int64_t out_stride) {
    return PartialSum{part, count, jstride, kstride, width, out, out_stride,
                      (width + kBlock - 1) / kBlock};
}

// The second passes (either may be absent: blocks 0), in one launch.
swiglu_status sum_partials(PartialSum A, PartialSum B, hipStream_t stream) {
    const int64_t blocks = A.blocks + B.blocks;
    if (blocks == 0) return SWIGLU_OK;
    void* args[] = {&A, &B};
    return hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_sum_partials_kernel),
                           dim3((uint32_t)blocks), dim3(kBlock), args, 0, stream) == hipSuccess
               ? SWIGLU_OK
               : SWIGLU_ERR_HIP;
}

// The one-shot backward for the given options (16-byte vectors only).
template <typename T, int VEC>
const void* bwd_bs1_kernel_for(bool in_place, bool has_bias, bool has_scale, bool want_ds) {
    if constexpr (VEC * sizeof(T) != 16) {
        return nullptr;
    } else {
#define SWIGLU_BS1(IP, B, S, D) reinterpret_cast<const void*>(&swiglu_bwd_bs1_kernel<T, VEC, IP, B, S, D>)
#define SWIGLU_BS1_S(IP, B) \
    (!has_scale ? SWIGLU_BS1(IP, B, false, false) \
                : want_ds ? SWIGLU_BS1(IP, B, true, true) : SWIGLU_BS1(IP, B, true, false))
        if (in_place) return has_bias ? SWIGLU_BS1_S(true, true) : SWIGLU_BS1_S(true, false);
        return has_bias ? SWIGLU_BS1_S(false, true) : SWIGLU_BS1_S(false, false);
#undef SWIGLU_BS1_S
#undef SWIGLU_BS1
    }
}

// The tile backward (dbias wanted, so there is a bias; 16-byte vectors only).
template <typename T, int VEC>
const void* bwd_tile_kernel_for(bool in_place, bool has_scale, bool want_ds) {
    if constexpr (VEC * sizeof(T) != 16) {
        return nullptr;
    } else {
#define SWIGLU_BST(IP, S, D) reinterpret_cast<const void*>(&swiglu_bwd_bs_tile_kernel<T, VEC, IP, true, S, D>)
#define SWIGLU_BST_S(IP) \
    (!has_scale ? SWIGLU_BST(IP, false, false) \
                : want_ds ? SWIGLU_BST(IP, true, true) : SWIGLU_BST(IP, true, false))
        return in_place ? SWIGLU_BST_S(true) : SWIGLU_BST_S(false);
#undef SWIGLU_BST_S
#undef SWIGLU_BST
    }
}

// ops: dy, gate, up, dgate, dup.
template <typename T, int VEC>
swiglu_status bwd_bs_launch(const Operand* ops, const BsArgs& A, int64_t rows, int64_t n,
                            bool in_place, float* dbias, float* dscale, int64_t dscale_stride,
                            void* workspace, hipStream_t stream) {
    const uint32_t nv = (uint32_t)(n / VEC);
    const uint32_t tiles = (nv + kBlock - 1) / kBlock;
    // With dbias, wide rows of 16-byte vectors take the one-shot tile kernel
    // (kTileRows rows per partial); the row loop takes the rest.
    const bool tile = SWIGLU_BS_TILE && dbias != nullptr && nv >= 64u && VEC * sizeof(T) == 16;
    const int64_t group_rows = tile ? (int64_t)kTileRows : (int64_t)kBsRows;
    const int64_t groups = bs_groups(rows, group_rows);
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
    G.total_rows = rows;
    // Without dbias, wide rows of 16-byte vectors take the one-shot kernel
    // (the row loop and the tile kernel exist for the dbias column sums).
    const bool one_shot = SWIGLU_BS_ONE_SHOT && dbias == nullptr && nv >= (uint32_t)kBlock &&
                          VEC * sizeof(T) == 16;
    void* args[] = {&dyp, &dys, &gp, &gs, &upp, &us, &dgp, &dgs, &dup, &dus,
                    &bg, &bu, &sc, &scs, &part_db, &part_ds, &G};
    void* args1[] = {&dyp, &dys, &gp, &gs, &upp, &us, &dgp, &dgs, &dup, &dus,
                     &bg, &bu, &sc, &scs, &part_ds, &G};
    const void* k1 = one_shot ? bwd_bs1_kernel_for<T, VEC>(in_place, bg != nullptr,
                                                           A.scale != nullptr, dscale != nullptr)
                              : nullptr;
    const void* kt = tile ? bwd_tile_kernel_for<T, VEC>(in_place, A.scale != nullptr,
                                                        dscale != nullptr)
                          : nullptr;
    const int64_t rows_per_launch = one_shot ? (int64_t)kMaxGridY : (int64_t)kMaxGridY * group_rows;
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
        G.group0 = r0 / group_rows;
        if (one_shot) {
            // with a bias, a block takes two rows (see the kernel)
            const uint32_t gy =
                (uint32_t)(bg != nullptr && kBiasRows == 2 ? (rc + 1) / 2 : rc);
            if (hipLaunchKernel(k1, dim3(tiles, gy), dim3(kBlock), args1, 0, stream) !=
                hipSuccess)
                return SWIGLU_ERR_HIP;
            continue;
        }
        const uint32_t gy = (uint32_t)bs_groups(rc, group_rows);
        if (tile) {
            // one block per 64-vector chunk: tiles * kWaves chunks, so that
            // every dscale partial the second pass reads is written
            if (hipLaunchKernel(kt, dim3(tiles * kWaves, gy), dim3(kTileThreads), args, 0,
                                stream) != hipSuccess)
                return SWIGLU_ERR_HIP;
            continue;
        }
        if (hipLaunchKernel(k, dim3(tiles, gy), dim3(kBlock), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    PartialSum sdb{}, sds{};
    if (dbias != nullptr) sdb = partial_sum(part_db, groups, 2 * n, 1, 2 * n, dbias, 1);
    if (dscale != nullptr)
        sds = partial_sum(part_ds, (int64_t)tiles * kWaves, rows, 1, rows, dscale, dscale_stride);
    return sum_partials(sdb, sds, stream);
}

}  // namespace

extern "C" {

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
    const int vb = vec_bytes((int)esz, n, ops, bias != nullptr ? 5 : 3);
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

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free backward: a file-scope device array
// that every GPU the library runs on holds until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory, so it is
// never passed to a kernel or a copy: its device address is looked up once
// per device (with that device current) and the looked-up pointer is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SWIGLU_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of `scratch` on the current device.
swiglu_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SWIGLU_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SWIGLU_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SWIGLU_OK;
}

// The backward with its partial sums in `workspace` (caller's), or, with
// use_static, in the static scratch (workspace and workspace_bytes unused).
swiglu_status bias_scale_bwd(const void* dy, int64_t dy_row_stride, void* x, int64_t x_row_stride,
                             const void* bias, const float* scale, int64_t scale_stride, void* dx,
                             int64_t dx_row_stride, float* dbias, float* dscale,
                             int64_t dscale_stride, void* workspace, size_t workspace_bytes,
                             bool use_static, int64_t rows, int64_t n, swiglu_dtype dtype,
                             int in_place, hipStream_t stream) {
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
    if (use_static) {
        if (need > SWIGLU_NOALLOC_SCRATCH_BYTES) return SWIGLU_ERR_SCRATCH_LIMIT;
        workspace = nullptr;           // looked up after validation, just before the launch
    } else if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                            (uintptr_t)workspace % 16)) {
        return SWIGLU_ERR_WORKSPACE;
    }

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
    if (need > 0 && !use_static)       // the static array is no caller's memory
        outs[nout++] = Span{(uintptr_t)workspace, (uintptr_t)workspace + need};
    for (int i = 0; i < nout; ++i) {
        for (int j = (i == 0 ? 2 - (ip ? 1 : 0) : 0); j < nin; ++j)   // dx vs dy/x: checked above
            if (spans_overlap(outs[i], ins[j])) return SWIGLU_ERR_ALIASING;
        for (int j = i + 1; j < nout; ++j)
            if (spans_overlap(outs[i], outs[j])) return SWIGLU_ERR_ALIASING;
    }

    if (use_static && need > 0 && (st = scratch_on_current_device(&workspace)) != SWIGLU_OK)
        return st;

    const BsArgs A{bias, scale, scale_stride};
    const Operand ops[7] = {ody, ox, Operand{offset(x, n, esz), x_row_stride}, odx,
                            Operand{offset(dx, n, esz), dx_row_stride}, Operand{bias, 0},
                            Operand{offset(bias, n, esz), 0}};
    const int vb = vec_bytes((int)esz, n, ops, bias != nullptr ? 7 : 5);
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

}  // namespace

extern "C" {

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_bias_scale_bwd(
    const void* dy, int64_t dy_row_stride, void* x, int64_t x_row_stride, const void* bias,
    const float* scale, int64_t scale_stride, void* dx, int64_t dx_row_stride, float* dbias,
    float* dscale, int64_t dscale_stride, void* workspace, size_t workspace_bytes, int64_t rows,
    int64_t n, swiglu_dtype dtype, int in_place, hipStream_t stream) {
    return bias_scale_bwd(dy, dy_row_stride, x, x_row_stride, bias, scale, scale_stride, dx,
                          dx_row_stride, dbias, dscale, dscale_stride, workspace, workspace_bytes,
                          false, rows, n, dtype, in_place, stream);
}

__attribute__((visibility("default"))) swiglu_status swiglu_gateup_bias_scale_bwd_noalloc(
    const void* dy, int64_t dy_row_stride, void* x, int64_t x_row_stride, const void* bias,
    const float* scale, int64_t scale_stride, void* dx, int64_t dx_row_stride, float* dbias,
    float* dscale, int64_t dscale_stride, int64_t rows, int64_t n, swiglu_dtype dtype,
    int in_place, hipStream_t stream) {
    return bias_scale_bwd(dy, dy_row_stride, x, x_row_stride, bias, scale, scale_stride, dx,
                          dx_row_stride, dbias, dscale, dscale_stride, nullptr, 0, true, rows, n,
                          dtype, in_place, stream);
}

}  // extern "C"
