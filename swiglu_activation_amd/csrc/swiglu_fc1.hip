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
//  * k is walked in tiles of TILE_K (64) through a ring of STAGES (2) LDS
//    stages, each 256 token rows + 256 weight rows of TILE_K bf16. Global
//    memory is copied straight into LDS (global_load_lds_dwordx4: no
//    registers, no LDS write instructions); the copies of the next
//    STAGES - 1 tiles are in flight while one tile feeds the MFMAs. Each
//    stage is its own LDS array and the loop is unrolled over the ring, so
//    the compiler can tell the stage being read from the ones being filled
//    and waits only where the data is needed. (64-wide tiles in 2 stages
//    measured faster than 32-wide tiles in 3 to 5: each copy instruction
//    then reads whole 128-byte lines.)
//  * A copy instruction writes 1 KiB of LDS in lane order (rows of
//    2 TILE_K bytes), so the layout is chosen through the global addresses:
//    the 16-byte chunks of a row are permuted by an XOR with bits of the
//    row index, which makes the fragment reads free of bank conflicts.
//  * The next k step's fragments are read while the current step's MFMAs
//    run; one barrier per tile hands a filled stage to the readers and an
//    emptied one to the copies.
//  * The copies of a tile are spread thinly over two k steps (one every two
//    MFMAs), not issued in a burst: a burst fills the copy queue, and the
//    wave, which issues in order, then stalls in front of its next MFMA.
//    Each copy is addressed as a wave-uniform base in scalar registers plus
//    a fixed 32-bit lane offset, so no vector instruction sits between two
//    copies (which limits lda and ldw to 2^28 elements).
//  * Rows past m (tokens) or n (features) are clamped to the last valid row:
//    they copy real data, which reaches only accumulators that are never
//    stored.
#include "swiglu_device.h"

namespace {

using namespace swiglu_impl;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

#ifndef SWIGLU_FC_GROUP
#define SWIGLU_FC_GROUP 32      // token tiles that share a weight tile in the launch order
#endif
#ifndef SWIGLU_FC_XCD
#define SWIGLU_FC_XCD 0         // give each XCD a contiguous range of the launch order
#endif
#ifndef SWIGLU_FC_LDS_EPI
#define SWIGLU_FC_LDS_EPI 1     // stage the epilogue through LDS for whole-line stores
#endif
#ifndef SWIGLU_FC_NT_EPI
#define SWIGLU_FC_NT_EPI 0      // nontemporal hint on the epilogue's stores
#endif
#ifndef SWIGLU_FC_COPYMAP
#define SWIGLU_FC_COPYMAP 0     // 1: each wave copies a contiguous band of rows
#endif
#ifndef SWIGLU_FC_CPOL
#define SWIGLU_FC_CPOL 0        // cache-policy bits of the copies (gfx950: 1 sc0, 2 nt)
#endif
#ifndef SWIGLU_FC_SCHED
#define SWIGLU_FC_SCHED 1       // pin the interleaving of MFMAs and memory instructions
#endif
#ifndef SWIGLU_FC_SADDR
#define SWIGLU_FC_SADDR 1       // copies as a wave-uniform base (SGPRs) plus a fixed 32-bit lane offset
#endif
#ifndef SWIGLU_FC_SPREAD
#define SWIGLU_FC_SPREAD 2      // copy issue: 0 packed early in the step after the barrier; N >= 1
#endif                          // spread evenly over that step and the next N - 1 steps

#ifndef SWIGLU_FC_WAVES
#define SWIGLU_FC_WAVES 4       // waves per workgroup: 4 (128 x 64 wave tiles) or 8 (64 x 64)
#endif
static_assert(SWIGLU_FC_WAVES == 4 || SWIGLU_FC_WAVES == 8, "wave count");
constexpr int kFcWaveT = SWIGLU_FC_WAVES == 4 ? 128 : 64;   // tokens per wave
constexpr int kFcWaveF = 64;                         // features per wave (gate and up each)
constexpr int kFcWavesT = SWIGLU_FC_WAVES / 2, kFcWavesF = 2;
constexpr int kFcWaves = kFcWavesT * kFcWavesF;
constexpr int kFcThreads = 64 * kFcWaves;
constexpr int kFcMT = kFcWaveT / 32;                 // 32x32 tiles per wave along tokens
constexpr int kFcMF = kFcWaveF / 32;                 // ... along features (each: gate + up)
constexpr int kFcTileT = kFcWaveT * kFcWavesT;       // tokens per workgroup
constexpr int kFcTileF = kFcWaveF * kFcWavesF;       // features per workgroup
#ifndef SWIGLU_FC_TILE_K
#define SWIGLU_FC_TILE_K 64     // k per stage (32 or 64)
#endif
constexpr int kFcTileK = SWIGLU_FC_TILE_K;           // k per stage
#ifndef SWIGLU_FC_STAGES
#define SWIGLU_FC_STAGES 2      // LDS stages in the ring (2 to 5; x k per stage <= 160 KiB)
#endif
constexpr int kFcStages = SWIGLU_FC_STAGES;
constexpr int kFcRowsA = kFcTileT;                   // token rows per stage
constexpr int kFcRows = kFcTileT + 2 * kFcTileF;     // + gate rows + up rows
constexpr int kFcRowElems = kFcTileK;                // bf16 per LDS row (no padding)
constexpr int kFcStageElems = kFcRows * kFcRowElems;
constexpr int kFcChunks = kFcTileK / 8;              // 16-byte chunks per row
constexpr int kFcCopyRows = 64 / kFcChunks;          // rows per copy instruction (one wave)
constexpr int kFcCopies = kFcRows / kFcCopyRows / kFcWaves;   // copies per thread per tile
constexpr int kFcMfma = 2 * kFcMF * kFcMT;           // MFMAs per wave per k step
constexpr int kFcReads = kFcMT + 2 * kFcMF;          // fragment reads per k step
constexpr int kFcSteps = kFcTileK / 16;              // MFMA k steps per stage
constexpr int64_t kFcMaxLd = (int64_t)1 << 28;      // largest lda / ldw (elements)
constexpr int kFcSpread = SWIGLU_FC_SPREAD > 0 ? SWIGLU_FC_SPREAD : 1;   // steps a tile's copies span
// The rest of a tile's copies go into the next slot's steps before its last
// one (steps 0 and 1 of four, step 0 of two); with two stages that slot's
// wait needs them, so at least one step must follow.
static_assert(kFcSpread <= (kFcSteps == 4 ? 3 : 2) && (kFcStages > 2 || kFcSpread <= kFcSteps - 1),
              "a tile's copies are all issued before the wait that needs them");
// First copy issued in step j of the span (j = 0: the step after the barrier).
constexpr int copy_begin(int j) { return j * kFcCopies / kFcSpread; }
static_assert(kFcTileK == 32 || kFcTileK == 64, "4 or 8 chunks per row");
static_assert(kFcSteps % 2 == 0, "fragment sets alternate within a stage");
static_assert(kFcCopies * kFcWaves * kFcCopyRows == kFcRows, "whole copies per stage");
static_assert(kFcRowsA % kFcCopyRows == 0 && kFcTileF % kFcCopyRows == 0, "copies do not straddle");
static_assert(kFcStages * kFcStageElems * 2 <= 160 * 1024, "the ring must fit in LDS");

struct Fc1Args {
    const uint16_t* a;   // [m, k] tokens, row stride lda
    const uint16_t* w;   // [2n, k] weights, row stride ldw
    uint16_t* y;         // [m, n], row stride ldy
    uint16_t* x;         // NULL or [m, 2n], row stride ldx
    int64_t lda, ldw, ldy, ldx;
    int64_t m, n, k;
};

// The LDS ring: one array per stage.
static_assert(kFcStages >= 2 && kFcStages <= 5, "ring size");
__shared__ __attribute__((aligned(16))) uint16_t fc_stage0[kFcStageElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_stage1[kFcStageElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_stage2[kFcStageElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_stage3[kFcStageElems];
#if SWIGLU_FC_STAGES == 5
__shared__ __attribute__((aligned(16))) uint16_t fc_stage4[kFcStageElems];
#endif

template <int S>
__device__ __forceinline__ uint16_t* stage() {
    static_assert(S >= 0 && S < kFcStages, "stage index");
    if constexpr (S == 0) return fc_stage0;
    else if constexpr (S == 1) return fc_stage1;
    else if constexpr (S == 2) return fc_stage2;
    else if constexpr (S == 3) return fc_stage3;
#if SWIGLU_FC_STAGES == 5
    else return fc_stage4;
#endif
}

// Stage s, chosen at run time (0 <= s < stages).
__device__ __forceinline__ uint16_t* stage_at(int s) {
    uint16_t* p = stage<0>();
    if (s == 1) p = stage<1>();
    if constexpr (kFcStages > 2) if (s == 2) p = stage<2 % kFcStages>();
    if constexpr (kFcStages > 3) if (s == 3) p = stage<3 % kFcStages>();
    if constexpr (kFcStages > 4) if (s == 4) p = stage<4 % kFcStages>();
    return p;
}

// Slot of 16-byte chunk c in LDS row r. A fragment read takes one chunk
// from each of 16 consecutive rows per LDS cycle; the swizzle spreads them
// over all 64 banks.
__device__ __forceinline__ int chunk_slot(int r, int c) {
    if constexpr (kFcChunks == 4) return c ^ ((r >> 2) & 3);
    else return c ^ ((r >> 1) & 7);
}

// The block of kFcCopyRows LDS rows that copy i of a wave fills: the waves
// interleave block by block (COPYMAP 0) or each takes a contiguous band.
__device__ __forceinline__ int copy_block(int i, int wave) {
#if SWIGLU_FC_COPYMAP
    return wave * kFcCopies + i;
#else
    return i * kFcWaves + wave;
#endif
}

// Source row of each of this thread's copies, at k = 0. Copy i of a wave
// fills LDS rows [R q, R q + R) of a stage, R = kFcCopyRows and
// q = copy_block(i, wave); lane l writes slot l % kFcChunks of row
// R q + l / kFcChunks, so it reads the chunk that belongs in that slot.
#if SWIGLU_FC_SADDR
// Copy i of a wave reads an 8-row block: a wave-uniform base (the block's
// first row, clamped) and a fixed per-lane byte offset within the block
// (at most 7 row strides + 112 bytes).
struct Sources {
    const char* base[kFcCopies];
    mutable uint32_t off[kFcCopies];
};
#else
struct Sources {
    const uint16_t* p[kFcCopies];
};
#endif

__device__ __forceinline__ void make_sources(const Fc1Args& P, int64_t t0, int64_t f0,
                                             Sources& src) {
#if SWIGLU_FC_SADDR
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kFcCopies; ++i) {
        const int r0 = copy_block(i, wave) * kFcCopyRows;          // the block's first row
        const int r = r0 + lane / kFcChunks;
        const int c = chunk_slot(r, lane % kFcChunks);
        const uint16_t* rowbase;
        int64_t b, row, ld;
        if (r0 < kFcRowsA) {
            rowbase = P.a;
            ld = P.lda;
            b = t0 + r0 < P.m ? t0 + r0 : P.m - 1;
            row = t0 + r < P.m ? t0 + r : P.m - 1;
        } else {
            const int w0 = r0 - kFcRowsA, wr = r - kFcRowsA;         // gate rows, then up rows
            rowbase = P.w + (w0 < kFcTileF ? 0 : P.n) * P.ldw;
            ld = P.ldw;
            b = f0 + (w0 % kFcTileF) < P.n ? f0 + (w0 % kFcTileF) : P.n - 1;
            row = f0 + (wr % kFcTileF) < P.n ? f0 + (wr % kFcTileF) : P.n - 1;
        }
        src.base[i] = reinterpret_cast<const char*>(rowbase + b * ld);
        src.off[i] = (uint32_t)((row - b) * ld * 2 + c * 16);
    }
#else
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kFcCopies; ++i) {
        const int r = copy_block(i, wave) * kFcCopyRows + lane / kFcChunks;
        const int c = chunk_slot(r, lane % kFcChunks);
        if (r < kFcRowsA) {
            const int64_t tok = t0 + r < P.m ? t0 + r : P.m - 1;
            src.p[i] = P.a + tok * P.lda + c * 8;
        } else {
            const int wr = r - kFcRowsA;                       // gate rows, then up rows
            const int64_t f = f0 + (wr % kFcTileF) < P.n ? f0 + (wr % kFcTileF) : P.n - 1;
            src.p[i] = P.w + ((wr < kFcTileF ? 0 : P.n) + f) * P.ldw + c * 8;
        }
    }
#endif
}

// Starts copies [I0, I1) of k tile t into stage S.
template <int S, int I0 = 0, int I1 = kFcCopies>
__device__ __forceinline__ void copy_tile(const Sources& src, int t) {
#if SWIGLU_FC_SADDR
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tb = (int64_t)t * kFcTileK * 2;                  // the tile's byte offset
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        uint16_t* dst = stage<S>() + copy_block(i, wave) * kFcCopyRows * kFcRowElems;
        // (the offset is made opaque in place, so that the compiler neither
        // folds base and offset into one loop-invariant vector pointer nor
        // copies the offset into a scratch register for each copy)
        asm volatile("" : "+v"(src.off[i]));
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.base[i] + tb + src.off[i]),
                                         (lds_void*)(dst), 16, 0, SWIGLU_FC_CPOL);
    }
#else
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        uint16_t* dst = stage<S>() + copy_block(i, wave) * kFcCopyRows * kFcRowElems;
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(src.p[i] + (int64_t)t * kFcTileK),
            (lds_void*)(dst), 16, 0, SWIGLU_FC_CPOL);
    }
#endif
}

// s_waitcnt: at most N copies (vector memory operations) outstanding, and
// no LDS operation.
template <int N>
__device__ __forceinline__ void wait_copies_and_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt in bits [3:0] and [15:14], expcnt (7: not waited on) in [6:4],
    // lgkmcnt (0) in [11:8]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier for the ring. The caller has waited for its own LDS
// reads and for the copies the next stage needs (s_waitcnt); the empty asm
// statements keep the compiler from moving memory accesses across the
// barrier. A fence here would drain every copy in flight.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Four fp32 values rounded to bf16 (nearest even) and stored as 8 bytes.
// A lane's four values are 16 bytes apart from its neighbours' in the row,
// so whole cache lines form only in L2: the stores carry no nontemporal
// hint (which would send the partial lines on to memory unmerged).
__device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        f32x2 pr = {v[2 * i], v[2 * i + 1]};
        w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
    }
#if SWIGLU_FC_NT_EPI
    __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(p));
#else
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
#endif
}

__device__ __forceinline__ bf16x8 frag(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// The fragments one wave needs for one 16-wide k step.
struct Frags {
    bf16x8 a[kFcMT], g[kFcMF], u[kFcMF];
};

// off: this lane's element offset for the step (its row within a 32-row
// tile, and the swizzled slot of its chunk).
template <int S>
__device__ __forceinline__ void load_frags(int wt, int wf, int off, Frags& F) {
    const uint16_t* base = stage<S>();
#pragma unroll
    for (int j = 0; j < kFcMT; ++j) F.a[j] = frag(base + (wt + 32 * j) * kFcRowElems + off);
#pragma unroll
    for (int i = 0; i < kFcMF; ++i) {
        F.g[i] = frag(base + (kFcRowsA + wf + 32 * i) * kFcRowElems + off);
        F.u[i] = frag(base + (kFcRowsA + kFcTileF + wf + 32 * i) * kFcRowElems + off);
    }
}

struct Acc {
    f32x16 g[kFcMF][kFcMT], u[kFcMF][kFcMT];   // [feature tile][token tile]
};

__device__ __forceinline__ void mfma_step(const Frags& C, Acc& acc) {
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j) {
            acc.g[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.g[i], C.a[j], acc.g[i][j], 0, 0, 0);
            acc.u[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.u[i], C.a[j], acc.u[i][j], 0, 0, 0);
        }
}

// Scheduling hints (instruction classes of the AMDGPU scheduler).
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100;

__device__ __forceinline__ void sched_reads_among_mfma() {
#if SWIGLU_FC_SCHED
#pragma unroll
    for (int q = 0; q < kFcReads; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, kFcMfma - kFcReads, 0);
    __builtin_amdgcn_sched_barrier(0);
#endif
}

template <int kUnused = 0>
__device__ __forceinline__ void sched_copies_reads_among_mfma() {
#if SWIGLU_FC_SCHED
    constexpr int per = kFcCopies / kFcReads;        // copies per fragment read
    static_assert(kUnused != 0 || per * kFcReads == kFcCopies, "copies spread evenly over the reads");
#pragma unroll
    for (int q = 0; q < kFcReads; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSgVmemRead, per, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, kFcMfma - kFcReads, 0);
    __builtin_amdgcn_sched_barrier(0);
#endif
}

// NC copies spread evenly over the step's MFMAs, the fragment reads after
// the first kFcReads of them.
template <int NC, int M = 0>
__device__ __forceinline__ void sched_mix_at() {
#if SWIGLU_FC_SCHED
    constexpr int nc = (M + 1) * NC / kFcMfma - M * NC / kFcMfma;
    if constexpr (nc > 0) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, nc, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if constexpr (M < kFcReads) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    if constexpr (M + 1 < kFcMfma) sched_mix_at<NC, M + 1>();
    else __builtin_amdgcn_sched_barrier(0);
#endif
}

// Launch order of the output tiles: consecutive workgroups take GROUP token
// tiles of one feature column of tiles before moving to the next feature
// tile, so each weight tile is fetched from HBM once per GROUP token tiles
// and the workgroups in flight share a working set that stays in the
// Infinity Cache.
__device__ __forceinline__ void tile_of(uint32_t b, uint32_t f_tiles, uint32_t t_tiles,
                                        uint32_t& ft, uint32_t& tt) {
#if SWIGLU_FC_XCD
    // Workgroups are dealt to the 8 XCDs round robin; renumber them so that
    // each XCD walks a contiguous range of the order above.
    const uint32_t total = f_tiles * t_tiles, q = total / 8, r = total % 8;
    const uint32_t xcd = b % 8, idx = b / 8;
    b = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
#endif
    const uint32_t per_group = SWIGLU_FC_GROUP * f_tiles;
    const uint32_t g = b / per_group, in = b % per_group;
    const uint32_t first_t = g * SWIGLU_FC_GROUP;
    const uint32_t gs = t_tiles - first_t < SWIGLU_FC_GROUP ? t_tiles - first_t : SWIGLU_FC_GROUP;
    tt = first_t + in % gs;
    ft = in / gs;
}

// Epilogue staging: a wave's tile (kFcWaveT tokens x 64 features of one output)
// in LDS rows of 72 bf16 (144 bytes, 16-byte aligned rows).
constexpr int kEpiPitch = kFcWaveF + 8;
constexpr int kEpiRegion = kFcWaveT * kEpiPitch;
// Regions per stage (at most half the waves, so that they spread over two
// or more stages) and the stages they take.
constexpr int kEpiPerStage = kFcStageElems / kEpiRegion < kFcWaves / 2 ? kFcStageElems / kEpiRegion
                                                                         : kFcWaves / 2;
static_assert(!SWIGLU_FC_LDS_EPI ||
                  (kEpiPerStage >= 1 && (kFcWaves + kEpiPerStage - 1) / kEpiPerStage <= kFcStages),
              "every wave's region fits in the stages");

// Writes the wave's kFcWaveT x 64 tile of one output, value(i, j, e) for
// accumulator element e of MFMA tile (feature i, token j), to out (row
// stride ld) at token tw, feature fw, skipping tokens >= m and features >= n.
// Register e of a 32x32 tile holds feature (e % 4) + 8 (e / 4) + 4 (lane / 32)
// and token lane % 32.
template <typename V>
__device__ __forceinline__ void epi_out(uint16_t* region, int64_t tw, int64_t fw, int64_t m,
                                        int64_t n, uint16_t* out, int64_t ld, V value) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = value(i, j, 4 * q + r);
                uint32_t w[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x2 pr = {v[2 * h], v[2 * h + 1]};
                    w[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                }
                const int row = 32 * j + lane % 32, col = 32 * i + 8 * q + 4 * (lane / 32);
                *reinterpret_cast<u32x2*>(region + row * kEpiPitch + col) = u32x2{w[0], w[1]};
            }
    // back by rows: lane l takes 16 bytes (8 features) of row 8 it + l / 8
    constexpr int kChunks = kFcWaveF / 8;             // 16-byte chunks per tile row
    constexpr int kRowsPerPass = 64 / kChunks;
#pragma unroll
    for (int it = 0; it < kFcWaveT / kRowsPerPass; ++it) {
        const int row = kRowsPerPass * it + lane / kChunks, col = 8 * (lane % kChunks);
        const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * kEpiPitch + col);
        const int64_t tok = tw + row, f = fw + col;
        if (tok < m && f < n) *reinterpret_cast<u32x4*>(out + tok * ld + f) = v;
    }
}

struct Ctx {
    Sources src;
    int wt, wf;
    int off[kFcSteps];   // this lane's fragment offset in each k step
    int kt_count;   // k tiles
    int pad;        // leading padding tiles that round the count up to the ring size
};

// Source tile of ring slot kt: padding slots and slots past the end are
// clamped to a real tile (their copies land in stages whose data is never
// multiplied in).
__device__ __forceinline__ int source_tile(const Ctx& c, int kt) {
    const int t = kt - c.pad;
    return t < 0 ? 0 : t < c.kt_count ? t : c.kt_count - 1;
}

// The fragments with the token operand zeroed when `live` is false, so a
// padding tile adds nothing.
__device__ __forceinline__ Frags masked(const Frags& F, bool live) {
    Frags r = F;
#pragma unroll
    for (int j = 0; j < kFcMT; ++j) r.a[j] = live ? F.a[j] : bf16x8{};
    return r;
}

// Ring slot kt (tile kt - pad), held in stage S = kt % stages. Entering: F0
// holds (or is receiving) the slot's first-step fragments, and the copies of
// the following slots up to kt + stages - 1 are in flight or done. The first step's MFMAs run
// while the second step's fragments are read. Then: wait for slot kt + 1,
// barrier (slot kt + 1 is complete for every wave, and stage S has been read
// by every wave), start the copies of slot kt + stages into stage S and read slot
// kt + 1's first-step fragments while the second step's MFMAs run. After the
// last slot these extra copies and reads are not used.
// One k step of stage S with fragments C while the next step's are read
// into N.
template <int S, int STEP>
__device__ __forceinline__ void inner_step(const Ctx& c, bool live, Frags& C, Frags& N, Acc& acc) {
    load_frags<S>(c.wt, c.wf, c.off[STEP + 1], N);
    mfma_step(masked(C, live), acc);
    sched_reads_among_mfma();
}

// inner_step that also issues copies [I0, I1) of slot ts into stage SP,
// spread over the step's MFMAs.
template <int S, int STEP, int SP, int I0, int I1>
__device__ __forceinline__ void copy_step(const Ctx& c, bool live, int ts, Frags& C, Frags& N,
                                          Acc& acc) {
    copy_tile<SP, I0, I1>(c.src, source_tile(c, ts));
    load_frags<S>(c.wt, c.wf, c.off[STEP + 1], N);
    mfma_step(masked(C, live), acc);
    sched_mix_at<I1 - I0>();
}

// MASK: the slot may be a padding slot (only in the first pass over the ring).
template <int S, bool MASK>
__device__ __forceinline__ void k_tile(const Ctx& c, int kt, Frags& F0, Frags& F1, Acc& acc) {
    constexpr int SN = (S + 1) % kFcStages;
    const bool live = !MASK || kt >= c.pad;
    // Steps 0 .. spread - 2 also issue the rest of the previous slot's
    // copies, into the stage that slot freed (there is none before slot 0).
    constexpr bool kTail = !(MASK && S == 0);
    constexpr int SP = (S + kFcStages - 1) % kFcStages;
    if constexpr (kTail && kFcSpread >= 2)
        copy_step<S, 0, SP, copy_begin(1), copy_begin(2)>(c, live, kt - 1 + kFcStages, F0, F1, acc);
    else
        inner_step<S, 0>(c, live, F0, F1, acc);
    if constexpr (kFcSteps == 4) {
        if constexpr (kTail && kFcSpread >= 3)
            copy_step<S, 1, SP, copy_begin(2), copy_begin(3)>(c, live, kt - 1 + kFcStages, F1, F0, acc);
        else
            inner_step<S, 1>(c, live, F1, F0, acc);
        inner_step<S, 2>(c, live, F0, F1, acc);
    }
    wait_copies_and_lds<(kFcStages - 2) * kFcCopies>();  // slots kt + 2 .. may be pending
    ring_barrier();
    copy_tile<S, 0, copy_begin(1)>(c.src, source_tile(c, kt + kFcStages));
    load_frags<SN>(c.wt, c.wf, c.off[0], F0);
    mfma_step(masked(F1, live), acc);
#if SWIGLU_FC_SPREAD == 0
    sched_copies_reads_among_mfma();
#else
    sched_mix_at<copy_begin(1)>();
#endif
}

// Slots kt .. kt + stages - 1: one pass over the ring.
template <bool MASK>
__device__ __forceinline__ void ring_pass(const Ctx& c, int kt, Frags& F0, Frags& F1, Acc& acc) {
    k_tile<0, MASK>(c, kt, F0, F1, acc);
    k_tile<1, MASK>(c, kt + 1, F0, F1, acc);
    if constexpr (kFcStages > 2) k_tile<2 % kFcStages, MASK>(c, kt + 2, F0, F1, acc);
    if constexpr (kFcStages > 3) k_tile<3 % kFcStages, MASK>(c, kt + 3, F0, F1, acc);
    if constexpr (kFcStages > 4) k_tile<4 % kFcStages, MASK>(c, kt + 4, F0, F1, acc);
}

__global__ __launch_bounds__(kFcThreads) void swiglu_fc1_kernel(Fc1Args P, uint32_t f_tiles,
                                                                uint32_t t_tiles) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t ft, tt;
    tile_of(blockIdx.x, f_tiles, t_tiles, ft, tt);
    const int64_t f0 = (int64_t)ft * kFcTileF;
    const int64_t t0 = (int64_t)tt * kFcTileT;

    Acc acc;
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j) {
            acc.g[i][j] = f32x16{};
            acc.u[i][j] = f32x16{};
        }

    Ctx c;
    make_sources(P, t0, f0, c.src);
    c.wf = (wave % kFcWavesF) * kFcWaveF;            // wave's feature offset
    c.wt = (wave / kFcWavesF) * kFcWaveT;            // wave's token offset
    c.kt_count = (int)(P.k / kFcTileK);
    const int slots = (c.kt_count + kFcStages - 1) / kFcStages * kFcStages;
    c.pad = slots - c.kt_count;
    {
        // A fragment lane reads row lane % 32 of a 32-row tile and chunk
        // 2 s + lane / 32 in step s.
        const int frow = lane % 32;
#pragma unroll
        for (int st = 0; st < kFcSteps; ++st)
            c.off[st] = frow * kFcRowElems + chunk_slot(frow, 2 * st + lane / 32) * 8;
    }

    // Fill the ring and wait for slot 0.
    copy_tile<0>(c.src, source_tile(c, 0));
    copy_tile<1>(c.src, source_tile(c, 1));
    if constexpr (kFcStages > 2) copy_tile<2 % kFcStages>(c.src, source_tile(c, 2));
    if constexpr (kFcStages > 3) copy_tile<3 % kFcStages>(c.src, source_tile(c, 3));
    if constexpr (kFcStages > 4) copy_tile<4 % kFcStages>(c.src, source_tile(c, 4));
    wait_copies_and_lds<(kFcStages - 1) * kFcCopies>();
    ring_barrier();
    Frags F0, F1;
    load_frags<0>(c.wt, c.wf, c.off[0], F0);

    // unrolled over the ring so that every stage is named statically
    // the padding slots all fall in the first pass, the only one that masks
    ring_pass<true>(c, 0, F0, F1, acc);
    for (int kt = kFcStages; kt < slots; kt += kFcStages) ring_pass<false>(c, kt, F0, F1, acc);
    // No copy may still be writing LDS when the workgroup ends.
    wait_copies_and_lds<0>();

#if SWIGLU_FC_LDS_EPI
    // Epilogue through LDS (free now): every wave writes its tile of each
    // output into a private LDS region in registers' order, then reads it
    // back by rows, so each store instruction writes 8 rows of 128 bytes.
    ring_barrier();                                   // every wave is done with the stages
    uint16_t* region = stage_at(wave / kEpiPerStage) + (wave % kEpiPerStage) * kEpiRegion;
    const int64_t tw = t0 + c.wt, fw = f0 + c.wf;     // the wave's first token and feature
    epi_out(region, tw, fw, P.m, P.n, P.y, P.ldy, [&](int i, int j, int e) {
        const float g = acc.g[i][j][e];
        float sig, osig;
        sigmoid_pair<uint16_t, false>(g, sig, osig);
        return (g * sig) * acc.u[i][j][e];
    });
    if (P.x != nullptr) {
        epi_out(region, tw, fw, P.m, P.n, P.x, P.ldx,
                [&](int i, int j, int e) { return acc.g[i][j][e]; });
        epi_out(region, tw, fw, P.m, P.n, P.x + P.n, P.ldx,
                [&](int i, int j, int e) { return acc.u[i][j][e]; });
    }
#else
    // Epilogue. Register v of a 32x32 tile holds feature
    // (v % 4) + 8 (v / 4) + 4 (lane / 32) and token lane % 32, so each group
    // of four registers is four consecutive features of one token.
#pragma unroll
    for (int i = 0; i < kFcMF; ++i)
#pragma unroll
        for (int j = 0; j < kFcMT; ++j) {
            const int64_t tok = t0 + c.wt + 32 * j + lane % 32;
            if (tok >= P.m) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t f = f0 + c.wf + 32 * i + 8 * q + 4 * (lane / 32);
                if (f >= P.n) continue;                 // n is a multiple of 64
                float yv[4], gv[4], uv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    gv[r] = acc.g[i][j][4 * q + r];
                    uv[r] = acc.u[i][j][4 * q + r];
                    float sig, osig;
                    sigmoid_pair<uint16_t, false>(gv[r], sig, osig);
                    yv[r] = (gv[r] * sig) * uv[r];
                }
                store4(P.y + tok * P.ldy + f, yv);
                if (P.x != nullptr) {
                    store4(P.x + tok * P.ldx + f, gv);
                    store4(P.x + tok * P.ldx + P.n + f, uv);
                }
            }
        }
#endif
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
    if (n % 64 != 0 || k % 64 != 0) return SWIGLU_ERR_BAD_SHAPE;
    swiglu_status st;
    if ((st = check_operand(m, lda, k, 2)) != SWIGLU_OK) return st;
    if ((st = check_operand(2 * n, ldw, k, 2)) != SWIGLU_OK) return st;
#if SWIGLU_FC_SADDR
    // A copy reads 8 rows through one 32-bit byte offset per lane:
    // 7 row strides + 112 bytes must stay below 2^32.
    if (lda > kFcMaxLd || ldw > kFcMaxLd) return SWIGLU_ERR_BAD_STRIDE;
#endif
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
    // One launch stays below 2^32 work-items and takes at most 65535 token tiles.
    const int64_t rows_per_launch =
        swiglu_host::fc1_rows_per_launch(n, kFcTileF, kFcTileT, kMaxGridY, kFcThreads);
    if (rows_per_launch <= 0) return SWIGLU_ERR_BAD_SHAPE;
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
