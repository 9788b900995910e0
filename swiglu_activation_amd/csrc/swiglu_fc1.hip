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
//    token. The epilogue passes each wave's tile through LDS (free once the
//    k loop ends), so every store instruction writes whole 128-byte rows.
//  * A workgroup of 4 waves computes 256 tokens x 128 features of y; each
//    wave 128 tokens x 64 features, i.e. 4 x 2 MFMA tiles for the gate and
//    4 x 2 for the up projection (256 fp32 accumulators per lane, in the
//    accumulation registers). Per 16-wide k step a wave reads 8 fragments
//    from LDS for 16 MFMAs: 1/64 byte of LDS traffic per flop.
//  * k is walked in tiles of 64 through two rings of LDS stages: the token
//    rows (256 x 64 bf16, 32 KiB) in A_STAGES (2) stages and the weight rows
//    (256 x 64 bf16) in W_STAGES (3) stages, 160 KiB in all. Global memory
//    is copied straight into LDS (global_load_lds_dwordx4: no registers, no
//    LDS write instructions). A tile's token copies are issued right after
//    the barrier that frees their stage, one tile ahead; its weight copies
//    (the operand that misses L2 more often: each weight tile is shared by
//    fewer of the workgroups an L2 serves) W_STAGES - 1 tiles ahead, issued
//    after the token copies so that a wait for the tokens never waits for
//    them. Each stage is its own LDS array and the loop is unrolled over
//    lcm(A_STAGES, W_STAGES) tiles, so every stage is named statically.
//  * A copy instruction writes 1 KiB of LDS in lane order (rows of
//    2 TILE_K bytes), so the layout is chosen through the global addresses:
//    the 16-byte chunks of a row are permuted by an XOR with bits of the
//    row index, which makes the fragment reads free of bank conflicts.
//  * The next k step's fragments are read while the current step's MFMAs
//    run; one barrier per tile hands a filled stage to the readers and an
//    emptied one to the copies.
//  * A tile's copies are spread evenly over the k steps, four per step
//    (half of the next slot's token copies in step 0, the weight copies in
//    steps 1 and 2, half of the token copies after the barrier), not issued
//    in a burst: a burst fills the copy queue, and the wave, which issues in
//    order, then stalls in front of its next MFMA. Each step is written out
//    as its 16 MFMAs with the fragment reads and copies pinned after chosen
//    ones (scheduling barriers), so the compiler cannot bunch them.
//    Each copy is addressed as a wave-uniform base in scalar registers plus
//    a fixed 32-bit lane offset, so no vector instruction sits between two
//    copies (which limits lda and ldw to 2^28 elements).
//  * Rows past m (tokens) or n (features) are clamped to the last valid row:
//    they copy real data, which reaches only accumulators that are never
//    stored.
//  * With a workspace, the last quarter of a large launch's tiles is a pool
//    taken through per-XCD queues, so XCDs running at higher clocks take
//    more tiles instead of idling at the end (below, at the kernel).
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
#ifndef SWIGLU_FC_POOL_DIV
#define SWIGLU_FC_POOL_DIV 4    // with a workspace: the last 1 / POOL_DIV of a large launch is a pool
#endif
#ifndef SWIGLU_FC_SURPLUS_DIV
#define SWIGLU_FC_SURPLUS_DIV 4 // ... taken by 1 + 1 / SURPLUS_DIV times as many workgroups
#endif
#ifndef SWIGLU_FC_LDS_EPI
#define SWIGLU_FC_LDS_EPI 1     // stage the epilogue through LDS for whole-line stores
#endif
#ifndef SWIGLU_FC_NT_EPI
#define SWIGLU_FC_NT_EPI 0      // nontemporal hint on the epilogue's stores
#endif
#ifndef SWIGLU_FC_CPOL
#define SWIGLU_FC_CPOL 0        // cache-policy bits of the copies (gfx950: 1 sc0, 2 nt)
#endif
#ifndef SWIGLU_FC_SCHED
#define SWIGLU_FC_SCHED 2       // 2: a fixed instruction order per step; 1: pinned interleaving hints
#endif
#ifndef SWIGLU_FC_SADDR
#define SWIGLU_FC_SADDR 1       // copies as a wave-uniform base (SGPRs) plus a fixed 32-bit lane offset
#endif
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
constexpr int kFcTileK = 64;                         // k per stage
#ifndef SWIGLU_FC_SPLIT
#define SWIGLU_FC_SPLIT 4       // copy issue: 1 token and weight groups in one step each; 2 in halves
#endif                          // over two steps each; 4 one half-group in every step
#ifndef SWIGLU_FC_A_STAGES
#define SWIGLU_FC_A_STAGES 2    // LDS stages of token rows
#endif
#ifndef SWIGLU_FC_W_STAGES
#define SWIGLU_FC_W_STAGES 3    // LDS stages of weight rows (2 or 3)
#endif
constexpr int kFcAStages = SWIGLU_FC_A_STAGES, kFcWStages = SWIGLU_FC_W_STAGES;
static_assert(kFcAStages == 2 && (kFcWStages == 2 || kFcWStages == 3), "ring sizes");
constexpr int kFcPeriod = kFcWStages == 3 ? 6 : 2;    // lcm of the ring sizes
constexpr int kFcRowsA = kFcTileT;                   // token rows per stage
constexpr int kFcRowsW = 2 * kFcTileF;               // gate rows + up rows per stage
constexpr int kFcRowElems = kFcTileK;                // bf16 per LDS row (no padding)
constexpr int kFcAElems = kFcRowsA * kFcRowElems;
constexpr int kFcWElems = kFcRowsW * kFcRowElems;
constexpr int kFcChunks = kFcTileK / 8;              // 16-byte chunks per row
constexpr int kFcCopyRows = 64 / kFcChunks;          // rows per copy instruction (one wave)
constexpr int kFcCopiesA = kFcRowsA / kFcCopyRows / kFcWaves;   // token copies per thread per tile
constexpr int kFcCopiesW = kFcRowsW / kFcCopyRows / kFcWaves;   // weight copies ...
constexpr int kFcCopies = kFcCopiesA + kFcCopiesW;
constexpr int kFcMfma = 2 * kFcMF * kFcMT;           // MFMAs per wave per k step
constexpr int kFcReads = kFcMT + 2 * kFcMF;          // fragment reads per k step
constexpr int kFcSteps = kFcTileK / 16;              // MFMA k steps per stage
constexpr int64_t kFcMaxLd = (int64_t)1 << 28;      // largest lda / ldw (elements)
static_assert(kFcSteps == 4, "four k steps per tile");
static_assert(kFcCopiesA * kFcWaves * kFcCopyRows == kFcRowsA &&
                  kFcCopiesW * kFcWaves * kFcCopyRows == kFcRowsW, "whole copies per stage");
static_assert(kFcTileF % kFcCopyRows == 0, "copies do not straddle gate and up rows");
static_assert((kFcAStages * kFcAElems + kFcWStages * kFcWElems) * 2 <= 160 * 1024,
              "the rings must fit in LDS");

struct Fc1Args {
    const uint16_t* a;   // [m, k] tokens, row stride lda
    const uint16_t* w;   // [2n, k] weights, row stride ldw
    uint16_t* y;         // [m, n], row stride ldy
    uint16_t* x;         // NULL or [m, 2n], row stride ldx
    int64_t lda, ldw, ldy, ldx;
    int64_t m, n, k;
};

// The LDS rings: one array per stage.
__shared__ __attribute__((aligned(16))) uint16_t fc_a0[kFcAElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_a1[kFcAElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_w0[kFcWElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_w1[kFcWElems];
__shared__ __attribute__((aligned(16))) uint16_t fc_w2[kFcWElems];

template <int S>
__device__ __forceinline__ uint16_t* stage_a() {
    static_assert(S >= 0 && S < kFcAStages, "stage index");
    if constexpr (S == 0) return fc_a0;
    else return fc_a1;
}

template <int S>
__device__ __forceinline__ uint16_t* stage_w() {
    static_assert(S >= 0 && S < kFcWStages, "stage index");
    if constexpr (S == 0) return fc_w0;
    else if constexpr (S == 1) return fc_w1;
    else return fc_w2;
}

// The epilogue's staging area of wave w: one stage array per wave (each
// holds at least a wave's 128 x 72 staging tile).
__device__ __forceinline__ uint16_t* epi_region(int w) {
    uint16_t* p = stage_a<0>();
    if (w == 1) p = stage_a<1>();
    if (w == 2) p = stage_w<0>();
    if (w == 3) p = stage_w<1>();
    if constexpr (kFcWStages > 2) if (w == 4) p = stage_w<2 % kFcWStages>();
    return p;
}

// Slot of 16-byte chunk c in LDS row r. A fragment read takes one chunk
// from each of 16 consecutive rows per LDS cycle; the swizzle spreads them
// over all 64 banks.
__device__ __forceinline__ int chunk_slot(int r, int c) {
    if constexpr (kFcChunks == 4) return c ^ ((r >> 2) & 3);
    else return c ^ ((r >> 1) & 7);
}

// The block of kFcCopyRows LDS rows that copy i of a wave fills, in the
// combined row space (token rows [0, kFcRowsA), then gate and up rows):
// copies [0, kFcCopiesA) take token rows and the rest weight rows, and the
// waves interleave block by block.
__device__ __forceinline__ int copy_block(int i, int wave) {
    if (i < kFcCopiesA) return i * kFcWaves + wave;
    return kFcRowsA / kFcCopyRows + (i - kFcCopiesA) * kFcWaves + wave;
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

// One copy: 16 bytes per lane of tile t, from the lane's source into the
// 1 KiB block of LDS at dst.
__device__ __forceinline__ void copy_one(const Sources& src, int i, int t, uint16_t* dst) {
#if SWIGLU_FC_SADDR
    const int64_t tb = (int64_t)t * kFcTileK * 2;                  // the tile's byte offset
    // (the offset is made opaque in place, so that the compiler neither
    // folds base and offset into one loop-invariant vector pointer nor
    // copies the offset into a scratch register for each copy)
    asm volatile("" : "+v"(src.off[i]));
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.base[i] + tb + src.off[i]),
                                     (lds_void*)(dst), 16, 0, SWIGLU_FC_CPOL);
#else
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.p[i] + (int64_t)t * kFcTileK),
                                     (lds_void*)(dst), 16, 0, SWIGLU_FC_CPOL);
#endif
}

// Starts token copies [I0, I1) of k tile t into token stage S.
template <int S, int I0 = 0, int I1 = kFcCopiesA>
__device__ __forceinline__ void copy_a(const Sources& src, int t) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = I0; i < I1; ++i)
        copy_one(src, i, t, stage_a<S>() + copy_block(i, wave) * kFcCopyRows * kFcRowElems);
}

// Starts weight copies [I0, I1) (counted among the weight copies) of k tile
// t into weight stage S.
template <int S, int I0 = 0, int I1 = kFcCopiesW>
__device__ __forceinline__ void copy_w(const Sources& src, int t) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = I0; j < I1; ++j) {
        const int q = copy_block(kFcCopiesA + j, wave) - kFcRowsA / kFcCopyRows;
        copy_one(src, kFcCopiesA + j, t, stage_w<S>() + q * kFcCopyRows * kFcRowElems);
    }
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
template <int SA, int SW>
__device__ __forceinline__ void load_frags(int wt, int wf, int off, Frags& F) {
    const uint16_t* ta = stage_a<SA>();
    const uint16_t* tw = stage_w<SW>();
#pragma unroll
    for (int j = 0; j < kFcMT; ++j) F.a[j] = frag(ta + (wt + 32 * j) * kFcRowElems + off);
#pragma unroll
    for (int i = 0; i < kFcMF; ++i) {
        F.g[i] = frag(tw + (wf + 32 * i) * kFcRowElems + off);
        F.u[i] = frag(tw + (kFcTileF + wf + 32 * i) * kFcRowElems + off);
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
// in LDS rows of 72 bf16 (144 bytes, 16-byte aligned rows), in the stage
// arrays once the k loop is done: kEpiPer regions per array.
constexpr int kEpiPitch = kFcWaveF + 8;
constexpr int kEpiRegion = kFcWaveT * kEpiPitch;
constexpr int kEpiPer = kFcAElems / kEpiRegion;      // (token and weight stages are the same size)
static_assert(kFcAElems == kFcWElems, "stage arrays of one size");
static_assert(!SWIGLU_FC_LDS_EPI ||
                  (kEpiPer >= 1 && (kFcWaves + kEpiPer - 1) / kEpiPer <= kFcAStages + kFcWStages),
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
#if SWIGLU_FC_NT_EPI
        if (tok < m && f < n) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + tok * ld + f));
#else
        if (tok < m && f < n) *reinterpret_cast<u32x4*>(out + tok * ld + f) = v;
#endif
    }
}

struct Ctx {
    Sources src;
    int wt, wf;
    int off[kFcSteps];   // this lane's fragment offset in each k step
    int kt_count;        // k tiles
    int pad;             // slots skipped at the start so that the slot count is a whole
                         // number of periods: real tile t is slot t + pad
};

// Source tile of slot kt; slots past the end are clamped to the last tile
// (their copies land in stages that are never multiplied in).
__device__ __forceinline__ int source_tile(const Ctx& c, int kt) {
    const int t = kt - c.pad;
    return t < 0 ? 0 : t < c.kt_count ? t : c.kt_count - 1;
}

#ifndef SWIGLU_FC_COPY_POS
#define SWIGLU_FC_COPY_POS 9    // strict schedule: MFMA index after which a step's first copy goes
#endif
#ifndef SWIGLU_FC_COPY_STRIDE
#define SWIGLU_FC_COPY_STRIDE 2 // ... and the MFMAs between two copies
#endif
#ifndef SWIGLU_FC_COPY_POS0
#define SWIGLU_FC_COPY_POS0 SWIGLU_FC_COPY_POS   // ... for step 0's copies
#endif
#ifndef SWIGLU_FC_COPY_POS3
#define SWIGLU_FC_COPY_POS3 1   // SPLIT 3: positions of the token copies after the barrier
#endif
#ifndef SWIGLU_FC_COPY_STRIDE3
#define SWIGLU_FC_COPY_STRIDE3 2
#endif
#ifndef SWIGLU_FC_READ_STRIDE
#define SWIGLU_FC_READ_STRIDE 1 // strict schedule: MFMAs between two fragment reads (from MFMA 0)
#endif

// One k step in a fixed instruction order (SWIGLU_FC_SCHED 2): MFMA m of
// the step (the order of mfma_step), then, at their positions, one fragment
// read of the next step into N and one copy (copy(q) issues the step's copy
// q), with a scheduling barrier after every group so that nothing moves.
template <int SA, int SW, int NC, int POS, int STRIDE, class CopyFn>
__device__ __forceinline__ void step_strict(const Ctx& c, int off, const Frags& C, Frags& N,
                                            Acc& acc, CopyFn copy) {
    static_assert(NC == 0 || POS + (NC - 1) * STRIDE < kFcMfma,
                  "every copy of the step has an MFMA to follow");
    static_assert((kFcReads - 1) * SWIGLU_FC_READ_STRIDE < kFcMfma, "every read has an MFMA to follow");
    const uint16_t* ta = stage_a<SA>();
    const uint16_t* tw = stage_w<SW>();
#pragma unroll
    for (int m = 0; m < kFcMfma; ++m) {
        const int i = m / (2 * kFcMT), j = (m / 2) % kFcMT;
        if (m & 1)
            acc.u[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.u[i], C.a[j], acc.u[i][j], 0, 0, 0);
        else
            acc.g[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(C.g[i], C.a[j], acc.g[i][j], 0, 0, 0);
        if (m % SWIGLU_FC_READ_STRIDE == 0 && m / SWIGLU_FC_READ_STRIDE < kFcReads) {
            const int r = m / SWIGLU_FC_READ_STRIDE;
            if (r < kFcMT) N.a[r] = frag(ta + (c.wt + 32 * r) * kFcRowElems + off);
            else if (r < kFcMT + kFcMF) N.g[r - kFcMT] = frag(tw + (c.wf + 32 * (r - kFcMT)) * kFcRowElems + off);
            else N.u[r - kFcMT - kFcMF] =
                     frag(tw + (kFcTileF + c.wf + 32 * (r - kFcMT - kFcMF)) * kFcRowElems + off);
        }
        if (m >= POS && (m - POS) % STRIDE == 0 && (m - POS) / STRIDE < NC) copy((m - POS) / STRIDE);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One k step of tile (SA, SW) with fragments C while the next step's are
// read into N.
template <int SA, int SW, int STEP>
__device__ __forceinline__ void inner_step(const Ctx& c, Frags& C, Frags& N, Acc& acc) {
    load_frags<SA, SW>(c.wt, c.wf, c.off[STEP + 1], N);
    mfma_step(C, acc);
    sched_reads_among_mfma();
}

// Copies that may still be in flight when slot kt + 1 must be complete: the
// token copies of slot kt + 1 were issued at the end of tile kt - 1, and
// with three weight stages only the weight copies issued by tile kt itself
// (of slot kt + 2) come after them.
constexpr int kWaitSlot = kFcWStages == 3 ? kFcCopiesW : 0;

// Slot kt at position J of the period: token stage J % A_STAGES, weight
// stage J % W_STAGES. Entering: F0 holds (or is receiving) the tile's first
// step's fragments; the token copies of slots up to kt + 1 and the weight
// copies of slots up to kt + W_STAGES - 2 are issued. Step 0 issues the
// weight copies of slot kt - 1 + W_STAGES into the weight stage that tile
// kt - 1 freed; steps 1 and 2 only compute; then wait for slot kt + 1 and
// barrier (every wave has read this tile's stages into registers), and step
// 3 issues the token copies of slot kt + A_STAGES into this tile's token
// stage while slot kt + 1's first fragments are read.
template <int J>
__device__ __forceinline__ void k_tile(const Ctx& c, int kt, Frags& F0, Frags& F1, Acc& acc) {
    constexpr int SA = J % kFcAStages, SW = J % kFcWStages;
    constexpr int SWP = (J + kFcPeriod - 1) % kFcWStages;     // tile kt - 1's weight stage
    constexpr int SAN = (J + 1) % kFcAStages, SWN = (J + 1) % kFcWStages;
#if SWIGLU_FC_SCHED == 2
    constexpr int SAP = (J + kFcPeriod - 1) % kFcAStages;     // tile kt - 1's token stage
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ta1 = source_tile(c, kt + 1), tw2 = source_tile(c, kt - 1 + kFcWStages);
    const int ta2 = source_tile(c, kt + kFcAStages);
    auto blk_a = [&](int i) { return copy_block(i, wave) * kFcCopyRows * kFcRowElems; };
    auto blk_w = [&](int j) {
        return (copy_block(kFcCopiesA + j, wave) - kFcRowsA / kFcCopyRows) * kFcCopyRows * kFcRowElems;
    };
    constexpr int P = SWIGLU_FC_COPY_POS, S = SWIGLU_FC_COPY_STRIDE;
#if SWIGLU_FC_SPLIT == 4
    constexpr int HA = kFcCopiesA / 2, HW = kFcCopiesW / 2;
    step_strict<SA, SW, HA, SWIGLU_FC_COPY_POS0, S>(c, c.off[1], F0, F1, acc, [&](int q) {
        copy_one(c.src, HA + q, ta1, stage_a<SAP>() + blk_a(HA + q));
    });
    step_strict<SA, SW, HW, P, S>(c, c.off[2], F1, F0, acc, [&](int q) {
        copy_one(c.src, kFcCopiesA + q, tw2, stage_w<SWP>() + blk_w(q));
    });
    step_strict<SA, SW, kFcCopiesW - HW, P, S>(c, c.off[3], F0, F1, acc, [&](int q) {
        copy_one(c.src, kFcCopiesA + HW + q, tw2, stage_w<SWP>() + blk_w(HW + q));
    });
    wait_copies_and_lds<kWaitSlot>();
    ring_barrier();
    step_strict<SAN, SWN, HA, P, S>(c, c.off[0], F1, F0, acc, [&](int q) {
        copy_one(c.src, q, ta2, stage_a<SA>() + blk_a(q));
    });
#elif SWIGLU_FC_SPLIT == 3
    // the weight copies over steps 0-2, all token copies after the barrier
    constexpr int W0 = (kFcCopiesW + 2) / 3, W1 = (kFcCopiesW + 1) / 3;
    step_strict<SA, SW, W0, P, S>(c, c.off[1], F0, F1, acc, [&](int q) {
        copy_one(c.src, kFcCopiesA + q, tw2, stage_w<SWP>() + blk_w(q));
    });
    step_strict<SA, SW, W1, P, S>(c, c.off[2], F1, F0, acc, [&](int q) {
        copy_one(c.src, kFcCopiesA + W0 + q, tw2, stage_w<SWP>() + blk_w(W0 + q));
    });
    step_strict<SA, SW, kFcCopiesW - W0 - W1, P, S>(c, c.off[3], F0, F1, acc, [&](int q) {
        copy_one(c.src, kFcCopiesA + W0 + W1 + q, tw2, stage_w<SWP>() + blk_w(W0 + W1 + q));
    });
    wait_copies_and_lds<kWaitSlot>();
    ring_barrier();
    step_strict<SAN, SWN, kFcCopiesA, SWIGLU_FC_COPY_POS3, SWIGLU_FC_COPY_STRIDE3>(
        c, c.off[0], F1, F0, acc, [&](int q) { copy_one(c.src, q, ta2, stage_a<SA>() + blk_a(q)); });
#else
#error "the strict schedule takes SWIGLU_FC_SPLIT 3 or 4"
#endif
#elif SWIGLU_FC_SPLIT == 4
    // one copy group per step: the second half of slot kt + 1's token
    // copies, the weight copies of slot kt - 1 + W_STAGES in two halves,
    // and after the barrier the first half of slot kt + 2's token copies
    constexpr int SAP = (J + kFcPeriod - 1) % kFcAStages;     // tile kt - 1's token stage
    constexpr int HA = kFcCopiesA / 2, HW = kFcCopiesW / 2;
    copy_a<SAP, HA, kFcCopiesA>(c.src, source_tile(c, kt + 1));
    load_frags<SA, SW>(c.wt, c.wf, c.off[1], F1);
    mfma_step(F0, acc);
    sched_mix_at<kFcCopiesA - HA>();
    copy_w<SWP, 0, HW>(c.src, source_tile(c, kt - 1 + kFcWStages));
    load_frags<SA, SW>(c.wt, c.wf, c.off[2], F0);
    mfma_step(F1, acc);
    sched_mix_at<HW>();
    copy_w<SWP, HW, kFcCopiesW>(c.src, source_tile(c, kt - 1 + kFcWStages));
    load_frags<SA, SW>(c.wt, c.wf, c.off[3], F1);
    mfma_step(F0, acc);
    sched_mix_at<kFcCopiesW - HW>();
    wait_copies_and_lds<kWaitSlot>();
    ring_barrier();
    copy_a<SA, 0, HA>(c.src, source_tile(c, kt + kFcAStages));
    load_frags<SAN, SWN>(c.wt, c.wf, c.off[0], F0);
    mfma_step(F1, acc);
    sched_mix_at<HA>();
#elif SWIGLU_FC_SPLIT == 2
    constexpr int SAP = (J + kFcPeriod - 1) % kFcAStages;     // tile kt - 1's token stage
    constexpr int HA = kFcCopiesA / 2, HW = kFcCopiesW / 2;
    copy_a<SAP, HA, kFcCopiesA>(c.src, source_tile(c, kt + 1));
    copy_w<SWP, 0, HW>(c.src, source_tile(c, kt - 1 + kFcWStages));
    load_frags<SA, SW>(c.wt, c.wf, c.off[1], F1);
    mfma_step(F0, acc);
    sched_mix_at<kFcCopiesA - HA + HW>();
    copy_w<SWP, HW, kFcCopiesW>(c.src, source_tile(c, kt - 1 + kFcWStages));
    load_frags<SA, SW>(c.wt, c.wf, c.off[2], F0);
    mfma_step(F1, acc);
    sched_mix_at<kFcCopiesW - HW>();
    inner_step<SA, SW, 2>(c, F0, F1, acc);
    wait_copies_and_lds<kWaitSlot>();
    ring_barrier();
    copy_a<SA, 0, HA>(c.src, source_tile(c, kt + kFcAStages));
    load_frags<SAN, SWN>(c.wt, c.wf, c.off[0], F0);
    mfma_step(F1, acc);
    sched_mix_at<HA>();
#else
    copy_w<SWP>(c.src, source_tile(c, kt - 1 + kFcWStages));
    load_frags<SA, SW>(c.wt, c.wf, c.off[1], F1);
    mfma_step(F0, acc);
    sched_mix_at<kFcCopiesW>();
    inner_step<SA, SW, 1>(c, F1, F0, acc);
    inner_step<SA, SW, 2>(c, F0, F1, acc);
    wait_copies_and_lds<kWaitSlot>();
    ring_barrier();
    copy_a<SA>(c.src, source_tile(c, kt + kFcAStages));
    load_frags<SAN, SWN>(c.wt, c.wf, c.off[0], F0);
    mfma_step(F1, acc);
    sched_mix_at<kFcCopiesA>();
#endif
}

// A whole period of slots from kt (a multiple of the period).
__device__ __forceinline__ void full_pass(const Ctx& c, int kt, Frags& F0, Frags& F1, Acc& acc) {
    k_tile<0>(c, kt, F0, F1, acc);
    k_tile<1 % kFcPeriod>(c, kt + 1, F0, F1, acc);
    if constexpr (kFcPeriod > 2) {
        k_tile<2 % kFcPeriod>(c, kt + 2, F0, F1, acc);
        k_tile<3 % kFcPeriod>(c, kt + 3, F0, F1, acc);
        k_tile<4 % kFcPeriod>(c, kt + 4, F0, F1, acc);
        k_tile<5 % kFcPeriod>(c, kt + 5, F0, F1, acc);
    }
}

// The first period: slots pad .. period - 1 (the same branch in every wave).
__device__ __forceinline__ void first_pass(const Ctx& c, Frags& F0, Frags& F1, Acc& acc) {
    if (c.pad <= 0) k_tile<0>(c, 0, F0, F1, acc);
    if (c.pad <= 1) k_tile<1 % kFcPeriod>(c, 1, F0, F1, acc);
    if constexpr (kFcPeriod > 2) {
        if (c.pad <= 2) k_tile<2 % kFcPeriod>(c, 2, F0, F1, acc);
        if (c.pad <= 3) k_tile<3 % kFcPeriod>(c, 3, F0, F1, acc);
        if (c.pad <= 4) k_tile<4 % kFcPeriod>(c, 4, F0, F1, acc);
        if (c.pad <= 5) k_tile<5 % kFcPeriod>(c, 5, F0, F1, acc);
    }
}

// Fill for a first slot P: token copies of slots P and P + 1, weight copies
// of slots P .. P + W_STAGES - 2 (slot P + W_STAGES - 1's are issued by tile
// P itself); wait for slot P, barrier, and read its first fragments.
template <int P>
__device__ __forceinline__ void prologue(const Ctx& c, Frags& F0) {
    copy_a<P % kFcAStages>(c.src, source_tile(c, P));
    copy_w<P % kFcWStages>(c.src, source_tile(c, P));
#if SWIGLU_FC_SPLIT == 2 || SWIGLU_FC_SPLIT == 4
    // the second half of slot P + 1's token copies is issued by tile P
    copy_a<(P + 1) % kFcAStages, 0, kFcCopiesA / 2>(c.src, source_tile(c, P + 1));
    if constexpr (kFcWStages == 3) copy_w<(P + 1) % kFcWStages>(c.src, source_tile(c, P + 1));
    wait_copies_and_lds<kFcCopiesA / 2 + (kFcWStages == 3 ? kFcCopiesW : 0)>();
#else
    copy_a<(P + 1) % kFcAStages>(c.src, source_tile(c, P + 1));
    if constexpr (kFcWStages == 3) copy_w<(P + 1) % kFcWStages>(c.src, source_tile(c, P + 1));
    wait_copies_and_lds<kFcCopiesA + (kFcWStages == 3 ? kFcCopiesW : 0)>();
#endif
    ring_barrier();
    load_frags<P % kFcAStages, P % kFcWStages>(c.wt, c.wf, c.off[0], F0);
}

// Dynamic tail. Under full load the XCDs run at clocks several percent
// apart, and the hardware deals the workgroups to them in turn, a fixed share
// each, so the fastest XCD idles while the slowest finishes. With a
// workspace, the first tiles of the launch order still go one per workgroup
// (tile blockIdx.x), but the last tiles form a pool that later workgroups
// take from as they start: those run wherever an XCD has room, so the faster
// XCDs take more of them. The grid holds more pool workgroups than pool
// tiles (the surplus finds the pool empty and ends at once).
// The pool is split into 8 queues, one per XCD, in the order the hardware
// would deal its tiles (pool tile p to queue p % 8); a workgroup takes from
// the queue of the XCD it runs on, so the tiles that an L2 serves at one
// time stay those of one workgroup per tile, and from the other queues once
// its own is empty. The workspace holds the 8 queue counters and a count of
// the pool workgroups that have taken their tile; the last of them sets all
// nine back to zero.
constexpr uint32_t kFcQueues = 8;
constexpr uint32_t kFcQueueStride = 32;            // 32-bit words between counters (128 bytes)
constexpr uint32_t kFcDoneWord = kFcQueues * kFcQueueStride;
constexpr size_t kFcWorkspaceBytes = (kFcQueues + 1) * kFcQueueStride * 4;

__device__ __forceinline__ uint32_t queue_len(uint32_t pool, uint32_t q) {
    return pool > q ? (pool - 1 - q) / kFcQueues + 1 : 0;
}

__device__ __forceinline__ uint32_t fetch_add_agent(uint32_t* p) {
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A pool tile (in [0, pool)) for a workgroup on XCD home: from its own queue,
// else from the first other queue that still has one; pool if none is left.
// A queue once found empty stays empty (its counter only grows).
__device__ uint32_t take_pool_tile(uint32_t* ws, uint32_t home, uint32_t pool) {
    for (uint32_t s = 0; s < kFcQueues; ++s) {
        const uint32_t q = (home + s) % kFcQueues;
        const uint32_t len = queue_len(pool, q);
        if (len == 0) continue;
        const uint32_t j = fetch_add_agent(ws + q * kFcQueueStride);
        if (j < len) return q + kFcQueues * j;
    }
    return pool;
}

// The XCD this wave runs on (hardware register XCC_ID, bits [3:0]).
__device__ __forceinline__ uint32_t xcd_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) % kFcQueues;
}

// Output tile b of the launch order: 256 tokens x 128 features of y.
__device__ __forceinline__ void fc1_tile(const Fc1Args& P, uint32_t b, uint32_t f_tiles,
                                         uint32_t t_tiles) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t ft, tt;
    tile_of(b, f_tiles, t_tiles, ft, tt);
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
    const int slots = (c.kt_count + kFcPeriod - 1) / kFcPeriod * kFcPeriod;
    c.pad = slots - c.kt_count;
    {
        // A fragment lane reads row lane % 32 of a 32-row tile and chunk
        // 2 s + lane / 32 in step s.
        const int frow = lane % 32;
#pragma unroll
        for (int st = 0; st < kFcSteps; ++st)
            c.off[st] = frow * kFcRowElems + chunk_slot(frow, 2 * st + lane / 32) * 8;
    }

    Frags F0, F1;
    switch (c.pad) {
        case 0: prologue<0>(c, F0); break;
        case 1: prologue<1 % kFcPeriod>(c, F0); break;
        case 2: prologue<2 % kFcPeriod>(c, F0); break;
        case 3: prologue<3 % kFcPeriod>(c, F0); break;
        case 4: prologue<4 % kFcPeriod>(c, F0); break;
        default: prologue<5 % kFcPeriod>(c, F0); break;
    }
    first_pass(c, F0, F1, acc);
    for (int kt = kFcPeriod; kt < slots; kt += kFcPeriod) full_pass(c, kt, F0, F1, acc);
    // No copy may still be writing LDS when the stages are reused.
    wait_copies_and_lds<0>();

#if SWIGLU_FC_LDS_EPI
    // Epilogue through LDS (free now): every wave writes its tile of each
    // output into a private LDS region in registers' order, then reads it
    // back by rows, so each store instruction writes 8 rows of 128 bytes.
    ring_barrier();                                   // every wave is done with the stages
    uint16_t* region = epi_region(wave / kEpiPer) + (wave % kEpiPer) * kEpiRegion;
    const int64_t tw = t0 + c.wt, fw = f0 + c.wf;     // the wave's first token and feature
    epi_out(region, tw, fw, P.m, P.n, P.y, P.ldy, [&](int i, int j, int e) {
        const float g = acc.g[i][j][e];
        float sig, osig, scl;
        sigmoid_pair<uint16_t, false>(g, sig, osig, scl);
        return ((g * sig) * acc.u[i][j][e]) * scl;
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
                    float sig, osig, scl;
                    sigmoid_pair<uint16_t, false>(gv[r], sig, osig, scl);
                    yv[r] = ((gv[r] * sig) * uv[r]) * scl;
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

// Workgroups below n_fixed compute tile blockIdx.x. The others (only with a
// workspace) each take one tile of the pool [n_fixed, total) through the
// queues in ws, which are all zero on entry and all zero again on exit.
__global__ __launch_bounds__(kFcThreads) void swiglu_fc1_kernel(Fc1Args P, uint32_t f_tiles,
                                                                uint32_t t_tiles, uint32_t* ws,
                                                                uint32_t n_fixed) {
    const uint32_t total = f_tiles * t_tiles;
    uint32_t b = blockIdx.x;
    if (b >= n_fixed) {
        // Thread 0 takes the tile and hands it to every wave through LDS
        // (stage memory, not yet in use).
        uint32_t* word = reinterpret_cast<uint32_t*>(stage_a<0>());
        if (threadIdx.x == 0) {
            const uint32_t pool = total - n_fixed;
            const uint32_t p = take_pool_tile(ws, xcd_id(), pool);
            *word = n_fixed + p;
            // Count this workgroup once its tile is taken. The last pool
            // workgroup to be counted has seen every other one take its
            // tile, so no counter is touched again in this launch: it
            // clears them for the next launch on this workspace.
            const uint32_t done = fetch_add_agent(ws + kFcDoneWord);
            if (done == gridDim.x - n_fixed - 1) {
                for (uint32_t q = 0; q <= kFcQueues; ++q)
                    __hip_atomic_store(ws + q * kFcQueueStride, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_copies_and_lds<63>();
        ring_barrier();
        b = __builtin_amdgcn_readfirstlane(*word);
        // every wave has read the word before any copy can land on it
        wait_copies_and_lds<63>();
        ring_barrier();
        if (b >= total) return;
    }
    fc1_tile(P, b, f_tiles, t_tiles);
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) size_t swiglu_fc1_workspace_size(void) {
    return kFcWorkspaceBytes;
}

__attribute__((visibility("default"))) swiglu_status swiglu_fc1_fwd(
    const void* a, int64_t lda, const void* w, int64_t ldw, void* y, int64_t ldy, void* x_out,
    int64_t ldx, int64_t m, int64_t n, int64_t k, swiglu_dtype dtype, void* workspace,
    hipStream_t stream) {
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
    if (workspace != nullptr) {
        if ((uintptr_t)workspace % 16 != 0) return SWIGLU_ERR_BAD_STRIDE;
        const swiglu_host::Span sw{(uintptr_t)workspace, (uintptr_t)workspace + kFcWorkspaceBytes};
        if (swiglu_host::spans_overlap(sw, swiglu_host::span_of(oa, m, k, 2)) ||
            swiglu_host::spans_overlap(sw, swiglu_host::span_of(ow, 2 * n, k, 2)) ||
            swiglu_host::spans_overlap(sw, swiglu_host::span_of(oy, m, n, 2)) ||
            (x_out != nullptr && swiglu_host::spans_overlap(sw, swiglu_host::span_of(ox, m, 2 * n, 2))))
            return SWIGLU_ERR_ALIASING;
    }
    // With a workspace, launches of at least 16 tiles per CU end on a pool
    // (a tile is one workgroup on one CU, whose LDS its stages fill).
    int64_t cus = 0;
    if (workspace != nullptr) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SWIGLU_ERR_HIP;
        cus = v;
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
    uint32_t t_tiles = 0, n_fixed = 0;
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    void* args[] = {&P, const_cast<uint32_t*>(&f_tiles), &t_tiles, &ws, &n_fixed};
    for (int64_t r0 = 0; r0 < m; r0 += rows_per_launch) {
        const int64_t mc = m - r0 < rows_per_launch ? m - r0 : rows_per_launch;
        P.a = static_cast<const uint16_t*>(a) + r0 * lda;
        P.y = static_cast<uint16_t*>(y) + r0 * ldy;
        P.x = x_out ? static_cast<uint16_t*>(x_out) + r0 * ldx : nullptr;
        P.m = mc;
        t_tiles = (uint32_t)((mc + kFcTileT - 1) / kFcTileT);
        const uint32_t tiles = f_tiles * t_tiles;
        const swiglu_host::Fc1Pool pool = swiglu_host::fc1_pool(tiles, cus, kFcThreads, SWIGLU_FC_POOL_DIV, SWIGLU_FC_SURPLUS_DIV);
        n_fixed = pool.n_fixed;
        const uint32_t grid = pool.grid;
        if (hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_fc1_kernel), dim3(grid),
                            dim3(kFcThreads), args, 0, stream) != hipSuccess)
            return SWIGLU_ERR_HIP;
    }
    return SWIGLU_OK;
}

}  // extern "C"
