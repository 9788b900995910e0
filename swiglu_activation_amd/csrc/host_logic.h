// Host-side argument logic of the SwiGLU library: operand views, overlap
// tests, access-width choice and launch planning. Plain C++ (no HIP), so it
// is also compiled on its own by the CPU tests.
#ifndef SWIGLU_HOST_LOGIC_H
#define SWIGLU_HOST_LOGIC_H

#include <stdint.h>

namespace swiglu_host {

// One [rows, width] operand: base pointer and row stride, both in elements.
struct Operand {
    const void* p;
    int64_t stride;
};

struct Span {
    uintptr_t lo, hi;   // [lo, hi) in bytes
};

inline Span span_of(Operand o, int64_t rows, int64_t width, int64_t esz) {
    const uintptr_t lo = (uintptr_t)o.p;
    return {lo, lo + (uintptr_t)(((rows - 1) * o.stride + width) * esz)};
}

inline bool spans_overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

inline __int128 floor_div(__int128 a, __int128 b) {   // b > 0
    __int128 q = a / b;
    if ((a % b != 0) && (a < 0)) q -= 1;
    return q;
}

// Do two [rows, wa] and [rows, wb] views share at least one byte?
// Exact when both have the same row stride (the case of views into one
// buffer, such as the two halves of a packed [rows, 2n] tensor): row i of A
// and row j of B intersect iff -WB < d + (j - i) s < WA, with d the byte
// offset of B from A, s the byte stride and WA, WB the byte widths, so the
// views overlap iff an integer k = j - i in [-(rows-1), rows-1] satisfies it.
// With different strides the answer is conservative (any overlap of the
// spans counts).
inline bool views_overlap(Operand a, int64_t wa, Operand b, int64_t wb, int64_t rows,
                          int64_t esz) {
    if (rows <= 0 || wa <= 0 || wb <= 0) return false;
    if (!spans_overlap(span_of(a, rows, wa, esz), span_of(b, rows, wb, esz))) return false;
    if (rows == 1 || a.stride != b.stride) return true;
    const __int128 s = (__int128)a.stride * esz;
    const __int128 d = (__int128)(uintptr_t)b.p - (__int128)(uintptr_t)a.p;
    const __int128 WA = (__int128)wa * esz, WB = (__int128)wb * esz;
    __int128 klo = floor_div(-WB - d, s) + 1;          // smallest k with d + k s > -WB
    __int128 khi = -floor_div(-(WA - d), s) - 1;       // largest k with d + k s < WA
    if (klo < -(__int128)(rows - 1)) klo = -(__int128)(rows - 1);
    if (khi > (__int128)(rows - 1)) khi = (__int128)(rows - 1);
    return klo <= khi;
}

// Largest per-lane access (16, 8, 4 or 2 bytes; at least one element) that
// every operand's base pointer and row stride are aligned to and that divides
// the row width of n elements, so that n / VEC vectors cover every column of
// every operand (the views of a two-tensor call may be padded rows of wider
// buffers, where n need not be a multiple of the widest access the pointers
// and strides allow).
inline int vec_bytes(int esz, int64_t n, const Operand* ops, int nops) {
    int b = 16;
    for (; b > esz; b >>= 1) {
        bool ok = ((n * esz) % b) == 0;
        for (int i = 0; i < nops; ++i)
            ok = ok && ((uintptr_t)ops[i].p % (uintptr_t)b) == 0 && ((ops[i].stride * esz) % b) == 0;
        if (ok) break;
    }
    return b;
}

// Launch plan for rows of n elements accessed VEC at a time (VEC divides n,
// as vec_bytes guarantees). Wide rows (at least `block` vectors per half
// row): a 2D grid of (column tile, row) blocks. Narrow rows: a flat 1D grid
// over the linear (row, vector) index space, so no lane idles except in the
// last block; one launch covers at most 2^31 lanes. A plan with nv == 0
// (n == 0, never launched) has rows_per_launch 0.
struct Plan {
    bool wide;
    uint32_t nv;                 // vectors per half row
    uint32_t tiles;              // wide: column tiles per row; narrow: 0
    int64_t rows_per_launch;
};

constexpr int64_t kFlatLanes = (int64_t)1 << 31;   // lanes per narrow launch, at most

inline Plan make_plan(int64_t n, int vec, uint32_t block, uint32_t max_grid_y) {
    Plan P;
    P.nv = (uint32_t)(n / vec);
    P.wide = P.nv >= block;
    P.tiles = P.wide ? (P.nv + block - 1) / block : 0u;
    if (P.nv == 0) P.rows_per_launch = 0;
    else P.rows_per_launch = P.wide ? (int64_t)max_grid_y : kFlatLanes / P.nv;
    return P;
}

// Blocks of `block` lanes for `rows` narrow rows of nv vectors.
inline uint32_t flat_blocks(int64_t rows, uint32_t nv, uint32_t block) {
    return (uint32_t)((rows * nv + block - 1) / block);
}

// fc1 launches: token rows per launch when n features are cut in tiles of
// tile_f and tokens in tiles of tile_t, on a 1D grid of f_tiles x t_tiles
// workgroups of `threads` work-items. The grid's work-item count stays below
// 2^32 and a launch takes at most max_t token tiles. 0 when not even one
// token tile fits (the caller rejects that n).
inline int64_t fc1_rows_per_launch(int64_t n, int64_t tile_f, int64_t tile_t, int64_t max_t,
                                   int64_t threads) {
    const int64_t f_tiles = (n + tile_f - 1) / tile_f;
    const int64_t max_wg = (((int64_t)1 << 32) - 1) / threads;
    int64_t t = f_tiles > 0 ? max_wg / f_tiles : max_t;
    if (t > max_t) t = max_t;
    return t * tile_t;
}

// fc1 launch with a tile pool: the first n_fixed of `tiles` tiles go one per
// workgroup, the rest form the pool, and the grid holds `grid` workgroups
// (grid - n_fixed of them take from the pool: a quarter more than its
// tiles). Only launches of at least 16 tiles per CU get a pool (cus <= 0:
// none); n_fixed is a multiple of 8 (the pool starts on a whole round of the
// 8 XCDs), and the grid's work-item count stays below 2^32, the surplus
// shrinking first.
struct Fc1Pool {
    uint32_t n_fixed, grid;
};

inline Fc1Pool fc1_pool(uint32_t tiles, int64_t cus, int64_t threads, uint32_t pool_div = 4,
                        uint32_t surplus_div = 4) {
    if (cus <= 0 || (int64_t)tiles < 16 * cus) return {tiles, tiles};
    // (pool_div, surplus_div: the pool is 1 / pool_div of the launch, and
    // the pool workgroups 1 + 1 / surplus_div times its tiles)
    const uint32_t n_fixed = tiles / 8 * 8 - tiles / pool_div / 8 * 8;
    const uint32_t pool = tiles - n_fixed;
    const int64_t max_wg = (((int64_t)1 << 32) - 1) / threads;
    int64_t grid = (int64_t)tiles + (pool + surplus_div - 1) / surplus_div;
    if (grid > max_wg) grid = max_wg;
    if (grid <= (int64_t)tiles) return {tiles, tiles};
    return {n_fixed, (uint32_t)grid};
}

}  // namespace swiglu_host

#endif  // SWIGLU_HOST_LOGIC_H
