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
//  * The grid is one-shot. Wide rows (at least 256 vectors per half row):
//    blockIdx.y picks a row and blockIdx.x a 256-vector column tile; row
//    offsets are uniform per block and live in scalar registers, and no lane
//    divides. Narrow rows: a flat 1D grid over the (row, vector) lanes, each
//    lane finding its row with one fp64 multiply, so no lane idles. Enough
//    blocks are in flight that HBM stays saturated (131072 blocks for
//    8192 x 32768 bf16).
//  * Loads and stores carry the nontemporal hint: nothing is re-read, and
//    keeping the stream out of the caches measured faster on large shapes.
//  * Arithmetic is kept short because at 16 bytes per lane the forward has
//    only ~29 VALU slots per element pair at 8 TB/s: bf16 uses one exp2 and
//    one reciprocal per element with no selects; fp32 (half the elements per
//    lane, same bytes) affords a compensated exponential and a series at the
//    root of silu' for its tighter tolerance. bf16 results are rounded once,
//    nearest-even, by the hardware convert.
#include "swiglu_device.h"

namespace {

using namespace swiglu_impl;

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
        float sig, osig, scl;
        sigmoid_pair<T, false>(g[i], sig, osig, scl);
        out[i] = ((g[i] * sig) * u[i]) * scl;
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
        float sig, osig, scl;
        sigmoid_pair<T, true>(g[i], sig, osig, scl);
        const float h = h_factor<T>(g[i], osig);
        // sigma h = silu'(g) is at most 1.1 in magnitude, so forming it first
        // leaves only the last multiply to round into the subnormal range
        du[i] = (d[i] * (g[i] * sig)) * scl;
        dg[i] = ((d[i] * u[i]) * (sig * h)) * scl;
    }
    Vec<T, VEC>::store(dgp + row * dgs + c, dg);
    Vec<T, VEC>::store(dup + row * dus + c, du);
}


// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
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
    if (P.rows_per_launch <= 0) return SWIGLU_ERR_BAD_SHAPE;   // n == 0 is never planned
    G.nv = P.nv;
    G.inv_nv = 1.0 / (double)P.nv;
    for (int64_t r0 = 0; r0 < rows; r0 += P.rows_per_launch) {
        const int64_t rc = rows - r0 < P.rows_per_launch ? rows - r0 : P.rows_per_launch;
        for (int i = 0; i < NOPS; ++i)
            ptr[i] = const_cast<T*>(static_cast<const T*>(ops[i].p)) + r0 * ops[i].stride;
        G.rows = rc;
        const dim3 grid = P.wide ? dim3(P.tiles, (uint32_t)rc)
                                 : dim3(swiglu_host::flat_blocks(rc, P.nv, kBlock), 1);
        const hipError_t e = hipLaunchKernel(kernel, grid, dim3(kBlock), args, 0, stream);
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
    const int vb = vec_bytes((int)esz, n, ops, 3);
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
    const int vb = vec_bytes((int)esz, n, ops, 5);
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
        case SWIGLU_ERR_SCRATCH_LIMIT:
            return "SWIGLU_ERR_SCRATCH_LIMIT: the problem needs more than the static scratch holds";
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
