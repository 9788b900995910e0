// Empirical streaming ceiling for the SwiGLU access patterns (measurement only,
// not part of the SwiGLU path). Same grid, lane mapping, 16-byte vectors and
// nontemporal hints as the wide SwiGLU kernels, with the arithmetic replaced by
// an XOR, so the time is what the memory system allows for that mix:
//   pattern 0 (forward mix):  read two half rows of x, write one row of y;
//   pattern 1 (backward mix): read two half rows of x and one row of dy,
//                             write two half rows of dx.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// nv: 16-byte vectors per half row; x rows are 2*nv vectors, y/dy rows nv.
__global__ __launch_bounds__(256) void mix_2r1w(const u32x4* x, u32x4* y, uint32_t nv) {
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= nv) return;
    const size_t r = blockIdx.y;
    const u32x4* xr = x + r * 2 * nv + c;
    st(y + r * nv + c, ld(xr) ^ ld(xr + nv));
}

__global__ __launch_bounds__(256) void mix_3r2w(const u32x4* dy, const u32x4* x, u32x4* dx,
                                                uint32_t nv) {
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    if (c >= nv) return;
    const size_t r = blockIdx.y;
    const u32x4* xr = x + r * 2 * nv + c;
    const u32x4 a = ld(xr), b = ld(xr + nv), d = ld(dy + r * nv + c);
    u32x4* o = dx + r * 2 * nv + c;
    st(o, a ^ d);
    st(o + nv, b ^ d);
}

}  // namespace

extern "C" {

// Returns 0 on a successful launch, -1 on bad arguments, 1 on a launch error.
// rows <= 65535 (one launch); buffers must hold the extents described above.
__attribute__((visibility("default"))) int stream_ceiling_launch(
    int pattern, const void* x, const void* dy, void* out, int64_t rows, int64_t nv,
    hipStream_t stream) {
    if (rows <= 0 || rows > 65535 || nv <= 0 || nv > (int64_t)UINT32_MAX - 256 || !x || !out)
        return -1;
    if (((uintptr_t)x | (uintptr_t)out | (uintptr_t)dy) % 16) return -1;
    const dim3 grid((uint32_t)((nv + 255) / 256), (uint32_t)rows), block(256);
    const uint32_t v = (uint32_t)nv;
    if (pattern == 0) {
        hipLaunchKernelGGL(mix_2r1w, grid, block, 0, stream, (const u32x4*)x, (u32x4*)out, v);
    } else if (pattern == 1) {
        if (!dy) return -1;
        hipLaunchKernelGGL(mix_3r2w, grid, block, 0, stream, (const u32x4*)dy, (const u32x4*)x,
                           (u32x4*)out, v);
    } else {
        return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
