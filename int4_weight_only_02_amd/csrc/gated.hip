// gated.hip -- the gated activation of a gate/up projection pair for large M:
// Y = silu(gate) * up, elementwise from the two projections' fp32 outputs.  (For
// M <= 64 the small-M kernel applies the same function in its epilogue, with both
// tiles of a column pair in one workgroup, so neither output reaches memory.)
// Memory-bound: one thread takes four consecutive outputs (16-byte loads of each
// input, one 8- or 16-byte store).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

__global__ __launch_bounds__(256) void silu_mul_kernel(const float *G, const float *U, long long n4, void *Y,
                                                       int y_f32)
{
    const long long step = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += step) {
        const f32x4_t g = ((const f32x4_t *)G)[i];
        const f32x4_t u = ((const f32x4_t *)U)[i];
        f32x4_t y;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            y[r] = silu_f32(g[r]) * u[r];
        if (y_f32) {
            ((f32x4_t *)Y)[i] = y;
        } else {
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
            const u32x2_t o = {(uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16),
                               (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16)};
            ((u32x2_t *)Y)[i] = o;
        }
    }
}

} // namespace

hipError_t launch_silu_mul(const float *G, const float *U, long long n, void *Y, int y_f32, hipStream_t stream)
{
    const long long n4 = n / 4;
    long long blocks = (n4 + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (blocks < 1)
        return hipSuccess;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, G, U, n4, Y, y_f32);
    return hipGetLastError();
}

} // namespace w4a16
