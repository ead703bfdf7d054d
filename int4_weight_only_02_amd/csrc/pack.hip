// pack.hip -- put 4-bit codes and zero-points onto the packed grid (gfx950).
//
// The pages keep the AWQ grid and its packing unchanged when the target is
// re-packed after distillation (Pith review, Referee Report: Summary and
// Significance).  Layout (include/w4a16.h): eight codes per 32-bit word along
// K, low nibble first; eight zero-points per word along N.  HBM-bound, one pass.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

// 4 bytes b0..b3 (low nibbles) -> b0 | b1 << 4 | b2 << 8 | b3 << 12
__device__ __forceinline__ uint32_t squeeze4(uint32_t x)
{
    x &= 0x0F0F0F0Fu;
    x = (x | (x >> 4)) & 0x00FF00FFu;
    x = (x | (x >> 8)) & 0x0000FFFFu;
    return x;
}

// one thread: 16 code bytes (one 128-bit load) -> 2 packed words
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *codes, uint32_t *qweight, long long n16)
{
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long long)gridDim.x * 256) {
        const u32x4_t v = ((const u32x4_t *)codes)[i];
        uint2 o;
        o.x = squeeze4(v.x) | (squeeze4(v.y) << 16);
        o.y = squeeze4(v.z) | (squeeze4(v.w) << 16);
        ((uint2 *)qweight)[i] = o;
    }
}

// one thread per zero word (r, g): rows 8r .. 8r+7 of column g of zeros[N][G]
__global__ __launch_bounds__(256) void pack_zeros_kernel(const uint8_t *zeros, int N, int G, uint32_t *qzeros)
{
    const long long total = (long long)(N / 8) * G;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const long long r = i / G;
        const int g = (int)(i - r * G);
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            word |= (uint32_t)(zeros[(size_t)(8 * r + j) * G + g] & 15u) << (4 * j);
        qzeros[i] = word;
    }
}

} // namespace

hipError_t launch_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int G,
                       uint32_t *qweight, uint32_t *qzeros, hipStream_t stream)
{
    const long long n16 = (long long)N * K / 16;
    long long blocks = (n16 + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, qweight, n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_pack_zeros(zeros, N, G, qzeros, stream);
}

hipError_t launch_pack_zeros(const uint8_t *zeros, int N, int G, uint32_t *qzeros, hipStream_t stream)
{
    const long long nz = (long long)(N / 8) * G;
    long long zb = (nz + 255) / 256;
    if (zb > 4096)
        zb = 4096;
    if (zb == 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_zeros_kernel, dim3((unsigned)zb), dim3(256), 0, stream, zeros, N, G, qzeros);
    return hipGetLastError();
}

} // namespace w4a16
