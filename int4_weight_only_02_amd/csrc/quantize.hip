// quantize.hip -- round a weight matrix back onto the packed grid, keeping the
// grid's scales and zero-points (gfx950).
//
// The pages' distillation keeps the INT4 grid's per-group scales fixed and rounds
// the trained weights back onto it, so the packed format and the serving path do
// not change (Pith review, Referee Report: Summary and Significance; Assumptions &
// free parameters, second assumption).  Reading (no formula on the pages):
//   q[n,k] = clamp(round(W[n,k] / s[n,g]) + z[n,g], 0, 15),  g = k / 128,
// round to nearest with ties to even, applied before z is added; the quotient is
// an IEEE binary32 division (the library is built with correctly rounded fp32
// division), so the code decided here is the same one an exact-arithmetic host
// reference takes in binary32.
// Elementwise and HBM-bound: one thread turns 8 consecutive weights of a row (one
// 16-byte load of bfloat16) into one packed word (the codes never exist unpacked);
// consecutive threads read consecutive 16 bytes and write consecutive words.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

__device__ __forceinline__ uint32_t round_to_code(float w, float s, float z)
{
    float r = __builtin_rintf(w / s) + z; // v_rndne: nearest, ties to even
    r = r >= 0.f ? r : 0.f;               // also maps NaN to 0 (r >= 0 is false)
    r = r <= 15.f ? r : 15.f;
    return (uint32_t)r;
}

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *W, const uint16_t *scales,
                                                       const uint32_t *qzeros, int N, int K, int G,
                                                       uint32_t *qweight)
{
    const long long KW = K / 8;
    const long long words = (long long)N * KW;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words; i += (long long)gridDim.x * 256) {
        const int n = (int)(i / KW);
        const int g = (int)((i - (long long)n * KW) / (kGroup / 8));
        const float s = f16_bits_to_f32(scales[(size_t)n * G + g]);
        const float z = (float)((qzeros[(size_t)(n >> 3) * G + g] >> (4 * (n & 7))) & 15u);
        const u32x4_t v = ((const u32x4_t *)W)[i]; // weights k = 8w .. 8w+7 (pairs, low half first)
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            word |= round_to_code(bf16_lo(d[j]), s, z) << (8 * j);
            word |= round_to_code(bf16_hi(d[j]), s, z) << (8 * j + 4);
        }
        qweight[i] = word;
    }
}

} // namespace

hipError_t launch_quantize(const uint16_t *W, const uint16_t *scales, const uint32_t *qzeros, int N, int K,
                           uint32_t *qweight, hipStream_t stream)
{
    const long long words = (long long)N * (K / 8);
    long long blocks = (words + 255) / 256;
    if (blocks > 16384)
        blocks = 16384;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, scales, qzeros, N, K,
                       K / kGroup, qweight);
    return hipGetLastError();
}

} // namespace w4a16
