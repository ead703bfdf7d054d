// quantize.hip -- round a weight matrix back onto the packed grid, keeping the
// grid's scales and zero-points (gfx950).
//
// The pages' distillation keeps the INT4 grid's per-group scales fixed and rounds
// the trained weights back onto it, so the packed format and the serving path do
// not change (Pith review, Referee Report: Summary and Significance; Assumptions &
// free parameters, second assumption).  Reading (no formula on the pages):
//   q[n,k] = clamp(round(W[n,k] / s[n,g]) + z[n,g], 0, 15),  g = k / 128,
// round = the exact quotient to the nearest integer, ties to even, applied before
// z is added.
// Elementwise and HBM-bound: one thread turns 8 consecutive weights of a row (one
// 16-byte load of bfloat16) into one packed word (the codes never exist unpacked);
// consecutive threads read consecutive 16 bytes and write consecutive words.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

// round(w / s) to the nearest integer, ties to even, of the exact quotient, without
// a division: r = rint(w * (1/s)) is the answer or its neighbour (v_rcp_f32 is good
// to 1 ulp, so the product is within 2^-22 relative of w / s), and the remainder
// e = w - r s is exact in one fma (w has 8 significant bits, s 11, and r s lies
// within 1.5 s of w) while |w / s| < 2^21; larger quotients are clamped anyway.
// |e| > s/2: step towards e; |e| = s/2 (a tie, s/2 is exact): step only if r is odd.
// Infinite or NaN w leaves e NaN and r as the product rounded: the clamp below maps
// +inf to 15, -inf and NaN to 0.
__device__ __forceinline__ uint32_t round_to_code(float w, float s, float rs, float z)
{
    float r = __builtin_rintf(w * rs);
    const float e = __builtin_fmaf(-r, s, w);
    const float ae = __builtin_fabsf(e), h = 0.5f * s;
    const bool odd = ((int)r & 1) != 0;
    if (ae > h || (ae == h && odd))
        r += e > 0.f ? 1.f : -1.f;
    r += z;
    r = r >= 0.f ? r : 0.f; // also maps NaN to 0 (r >= 0 is false)
    r = r <= 15.f ? r : 15.f;
    return (uint32_t)r;
}

// kWordsPerThread words per thread, all their loads issued before any is used (the
// kernel is bound by the weight bytes in flight, not by the arithmetic)
constexpr int kWordsPerThread = 2;

__device__ __forceinline__ uint32_t quantize_word(u32x4_t v, float s, float z)
{
    const float rs = __builtin_amdgcn_rcpf(s);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w}; // weights k = 8w .. 8w+7 (pairs, low half first)
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        word |= round_to_code(bf16_lo(d[j]), s, rs, z) << (8 * j);
        word |= round_to_code(bf16_hi(d[j]), s, rs, z) << (8 * j + 4);
    }
    return word;
}

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *W, const uint16_t *scales,
                                                       const uint32_t *qzeros, int N, int K, int G,
                                                       uint32_t *qweight)
{
    // word i = n * KW + w (row n, word w of the row); N * K <= 2^31 - 256, so i fits in
    // 32 bits: one 32-bit division per word gives the row, a shift the group
    const uint32_t KW = (uint32_t)(K / 8);
    const uint32_t words = (uint32_t)N * KW;
    const uint32_t step = gridDim.x * 256u;
    for (uint32_t i0 = blockIdx.x * 256u + threadIdx.x; i0 < words; i0 += step * kWordsPerThread) {
        u32x4_t v[kWordsPerThread];
        float sc[kWordsPerThread], zf[kWordsPerThread];
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            const uint32_t iu = i0 + u * step;
            const uint32_t i = iu < words ? iu : words - 1;
            const uint32_t n = i / KW;
            const uint32_t g = (i - n * KW) >> 4; // 16 words per group of 128
            v[u] = ((const u32x4_t *)W)[i];
            sc[u] = f16_bits_to_f32(scales[(size_t)n * G + g]);
            zf[u] = (float)((qzeros[(size_t)(n >> 3) * G + g] >> (4 * (n & 7))) & 15u);
        }
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            const uint32_t i = i0 + u * step;
            if (i < words)
                qweight[i] = quantize_word(v[u], sc[u], zf[u]);
        }
    }
}

} // namespace

hipError_t launch_quantize(const uint16_t *W, const uint16_t *scales, const uint32_t *qzeros, int N, int K,
                           uint32_t *qweight, hipStream_t stream)
{
    const long long words = (long long)N * (K / 8);
    long long blocks = (words + 256 * kWordsPerThread - 1) / (256 * kWordsPerThread);
    if (blocks > 8192)
        blocks = 8192;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, scales, qzeros, N, K,
                       K / kGroup, qweight);
    return hipGetLastError();
}

} // namespace w4a16
