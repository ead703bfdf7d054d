// common.h -- device helpers shared by the gfx950 W4A16 kernels.
//
// Operand encoding used by every kernel (derived from the grid definition in
// include/w4a16.h, not from the pages, which print no kernel):
//   * A 4-bit code q becomes the bf16 number 128 + q exactly by OR-ing it into
//     the mantissa of bf16 128.0 (0x4300): in [128, 256) a bf16 ulp is 1.
//     The MFMA then multiplies bf16 activations by these exact biased codes and
//     accumulates in fp32.  The bias and the zero-point come out per group:
//       sum_{k in g} x_k (q_k - z) = P_g - (128 + z) * S_g,
//       P_g = sum x_k (128 + q_k),  S_g = sum x_k,
//     and the group result is scaled by s in fp32.  Nothing is rounded before
//     the products, which keeps the kernels far inside the accuracy budget.
//   * One 32-bit word holds codes k0..k7 of one column (nibble j = k_j).  The
//     mask-and-or (w >> 4i) & 0x000F000F | 0x43004300 yields the bf16 pair
//     (k_i, k_{i+4}), so one word becomes the 8-element MFMA fragment in the
//     order k0 k4 k1 k5 k2 k6 k3 k7.  Activations are permuted the same way
//     (x_permute8), so the contraction pairs each code with its own x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kGroup = 128;
constexpr uint32_t kCodeBias = 128;           // bf16 value of 0x4300
constexpr uint32_t kBiasBits = 0x43004300u;   // two bf16 128.0 halves

// 8 codes of one word -> MFMA fragment (bf16 128+q), element order k0 k4 k1 k5 k2 k6 k3 k7
__device__ __forceinline__ bf16x8_t codes_to_frag(uint32_t w)
{
    u32x4_t r;
    r.x = (w & 0x000F000Fu) | kBiasBits;
    r.y = ((w >> 4) & 0x000F000Fu) | kBiasBits;
    r.z = ((w >> 8) & 0x000F000Fu) | kBiasBits;
    r.w = ((w >> 12) & 0x000F000Fu) | kBiasBits;
    return __builtin_bit_cast(bf16x8_t, r);
}

// 8 consecutive bf16 activations x0..x7 (4 dwords, little-endian pairs) ->
// the same order as codes_to_frag: x0 x4 x1 x5 x2 x6 x3 x7
// One byte permute per dword: v_perm_b32(hi, lo, sel) picks result byte i from the
// eight bytes lo (selectors 0..3) and hi (4..7).
__device__ __forceinline__ u32x4_t x_permute8(u32x4_t d)
{
    u32x4_t r;
    r.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u); // x0 x4
    r.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u); // x1 x5
    r.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u); // x2 x6
    r.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u); // x3 x7
    return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// sum of the 8 bf16 values held in 4 dwords, in a fixed order
__device__ __forceinline__ float sum8_bf16(u32x4_t d)
{
    float a = (bf16_lo(d.x) + bf16_hi(d.x)) + (bf16_lo(d.y) + bf16_hi(d.y));
    float b = (bf16_lo(d.z) + bf16_hi(d.z)) + (bf16_lo(d.w) + bf16_hi(d.w));
    return a + b;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// silu(g) = g * sigmoid(g) = g / (1 + e^-g), fp32 (e^-g by the hardware exp2; -inf
// at g -> -inf gives -0, large g gives g)
__device__ __forceinline__ float silu_f32(float g)
{
    return g / (1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Order-preserving map of an fp32 logit into a u32 (larger float -> larger u32).
__device__ __forceinline__ uint32_t order_f32(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax key: larger logit wins, equal logits -> the smaller column wins.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col)
{
    return ((unsigned long long)order_f32(v) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

__device__ __forceinline__ int key_col(unsigned long long key)
{
    return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
}

} // namespace w4a16
