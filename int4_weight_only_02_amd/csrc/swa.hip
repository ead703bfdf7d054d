// swa.hip -- causal sliding-window attention of a query block (the drafter's long-
// context lever: Pith review, Assumptions & free parameters, an SWA window of 1024 or
// 2048 tokens; inputs of up to 8192 tokens in the pages' Figure 1), gfx950.
//
// Reading (the pages give no kernel or formula): scaled-dot-product attention of the
// last M tokens of a context of T, query i at position p_i = T - M + i, over the keys
// p_i - window < j <= p_i (causal), or, in the block mode, over every key of the block
// (T - M <= j < T) and the context keys p_i - window < j < T - M (the drafter proposes
// a whole block at once: mlsanity index page, Builds on, block diffusion), with
// grouped key/value heads (head h reads head h / (Hq / Hkv)).  K is token-major [T][Hkv][D]; V is kept transposed [Hkv][D][T], so
// that both matrix products read 8 or 16 contiguous bytes per lane.
//
// Split over keys (flash-decoding): workgroup (chunk, kv head) has one wave per query
// head of the group; a wave computes, for its 16 query rows and the chunk's kChunk
// keys,
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16: keys are the rows, so each lane ends up
//                  with 4 keys of one query -- exactly what the second product needs)
//   m = row max, P = exp(S - m) (masked keys 0), l = row sum
//   O~ = P V      (P from registers as a pair of bf16 values hi + lo, P - hi rounded
//                  again, in two MFMAs: P enters to about 2^-17; V^T rows as the B
//                  operand)
// and writes (m, l, O~) of its chunk; swa_combine_kernel adds the chunks in order:
//   O = sum_c e^(m_c - m) O~_c / sum_c e^(m_c - m) l_c,  m = max_c m_c.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr int kD = 128;
constexpr int kChunk = 128;                  // keys per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kOob = 0xFFFFFF00u;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane from global memory (offset voff of r) into LDS at dst + 16 * lane
// (dst the same for the whole wave)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

__global__ __launch_bounds__(1024) void swa_partial_kernel(SwaArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunk = blockIdx.x, kv = blockIdx.y;
    const int grp = a.Hq / a.Hkv;
    const int head = kv * grp + wave;
    const int h4 = lane >> 4, col = lane & 15;
    const int j0 = a.j_lo + chunk * kChunk;

    const __amdgpu_buffer_rsrc_t rq = rsrc(a.Q, (uint32_t)((size_t)a.M * a.Hq * kD * 2));
    const __amdgpu_buffer_rsrc_t rk = rsrc(a.K, (uint32_t)((size_t)a.T * a.Hkv * kD * 2));
    const __amdgpu_buffer_rsrc_t rv = rsrc(a.Vt, (uint32_t)((size_t)a.Hkv * kD * a.t_stride * 2));

    // The chunk's keys and values, shared by the group's waves, arrive in LDS by DMA:
    //   Kl: 128 keys x 16 units of 16 bytes (8 d each), unit c of key k at c ^ (k & 15)
    //   Vl: 128 d    x 16 units (8 keys each),          unit c of row d at c ^ (d & 15)
    // so that the 16 lanes of a fragment read hit 16 different units.
    __shared__ __align__(16) unsigned char Kl[kChunk * kD * 2];
    __shared__ __align__(16) unsigned char Vl[kD * kChunk * 2];
    const int nwaves = blockDim.x >> 6;
    for (int ins = wave; ins < 2 * (kChunk * kD * 2 / 1024); ins += nwaves) {
        const int kv_part = ins >= kChunk * kD * 2 / 1024; // 0: keys, 1: values
        const int slot = (ins - kv_part * (kChunk * kD * 2 / 1024)) * 64 + lane; // 16-byte slot
        const int row = slot >> 4, unit = (slot & 15) ^ (row & 15);
        if (!kv_part) {
            const int j = j0 + row;
            const uint32_t off = j < a.T ? (uint32_t)((j * a.Hkv + kv) * kD + 8 * unit) * 2u : kOob;
            dma16(rk, Kl + (slot - lane) * 16, off);
        } else {
            const uint32_t off = (uint32_t)((kv * kD + row) * a.t_stride + j0 + 8 * unit) * 2u;
            dma16(rv, Vl + (slot - lane) * 16, off);
        }
    }

    // Q^T as the B operand: lane (col = query, h4) holds d = 32 s + 8 h4 .. +7
    u32x4_t qf[4];
    const uint32_t qoff = col < a.M ? (uint32_t)((col * a.Hq + head) * kD + 8 * h4) * 2u : kOob;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        qf[s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, 64u * s, 0));

    // S^T for the chunk: key tile t, lane (col = key 16 t + col, h4) as the A operand;
    // result lane l: keys 16 t + 4 h4 + r of query col
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): this wave's DMA and Q have landed
    __syncthreads();                    // and every wave's DMA
    constexpr int kTiles = kChunk / 16;
    f32x4_t st[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int key = 16 * t + col;
        u32x4_t kf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kf[s] = *(const u32x4_t *)(Kl + (key * 16 + ((4 * s + h4) ^ (key & 15))) * 16);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mfma(kf[s], qf[s], acc);
        st[t] = acc;
    }

    // mask, scale (in log2 units) and the row max of query col over the chunk
    const int p = a.T - a.M + col; // the query's position (rows col >= M are never stored)
    const float sc = a.scale * kLog2e;
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + 16 * t + 4 * h4 + r;
            const bool ok = j < a.T && (a.block ? (j >= a.T - a.M || j > p - a.window)
                                                : (j <= p && j > p - a.window));
            st[t][r] = ok ? st[t][r] * sc : -INFINITY;
            mx = fmaxf(mx, st[t][r]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
    const float base = mx == -INFINITY ? 0.f : mx; // a chunk with no key of this query
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            st[t][r] = __builtin_amdgcn_exp2f(st[t][r] - base);
            sum += st[t][r];
        }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);

    // O~ = P V: k-step = key tiles (2 u, 2 u + 1); lane h4 holds keys 4 h4 .. +3 of both,
    // so its V^T reads are two 8-byte runs per d column
    f32x4_t o[kD / 16];
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
        o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kTiles / 2; ++u) {
        // P = hi + lo: hi = bf16(P), lo = bf16(P - hi) (P - hi is exact in fp32)
        u32x4_t ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x4_t &src = st[2 * u + (e >> 1)];
            const float x0 = src[2 * (e & 1)], x1 = src[2 * (e & 1) + 1];
            const uint32_t h2 = pack_bf16x2(x0, x1);
            ph[e] = h2;
            pl[e] = pack_bf16x2(x0 - __uint_as_float(h2 << 16), x1 - __uint_as_float(h2 & 0xFFFF0000u));
        }
        const int ja = j0 + 32 * u + 4 * h4, jb = ja + 16;
        // V of keys at or past T (row padding, whatever it holds) is replaced by 0: their
        // weights are 0, and 0 * NaN would not be
        uint32_t keep[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = (e < 2 ? ja : jb) + 2 * (e & 1);
            keep[e] = (j < a.T ? 0x0000FFFFu : 0u) | (j + 1 < a.T ? 0xFFFF0000u : 0u);
        }
        // keys ja - j0 = 32 u + 4 h4 (.. +3) and + 16: half of unit 4 u + h4 / 2 and of unit
        // 4 u + 2 + h4 / 2 of row d
        const int ua = 4 * u + (h4 >> 1), ub = ua + 2, half = (h4 & 1) * 8;
#pragma unroll
        for (int dt = 0; dt < kD / 16; ++dt) {
            const int d = dt * 16 + col;
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
            const u32x2_t va = *(const u32x2_t *)(Vl + (d * 16 + (ua ^ (d & 15))) * 16 + half);
            const u32x2_t vb = *(const u32x2_t *)(Vl + (d * 16 + (ub ^ (d & 15))) * 16 + half);
            const u32x4_t vf = {va.x & keep[0], va.y & keep[1], vb.x & keep[2], vb.y & keep[3]};
            o[dt] = mfma(ph, vf, o[dt]);
            o[dt] = mfma(pl, vf, o[dt]);
        }
    }

    // partials: ml[chunk][head][q] = (m, l) in log2 units, part[chunk][head][q][d]
    const size_t slot = ((size_t)chunk * a.Hq + head) * 16;
    if (lane < 16) {
        a.ml[(slot + col) * 2] = mx;
        a.ml[(slot + col) * 2 + 1] = sum;
    }
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a.part[(slot + 4 * h4 + r) * kD + dt * 16 + col] = o[dt][r];
}

// O[i][h][:] from the chunks in order; one workgroup of kD threads per (i, h).  The
// chunks' (m, l) pairs go through LDS once (all loads in flight together), then each
// thread adds its column of the chunk partials in chunk order, eight loads at a time.
constexpr int kCombineMax = 1024; // chunks per query handled by one pass of the LDS table

__global__ __launch_bounds__(kD) void swa_combine_kernel(SwaArgs a, int chunks)
{
    __shared__ float sm[kCombineMax], sw[kCombineMax];
    __shared__ float red[kD / 64];
    const int i = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const int n = chunks < kCombineMax ? chunks : kCombineMax;
    float mx = -INFINITY;
    for (int c = d; c < n; c += kD) {
        sm[c] = a.ml[(((size_t)c * a.Hq + h) * 16 + i) * 2];
        mx = fmaxf(mx, sm[c]);
    }
    // workgroup max: within each wave, then across the two waves
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((d & 63) == 0)
        red[d >> 6] = mx;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kD / 64; ++w)
        m = fmaxf(m, red[w]);
    for (int c = d; c < n; c += kD) // weight of each chunk (0 for chunks without keys)
        sw[c] = sm[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[c] - m);
    __syncthreads();
    float num = 0.f, den = 0.f;
    int c = 0;
    for (; c + 8 <= n; c += 8) {
        float pv[8], lv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t slot = ((size_t)(c + u) * a.Hq + h) * 16 + i;
            pv[u] = a.part[slot * kD + d];
            lv[u] = a.ml[slot * 2 + 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            num += sw[c + u] * pv[u];
            den += sw[c + u] * lv[u];
        }
    }
    for (; c < n; ++c) {
        const size_t slot = ((size_t)c * a.Hq + h) * 16 + i;
        num += sw[c] * a.part[slot * kD + d];
        den += sw[c] * a.ml[slot * 2 + 1];
    }
    const float y = num / den;
    const size_t o = ((size_t)i * a.Hq + h) * kD + d;
    if (a.o_f32)
        ((float *)a.O)[o] = y;
    else
        ((uint16_t *)a.O)[o] = f32_to_bf16_rne(y);
}

} // namespace

SwaPlan plan_swa(int M, int T, int Hq, int Hkv, int window)
{
    SwaPlan p{};
    // the first key any query sees, rounded down to a multiple of 8 so that every V run
    // a lane reads is 8-byte aligned (the extra keys are masked)
    p.j_lo = T - M - window + 1 > 0 ? (T - M - window + 1) / 8 * 8 : 0;
    p.chunks = (T - p.j_lo + kChunk - 1) / kChunk;
    // the scratch starts past the zero region (argmax keys, tickets, arrival counters),
    // so an attention call never disturbs the counters the other calls expect at zero
    p.ml_off = kZeroRegion;
    p.part_off = p.ml_off + (size_t)p.chunks * Hq * 16 * 2 * sizeof(float);
    p.part_off = (p.part_off + 255) / 256 * 256;
    p.ws_bytes = p.part_off + (size_t)p.chunks * Hq * 16 * kD * sizeof(float);
    (void)Hkv;
    return p;
}

hipError_t launch_swa(SwaArgs a, const SwaPlan &p, unsigned char *ws, hipStream_t stream)
{
    a.j_lo = p.j_lo;
    a.ml = (float *)(ws + p.ml_off);
    a.part = (float *)(ws + p.part_off);
    const int grp = a.Hq / a.Hkv;
    hipLaunchKernelGGL(swa_partial_kernel, dim3(p.chunks, a.Hkv), dim3(64 * grp), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(swa_combine_kernel, dim3(a.M, a.Hq), dim3(kD), 0, stream, a, p.chunks);
    return hipGetLastError();
}

} // namespace w4a16
