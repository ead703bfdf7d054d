// tiled.hip -- W4A16 linear for large M (prefill) on gfx950: LDS-tiled bf16 MFMA.
//
// At M in the thousands the layer is bound by the matrix cores.  Each workgroup
// computes a 128 x 128 tile of Y with 4 waves (64 x 64 each, 4 x 4 MFMA tiles of
// 16 x 16).  K advances one group (128) at a time:
//   * the X tile [128 rows x 128 k] is staged in LDS in fragment order, the
//     packed weights [128 columns x 16 words] are staged raw (64 B per column);
//   * every wave turns its words into exact bf16 codes 128 + q in registers
//     (common.h) and runs 4 k-steps of v_mfma_f32_16x16x32_bf16 into a fresh
//     per-group accumulator P;
//   * the group is folded in fp32: acc += s * (P - (128 + z) * S), where
//     S[m, g] = sum_{k in g} X[m, k] comes from a small pre-pass (gsum_kernel).
// Nothing is rounded before the fp32 accumulation, so the result stays within a
// few fp32 ulps of the exact product.  Global loads for group g+1 are issued
// before the MFMAs of group g.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr int BM = 128, BN = 128, kThreads = 256;
constexpr int kWPad = 5; // 16-byte units per staged weight column (4 data + 1 pad)

// S^T[g][m] = sum of the 128 activations of row m in group g (fixed summation order)
__global__ __launch_bounds__(256) void gsum_kernel(const uint16_t *X, int M, int K, int G, float *gsumT)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x; // one 16-byte chunk each
    const long long total = (long long)M * G * 16;
    if (i >= total)
        return; // total is a multiple of 16, so whole 16-lane teams exit together
    const int c = (int)(i & 15);
    const long long t = i >> 4;
    const int g = (int)(t % G);
    const int m = (int)(t / G);
    const u32x4_t v = *(const u32x4_t *)(X + (size_t)m * K + (size_t)g * kGroup + c * 8);
    float s = sum8_bf16(v);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if (c == 0)
        gsumT[(size_t)g * M + m] = s;
}

__global__ __launch_bounds__(kThreads) void tiled_kernel(TiledArgs a, TiledPlan p)
{
    __shared__ u32x4_t xs[16 * BM];      // [chunk c][row]: 8 activations in fragment order
    __shared__ u32x4_t wsm[BN * kWPad];  // [column][quarter-group] packed words
    __shared__ __align__(16) float gs[BM];

    const int M = a.M, N = a.N, K = a.K, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 4, col = lane & 15;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const float *gsumT = (const float *)(a.ws + p.off_gsum);

    u32x4_t xr[8], wr[2];
    float gr = 0.f;

    auto load_group = [&](int g) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int u = tid + kThreads * i;
            const int row = m0 + (u >> 4);
            const int c = u & 15;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row < M)
                v = *(const u32x4_t *)(a.X + (size_t)row * K + (size_t)g * kGroup + c * 8);
            xr[i] = v;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + kThreads * i;
            int cn = n0 + (u >> 2);
            cn = cn < N ? cn : N - 1;
            wr[i] = *((const u32x4_t *)(a.qw + (size_t)cn * (K / 8)) + 4 * g + (u & 3));
        }
        if (tid < BM)
            gr = (m0 + tid < M) ? gsumT[(size_t)g * M + m0 + tid] : 0.f;
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_group(0);
    for (int g = 0; g < G; ++g) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int u = tid + kThreads * i;
            xs[(u & 15) * BM + (u >> 4)] = x_permute8(xr[i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int u = tid + kThreads * i;
            wsm[(u >> 2) * kWPad + (u & 3)] = wr[i];
        }
        if (tid < BM)
            gs[tid] = gr;
        __syncthreads();
        if (g + 1 < G)
            load_group(g + 1);

        float sc[4], cz[4];
        u32x4_t wb[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int cl = wn * 64 + nt * 16 + col;
            int cn = n0 + cl;
            cn = cn < N ? cn : N - 1;
            sc[nt] = f16_bits_to_f32(a.scales[(size_t)cn * G + g]);
            cz[nt] = (float)(kCodeBias + ((a.qz[(size_t)(cn >> 3) * G + g] >> ((cn & 7) * 4)) & 15u));
            wb[nt] = wsm[cl * kWPad + h];
        }

        f32x4_t P[4][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8_t bfr[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const uint32_t wj = ks == 0 ? wb[nt].x : ks == 1 ? wb[nt].y : ks == 2 ? wb[nt].z : wb[nt].w;
                bfr[nt] = codes_to_frag(wj);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, xs[(4 * h + ks) * BM + wm * 64 + mt * 16 + col]);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const f32x4_t cin = ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : P[mt][nt];
                    P[mt][nt] = mfma16x16x32(af, bfr[nt], cin);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const f32x4_t S = *(const f32x4_t *)&gs[wm * 64 + mt * 16 + 4 * h];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[mt][nt][r] = fmaf(sc[nt], fmaf(-cz[nt], S[r], P[mt][nt][r]), acc[mt][nt][r]);
        }
    }

#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int cn = n0 + wn * 64 + nt * 16 + col;
            if (cn >= N)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + mt * 16 + 4 * h + r;
                if (row < M) {
                    const size_t o = (size_t)row * N + cn;
                    if (a.y_f32)
                        ((float *)a.Y)[o] = acc[mt][nt][r];
                    else
                        ((uint16_t *)a.Y)[o] = f32_to_bf16_rne(acc[mt][nt][r]);
                }
            }
        }
}

} // namespace

TiledPlan plan_tiled(int M, int N, int K)
{
    TiledPlan p{};
    p.G = K / kGroup;
    p.tiles_m = (M + BM - 1) / BM;
    p.tiles_n = (N + BN - 1) / BN;
    p.off_gsum = kZeroRegion;
    p.ws_bytes = p.off_gsum + (size_t)p.G * M * sizeof(float);
    return p;
}

hipError_t launch_tiled(const TiledArgs &a, const TiledPlan &p, hipStream_t stream)
{
    const long long chunks = (long long)a.M * p.G * 16;
    hipLaunchKernelGGL(gsum_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, a.X, a.M, a.K, p.G,
                       (float *)(a.ws + p.off_gsum));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(tiled_kernel, dim3(p.tiles_n, p.tiles_m), dim3(kThreads), 0, stream, a, p);
    return hipGetLastError();
}

} // namespace w4a16
