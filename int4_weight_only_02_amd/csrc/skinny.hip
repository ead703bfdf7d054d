// skinny.hip -- W4A16 linear for small M (decode, draft-block verification) on gfx950,
// and the fused lm_head greedy-verify epilogue.
//
// At M <= 16 per m-block the layer is bound by HBM: every packed weight byte is
// read once and used for at most 16 rows.  The kernel streams the packed words
// with 128-bit loads straight into MFMA B fragments (no LDS staging of weights):
//   * one wave owns a 16-column tile; lane l holds column l%16 and, per group of
//     128 codes, one 16-byte load = 32 codes = the B operand of four
//     v_mfma_f32_16x16x32_bf16 (lane group l/16 covers codes 32*(l/16) .. +31);
//   * the activations of the workgroup's K range sit in LDS, permuted to the
//     fragment order, shared by the 8 waves (8 column tiles = a 128-column block);
//   * per group, the four MFMAs give P = sum x * (128 + q) exactly in fp32, and
//     the group is folded in fp32 as acc += s * (P - (128 + z) * sum x).
// Work is split stream-K style: units (m-block, column block, group) in that
// order are cut into one contiguous range per workgroup, so every shape spreads
// evenly over the 256 CUs whatever its N and K.  A column block shared by
// several workgroups is summed by the last to finish, in workgroup order, from
// fp32 partials in the workspace: results are deterministic.
//
// lm_head mode (the pages' greedy verifier: Pith review, Assumptions, "a correct
// verifier is lossless"; draft blocks of 16 tokens, free parameters) keeps the
// fp32 logits, folds each finished column into a per-row (value, column) key,
// reduces the keys with 64-bit atomic max (ties -> lowest column), and the last
// workgroup turns them into argmax ids and the accepted-prefix length.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockCols = kWaves * 16;     // columns per column block
constexpr int kSlotFloats = 16 * kBlockCols; // one fp32 partial: 16 rows x 128 columns
constexpr int kInner = 8;                    // groups whose weights are loaded together
constexpr int kCUs = 256;
constexpr size_t kLdsBudget = 160 * 1024 - 2048;

__device__ __forceinline__ long long unit_start(long long U, int grid, int w)
{
    return (long long)w * U / grid;
}

__device__ __forceinline__ int unit_owner(long long U, int grid, long long u)
{
    int w = (int)((u * grid) / U);
    while (w + 1 < grid && unit_start(U, grid, w + 1) <= u)
        ++w;
    return w;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m)
{
    uint32_t lo = __shfl_xor((int)(uint32_t)v, m);
    uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b)
{
    return a > b ? a : b;
}

__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kThreads) void skinny_kernel(SkinnyArgs a, SkinnyPlan p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ unsigned long long red[kWaves][16];
    __shared__ int s_first, s_last_w;

    const int M = a.M, N = a.N, K = a.K, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 4, col = lane & 15;
    const int w = blockIdx.x;
    const long long U = p.units;
    const int grid = p.grid, ncb = p.ncb, chunk = p.chunk;
    const long long u0 = unit_start(U, grid, w), u1 = unit_start(U, grid, w + 1);
    const int mrows = M < 16 ? M : 16;

    u32x4_t *xs = (u32x4_t *)smem;                                       // [g][chunk c][row]
    float *ssum = (float *)(smem + (size_t)chunk * 256 * mrows);        // [g][16]
    uint32_t *ticket = (uint32_t *)(a.ws + kOffTicket);
    unsigned long long *keys = (unsigned long long *)(a.ws + kOffKeys);
    uint32_t *counters = (uint32_t *)(a.ws + kOffCounters);
    float *partial = (float *)(a.ws + p.off_partial);

    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
    int cur_mb = -1;
    int st_mb = -1, st_c0 = 0, st_c1 = 0; // X groups [st_c0, st_c1) of m-block st_mb are in LDS

    auto flush_best = [&](int mb) {
        // reduce (value, column) keys over the 16 columns of each wave, then the waves
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            best[r] = max_u64(best[r], shfl_xor_u64(best[r], 1));
            best[r] = max_u64(best[r], shfl_xor_u64(best[r], 2));
            best[r] = max_u64(best[r], shfl_xor_u64(best[r], 4));
            best[r] = max_u64(best[r], shfl_xor_u64(best[r], 8));
        }
        if (col == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[wave][4 * h + r] = best[r];
        }
        __syncthreads();
        if (tid < 16 && mb * 16 + tid < M) {
            unsigned long long k = red[0][tid];
#pragma unroll
            for (int v = 1; v < kWaves; ++v)
                k = max_u64(k, red[v][tid]);
            if (k)
                atomicMax(&keys[mb * 16 + tid], k);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r)
            best[r] = 0ull;
    };

    long long u = u0;
    while (u < u1) {
        const long long per_mb = (long long)ncb * G;
        const int mb = (int)(u / per_mb);
        const long long rem = u - (long long)mb * per_mb;
        const int cb = (int)(rem / G);
        const int ga = (int)(rem - (long long)cb * G);
        const int gb = (int)((long long)G < ga + (u1 - u) ? (long long)G : ga + (u1 - u));
        const int m0 = mb * 16;
        const int Mb = M - m0 < 16 ? M - m0 : 16;
        const int ntile = cb * kBlockCols + wave * 16;
        const int n = ntile + col;
        const bool tile_live = ntile < N; // wave-uniform
        const int nl = n < N ? n : N - 1; // clamped row for loads; never stored

        if (a.lmhead && mb != cur_mb) {
            if (cur_mb >= 0)
                flush_best(cur_mb);
            cur_mb = mb;
        }

        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = ga; c0 < gb; c0 += chunk) {
            const int c1 = gb < c0 + chunk ? gb : c0 + chunk;
            if (!(mb == st_mb && c0 >= st_c0 && c1 <= st_c1)) {
                // stage X[m0 .. m0+Mb)[groups c0 .. c1) into LDS in fragment order,
                // with the per-(row, group) sums S used by the fold
                __syncthreads();
                const int ng = c1 - c0;
                const int total = Mb * ng * 16; // multiple of 16: one 16-lane team per (row, group)
                for (int i = tid; i < total; i += kThreads) {
                    const int c = i & 15;
                    const int t = i >> 4;
                    const int gl = t % ng;
                    const int m = t / ng;
                    const u32x4_t v = *(const u32x4_t *)(a.X + (size_t)(m0 + m) * K +
                                                         (size_t)(c0 + gl) * kGroup + c * 8);
                    float s = sum8_bf16(v);
                    s += __shfl_xor(s, 1);
                    s += __shfl_xor(s, 2);
                    s += __shfl_xor(s, 4);
                    s += __shfl_xor(s, 8);
                    if (c == 0)
                        ssum[gl * 16 + m] = s;
                    xs[(gl * 16 + c) * Mb + m] = x_permute8(v);
                }
                __syncthreads();
                st_mb = mb;
                st_c0 = c0;
                st_c1 = c1;
            }
            if (tile_live) {
                const u32x4_t *wrow = (const u32x4_t *)(a.qw + (size_t)nl * (K / 8)) + h;
                const uint16_t *srow = a.scales + (size_t)nl * G;
                const uint32_t *zrow = a.qz + (size_t)(nl >> 3) * G;
                const int zsh = (nl & 7) * 4;
                for (int g = c0; g < c1; g += kInner) {
                    u32x4_t wv[kInner];
                    uint32_t sv[kInner], zv[kInner];
#pragma unroll
                    for (int i = 0; i < kInner; ++i) {
                        if (g + i < c1) {
                            wv[i] = wrow[4 * (g + i)];
                            sv[i] = srow[g + i];
                            zv[i] = zrow[g + i];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < kInner; ++i) {
                        if (g + i < c1) {
                            const int gl = g + i - st_c0;
                            f32x4_t pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                u32x4_t xa = {0u, 0u, 0u, 0u};
                                if (col < Mb)
                                    xa = xs[(gl * 16 + 4 * h + j) * Mb + col];
                                const uint32_t wj = j == 0 ? wv[i].x : j == 1 ? wv[i].y : j == 2 ? wv[i].z : wv[i].w;
                                pacc = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xa), codes_to_frag(wj), pacc);
                            }
                            const float s = f16_bits_to_f32((uint16_t)sv[i]);
                            const float cz = (float)(kCodeBias + ((zv[i] >> zsh) & 15u));
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if (r < Mb) {
                                    const float S = ssum[gl * 16 + 4 * h + r];
                                    acc[r] = fmaf(s, fmaf(-cz, S, pacc[r]), acc[r]);
                                }
                            }
                        }
                    }
                }
            }
        }

        // ---- epilogue: finish the column block (directly, or by the last contributor)
        bool have = true;
        if (!(ga == 0 && gb == G)) {
            const int slot = (u == u0) ? 0 : 1;
            float *part = partial + ((size_t)w * 2 + slot) * kSlotFloats;
            if (tile_live) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * h + r < Mb)
                        st_agent(&part[(4 * h + r) * kBlockCols + wave * 16 + col], acc[r]);
            }
            __threadfence();
            __syncthreads();
            if (tid == 0) {
                const long long ub = ((long long)mb * ncb + cb) * G;
                const int wf = unit_owner(U, grid, ub);
                const int wl = unit_owner(U, grid, ub + G - 1);
                const uint32_t old = atomicAdd(&counters[wf], 1u);
                s_first = (old == (uint32_t)(wl - wf)) ? wf : -1;
                s_last_w = wl;
                if (s_first >= 0)
                    __hip_atomic_store(&counters[wf], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            const int wf = s_first, wl = s_last_w;
            have = wf >= 0;
            if (have) {
                __threadfence();
                const long long ub = ((long long)mb * ncb + cb) * G;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] = 0.f;
                for (int v = wf; v <= wl; ++v) {
                    const int sl = unit_start(U, grid, v) < ub ? 1 : 0;
                    const float *pv = partial + ((size_t)v * 2 + sl) * kSlotFloats;
                    if (tile_live) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * h + r < Mb)
                                acc[r] += ld_agent(&pv[(4 * h + r) * kBlockCols + wave * 16 + col]);
                    }
                }
            }
        }
        if (have && tile_live && n < N) {
            if (a.Y) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 4 * h + r;
                    if (row < Mb) {
                        const size_t o = (size_t)(m0 + row) * N + n;
                        if (a.y_f32)
                            ((float *)a.Y)[o] = acc[r];
                        else
                            ((uint16_t *)a.Y)[o] = f32_to_bf16_rne(acc[r]);
                    }
                }
            }
            if (a.lmhead) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * h + r < Mb)
                        best[r] = max_u64(best[r], argmax_key(acc[r], n));
            }
        }
        u += gb - ga;
    }

    if (a.lmhead) {
        if (cur_mb >= 0)
            flush_best(cur_mb);
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = atomicAdd(ticket, 1u);
            s_first = (old == (uint32_t)(grid - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (s_first && tid < 64) {
            __threadfence();
            int am = 0;
            bool mism = false;
            if (tid < M) {
                const unsigned long long k =
                    __hip_atomic_load(&keys[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                am = key_col(k);
                a.argmax_out[tid] = am;
                __hip_atomic_store(&keys[tid], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                mism = am != a.draft[tid];
            }
            const unsigned long long b = __ballot(mism);
            if (tid == 0) {
                a.accept_out[0] = b ? (int32_t)(__ffsll((long long)b) - 1) : (int32_t)M;
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

} // namespace

static void set_chunk(SkinnyPlan &p, int M, size_t lds_limit)
{
    const int mrows = M < 16 ? M : 16;
    int chunk = (int)(lds_limit / ((size_t)mrows * 256 + 64));
    if (chunk > p.G)
        chunk = p.G;
    if (chunk < 1)
        chunk = 1;
    p.chunk = chunk;
    p.lds_bytes = (size_t)chunk * 256 * mrows + (size_t)chunk * 64;
}

SkinnyPlan plan_skinny(int M, int N, int K, int lmhead)
{
    (void)lmhead;
    SkinnyPlan p{};
    p.G = K / kGroup;
    p.mblocks = (M + 15) / 16;
    p.ncb = (N + kBlockCols - 1) / kBlockCols;
    p.units = (long long)p.mblocks * p.ncb * p.G;
    set_chunk(p, M, kLdsBudget);
    long long grid = kCUs;
    if (grid > p.units)
        grid = p.units;
    if (grid > kMaxGrid)
        grid = kMaxGrid;
    p.grid = (int)grid;
    p.off_partial = kZeroRegion;
    p.ws_bytes = p.off_partial + (size_t)p.grid * 2 * kSlotFloats * sizeof(float);
    return p;
}

hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &plan, hipStream_t stream)
{
    // LDS per workgroup: whatever the device allows, up to the budget the plan assumed
    static size_t lds_limit = 0;
    if (lds_limit == 0) {
        int dev = 0, v = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess)
            return e;
        size_t lim = (size_t)v > 2048 ? (size_t)v - 2048 : 0;
        lds_limit = lim < kLdsBudget ? lim : kLdsBudget;
        if (lds_limit > 64 * 1024)
            (void)hipFuncSetAttribute((const void *)skinny_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)lds_limit);
    }
    SkinnyPlan p = plan;
    if (p.lds_bytes > lds_limit)
        set_chunk(p, a.M, lds_limit);
    hipLaunchKernelGGL(skinny_kernel, dim3(p.grid), dim3(kThreads), p.lds_bytes, stream, a, p);
    return hipGetLastError();
}

} // namespace w4a16
