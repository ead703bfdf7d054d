// gemv.hip -- W4A16 linear for a single activation row (M = 1, decode) on gfx950.
//
// The layer at M = 1 streams every packed byte once and uses it for one
// multiply-add, so the kernel is shaped around getting the whole stream in flight
// with as few load instructions as possible:
//
//   * A workgroup owns TC = 16 / PL adjacent columns (or TC = 5 with PL = 3, the 16th
//     lane column idle, where that makes the grid whole rounds of the CUs) and all of
//     K.  Its W waves split K: wave w takes the NG = GPW * PL groups from w * NG.  The grid is
//     N / TC small workgroups, so every CU holds many waves and all of its bytes
//     are requested at once; each lane issues GPW 128-bit code loads plus the
//     scale and zero word of each of its (column, group) pairs.
//   * Groups on the diagonal of one MFMA.  One v_mfma_f32_16x16x32_bf16 takes
//     sixteen A rows and sixteen B columns.  B column c + TC p holds the codes of
//     column c in group part p (lane (c + TC p, h) loads bytes 16h .. 16h+15 of
//     that group), and A row r holds X of group part r % PL, so D[4h + p][c + TC p]
//     is the dot product sum x * (128 + q) of column c over group part p (the other
//     products are discarded; the matrix cores have ample headroom here).
//   * X costs one load per lane per four groups: the wave loads its NG * 128
//     values as 8-value slots (slot s: group s / 16 of the wave), adds each group's
//     S = sum of X across the 16 lanes of a row, and parks the slots, permuted into
//     the fragment order, in its own LDS region; the MFMA A operands are read from
//     there.  No barrier precedes the contraction.
//   * The scale/zero fold runs per (column, group) in fp32:
//       y = sum_g s[g] * (P[g] - (128 + z[g]) * S[g]),
//     and the waves' partial sums meet in LDS, added in wave order.
//   * Act-order (GPTQ g_idx, stored permuted): the contraction needs X'[k] =
//     X[perm[k]].  The workgroup brings all of X into LDS by DMA, and each lane
//     gathers its slots from there through perm (one read per value); the rest is
//     unchanged, so the permuted copy of X never goes through HBM.
// All sums run in a fixed order: results are deterministic.
//
// The grid follows the pages' statement of the layer: packed uint4 codes with a
// per-group fp16 scale and a uint4 zero-point, group 128 (Pith review, Assumptions &
// free parameters: the drafter's GPTQ group size, act-order; Referee Report,
// Summary: the target's AWQ grid), and decode runs it at one row per step (mlsanity
// index page, Abstract: the drafter runs at every speculative decoding step).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr uint32_t kOobG = 0xFFFFFF00u; // an offset past the end of every tensor
constexpr int kRsrcWord3G = 0x00020000; // raw (untyped) buffer loads on gfx9-class GPUs
constexpr int kGemvMaxWaves = 16;
constexpr int kGemvMaxGroups = 12;      // groups per wave (NG)
constexpr int kGemvMaxLds = 64 * 1024;  // dynamic LDS without a per-kernel attribute

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_g(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3G);
}

__device__ __forceinline__ u32x4_t ld16_g(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS DMA: 16 bytes per lane from offset voff of r into LDS at dst + 16 * lane (dst
// the same for the whole wave); no registers involved
__device__ __forceinline__ void dma16_g(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

// sum over the 16 lanes of each lane row (quad swaps, then half-row and row mirrors);
// every lane of the row receives it
__device__ __forceinline__ float row_sum16(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// lane row 0 receives what lane row r (0..3) holds in v, column by column (the other
// rows receive other rows' values): a swap of rows 0 <-> 1 and 2 <-> 3, of the wave
// halves, or both
__device__ __forceinline__ uint32_t to_row0(uint32_t v, int r)
{
    if (r == 1)
        return __builtin_amdgcn_permlane16_swap(v, v, false, false)[1];
    if (r == 2)
        return __builtin_amdgcn_permlane32_swap(v, v, false, false)[1];
    if (r == 3) {
        const uint32_t x = __builtin_amdgcn_permlane32_swap(v, v, false, false)[1];
        return __builtin_amdgcn_permlane16_swap(x, x, false, false)[1];
    }
    return v;
}

// 8 codes -> MFMA fragment (bf16 128 + q), mask and bias held in registers
__device__ __forceinline__ bf16x8_t frag_r(uint32_t w, uint32_t mask, uint32_t bias)
{
    u32x4_t r;
    r.x = (w & mask) | bias;
    r.y = ((w >> 4) & mask) | bias;
    r.z = ((w >> 8) & mask) | bias;
    r.w = ((w >> 12) & mask) | bias;
    return __builtin_bit_cast(bf16x8_t, r);
}

// element p of v (p < PL)
template <int PL>
__device__ __forceinline__ float pick(f32x4_t v, int p)
{
    if constexpr (PL == 1)
        return v[0];
    else if constexpr (PL == 2)
        return p ? v[1] : v[0];
    else
        return (p & 2) ? ((p & 1) ? v[3] : v[2]) : ((p & 1) ? v[1] : v[0]);
}

// LDS layout (bytes): X slots [W][NG * 16] x 16, S [W][16] floats, wave partials
// [W][16] floats, then (act-order) X of the row, K bf16
__host__ __device__ constexpr int gemv_s_off(int W, int NG) { return W * NG * 256; }
__host__ __device__ constexpr int gemv_r_off(int W, int NG) { return W * NG * 256 + W * 64; }
__host__ __device__ constexpr int gemv_x_off(int W, int NG) { return W * NG * 256 + W * 128; }

// PAIR 1: a gated pair (the MLP's silu(x Wg^T) * (x Wu^T); Pith review, Referee Report,
// Summary): every wave loads the codes of the gate and of the up grid (qw2, scales2,
// qz2) for the same columns and groups, against the one slice of X, and the workgroup
// stores silu(gate) * up.  PAIR 2: the same two contractions, stored as they are (Y and
// Y2: a batch of two projections of one shape that read the same X).  Red then holds
// [W][2][16] partials.  PAIR 3: several projections of the same X and K in one launch
// (a.pr, a.count), each with its own run of workgroups; a workgroup finds its projection
// with one compare per entry and then works as a single launch would.
template <int GPW, int PL, bool AO, int PAIR = 0>
__global__ __launch_bounds__(64 * kGemvMaxWaves) void gemv_kernel(GemvArgs a)
{
    constexpr bool GATED = PAIR == 1, MULTI = PAIR == 3;
    static_assert(!(AO && PAIR), "the pairs have no act-order form");
    constexpr int TC = PL == 3 ? 5 : 16 / PL; // columns per workgroup
    constexpr int NG = GPW * PL;            // groups per wave
    constexpr int XR = NG / 4;              // X slots per lane
    static_assert(NG <= kGemvMaxGroups && NG % 4 == 0, "a lane row's slots hold one group");
    extern __shared__ __align__(16) unsigned char lds[];
    const int W = a.waves;
    const int G = a.G, K = a.K;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nid = lane & 15, h = lane >> 4;
    const int c = nid % TC, p = nid / TC;
    const bool plive = p < PL; // PL = 3: lane column 15 idle
    const uint32_t *qwp = a.qw, *qzp = a.qz;
    const uint16_t *sp = a.scales;
    void *Yp = a.Y;
    int N = a.N, bid = blockIdx.x;
    if constexpr (MULTI) {
        int q = 0;
#pragma unroll
        for (int j = 1; j < kMaxProblemsGemv; ++j)
            q += (j < a.count && bid >= a.pr[j].wg0) ? 1 : 0;
        const GemvArgs::Prob &pr = a.pr[q];
        qwp = pr.qw;
        sp = pr.scales;
        qzp = pr.qz;
        Yp = pr.Y;
        N = pr.N;
        bid -= pr.wg0;
    }
    const int n = bid * TC + c;
    const int g0 = w * NG;
    const uint32_t rowb = (uint32_t)(K / 2);
    u32x4_t *xs = (u32x4_t *)lds + w * NG * 16;             // this wave's X slots, fragment order
    float *Ss = (float *)(lds + gemv_s_off(W, NG)) + w * 16; // S of the wave's groups
    float *red = (float *)(lds + gemv_r_off(W, NG));         // [W][16] lane partials ([W][2][16] pairs)

    constexpr int NP = (PAIR == 1 || PAIR == 2) ? 2 : 1; // grids per wave: the first (gate), then the second (up)
    const __amdgpu_buffer_rsrc_t rw = rsrc_g(qwp, (uint32_t)N * rowb);
    const __amdgpu_buffer_rsrc_t rs = rsrc_g(sp, (uint32_t)N * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rz = rsrc_g(qzp, (uint32_t)(N / 8) * (uint32_t)G * 4u);
    const __amdgpu_buffer_rsrc_t rx = rsrc_g(a.X, (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t rw2 = NP == 2 ? rsrc_g(a.qw2, (uint32_t)N * rowb) : rw;
    const __amdgpu_buffer_rsrc_t rs2 = NP == 2 ? rsrc_g(a.scales2, (uint32_t)N * (uint32_t)G * 2u) : rs;
    const __amdgpu_buffer_rsrc_t rz2 = NP == 2 ? rsrc_g(a.qz2, (uint32_t)(N / 8) * (uint32_t)G * 4u) : rz;

    // 1. X: slot s = r * 64 + lane holds X'[(g0 + s / 16) * 128 + 8 (s % 16) .. + 8].
    //    Plain: one 16-byte load per slot.  Act-order: the row by DMA into LDS (every
    //    wave a share of it) and the slot's 8 entries of perm
    u32x4_t xv[XR];
    u32x4_t pv[AO ? XR : 1][2];
    unsigned char *xrow = lds + gemv_x_off(W, NG);
    if constexpr (AO) {
        const __amdgpu_buffer_rsrc_t rp = rsrc_g(a.perm, (uint32_t)K * 4u);
        const int xu = K / 8;
        for (int u0 = w * 64; u0 < xu; u0 += W * 64) {
            const int u = u0 + lane;
            dma16_g(rx, xrow + u0 * 16, u < xu ? 16u * (uint32_t)u : kOobG);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int slot = r * 64 + lane;
            const bool live = g0 * kGroup + slot * 8 < K;
            const uint32_t off = (uint32_t)(g0 * kGroup + slot * 8) * 4u;
            pv[r][0] = ld16_g(rp, live ? off : kOobG);
            pv[r][1] = ld16_g(rp, live ? off + 16u : kOobG);
        }
    } else {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int slot = r * 64 + lane;
            xv[r] = ld16_g(rx, g0 * kGroup + slot * 8 < K ? (uint32_t)(g0 * kGroup + slot * 8) * 2u : kOobG);
        }
    }
    asm volatile("" ::: "memory");

    // 2. the scale and zero word of the lane's column for instruction i = h (group
    //    g0 + h PL + p: lane row h loads what row 0 folds at instruction h, one load for
    //    all GPW instructions), then the codes: instruction i, lane (c + TC p, h) loads
    //    bytes 16h .. of group g0 + i PL + p of column n.  The small parameter loads go
    //    first, so that they do not queue behind the code loads
    static_assert(GPW <= 4, "one lane row per instruction");
    uint32_t sv[NP], zv[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int g = g0 + h * PL + p;
        const bool live = h < GPW && g < G && plive;
        // the offsets go through a register, so that the compiler keeps one unconditional
        // load each instead of a branch per case (whose register reuse could make the
        // second load wait for the load of X)
        uint32_t so = live ? ((uint32_t)n * (uint32_t)G + g) * 2u : kOobG;
        uint32_t zo = live ? ((uint32_t)(n >> 3) * (uint32_t)G + g) * 4u : kOobG;
        asm volatile("" : "+v"(so), "+v"(zo));
        sv[q] = __builtin_amdgcn_raw_buffer_load_b16(q ? rs2 : rs, so, 0, 0);
        zv[q] = __builtin_amdgcn_raw_buffer_load_b32(q ? rz2 : rz, zo, 0, 0);
    }
    u32x4_t wv[NP][GPW];
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int g = g0 + i * PL + p;
            wv[q][i] = ld16_g(q ? rw2 : rw,
                              (g < G && plive) ? (uint32_t)n * rowb + (uint32_t)g * 64u + 16u * h : kOobG);
        }
    // every load of the wave is issued before any arithmetic on X (the scheduler would
    // otherwise start the sums of X first and make the code loads wait for X to land)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (AO) {
        // the DMA and the perm loads were issued before the 3 GPW loads above:
        // vmcnt(3 GPW) means they have landed; the barrier makes every wave's part of
        // the row visible.  Then each slot gathers its 8 values (an entry of perm past
        // the row reads the row's last element)
        constexpr int kAfter = 3 * GPW;
        static_assert(kAfter < 16, "vmcnt field");
        __builtin_amdgcn_s_waitcnt(0x0F70 | kAfter);
        __syncthreads();
        const uint16_t *xr16 = (const uint16_t *)xrow;
        const uint32_t last = (uint32_t)K - 1u;
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = xr16[min(pv[r][0][e], last)];
                v[4 + e] = xr16[min(pv[r][1][e], last)];
            }
            const int slot = r * 64 + lane;
            const bool live = g0 * kGroup + slot * 8 < K;
            xv[r] = live ? u32x4_t{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)}
                         : u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    // 3. S of each group (the slot's 8 values, then across the 16 slots of the group,
    //    in a fixed order) and the slots in fragment order, into the wave's LDS region
#pragma unroll
    for (int r = 0; r < XR; ++r) {
        const float ps = row_sum16(sum8_bf16(xv[r]));
        if (nid == 0)
            Ss[r * 4 + h] = ps;
        xs[r * 64 + lane] = x_permute8(xv[r]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): the wave's LDS writes are done
    asm volatile("" ::: "memory");

    // 4. per instruction, four MFMAs (A row r: X of group part r % PL), then the fold
    //    s * (P - (128 + z) * S) of the lane's (column, group) pair
    uint32_t mask = 0x000F000Fu, bias = kBiasBits;
    asm volatile("" : "+v"(mask));
    asm volatile("" : "+v"(bias));
    const int zsh = (n & 7) * 4;
    const int m = nid % PL;
    float acc[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        acc[q] = 0.f;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            if (g0 + i * PL < G) {
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4_t xf = xs[(i * PL + m) * 16 + 4 * h + j];
                    const uint32_t wj = j == 0 ? wv[q][i].x : j == 1 ? wv[q][i].y : j == 2 ? wv[q][i].z : wv[q][i].w;
                    d = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf), frag_r(wj, mask, bias), d);
                }
                const bool live = g0 + i * PL + p < G && plive;
                const float s = live ? f16_bits_to_f32((uint16_t)to_row0(sv[q], i)) : 0.f;
                const float zb = -(float)(kCodeBias + ((to_row0(zv[q], i) >> zsh) & 15u));
                acc[q] = fmaf(s, fmaf(zb, Ss[i * PL + p], pick<PL>(d, p)), acc[q]);
            }
        }
    }

    // 5. lane (c + TC p, 0) holds column c's sum over the wave's groups of part p.  Wave
    //    0 adds the W waves' partials in a fixed tree: lane slot + 16 k adds those of
    //    waves k, k + 4, ... (all its reads in flight together), the four lane rows are
    //    added by two exchanges, then the parts p by log2(PL) more (PL = 3: lane c adds
    //    those of lanes c + 5 and c + 10)
    if (lane < 16) {
#pragma unroll
        for (int q = 0; q < NP; ++q)
            red[(w * NP + q) * 16 + lane] = acc[q];
    }
    __syncthreads();
    if (w == 0) {
        const int slot = lane & 15, k = lane >> 4;
        float yq[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            // every read in flight at once (a wave index past W reads wave 0's slot and
            // adds zero), then the sum in wave order
            float rv[kGemvMaxWaves / 4];
#pragma unroll
            for (int j = 0; j < kGemvMaxWaves / 4; ++j) {
                const int v = 4 * j + k;
                rv[j] = red[((v < W ? v : 0) * NP + q) * 16 + slot];
            }
            float y = 0.f;
#pragma unroll
            for (int j = 0; j < kGemvMaxWaves / 4; ++j)
                y += 4 * j + k < W ? rv[j] : 0.f;
            // the four lane rows: two lane swaps (VALU, no LDS round trip); each lane
            // adds its own value and its partner's, as an exchange with lane ^ 16, then
            // lane ^ 32, would
            {
                const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
                y = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
                const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
                y = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
            }
            if constexpr (PL == 3) {
                const float y1 = __shfl(y, (lane + TC) & 63), y2 = __shfl(y, (lane + 2 * TC) & 63);
                y = (y + y1) + y2;
            } else if constexpr (PL == 2) {
                // lane ^ 8 within the row: a rotation of the row by 8 lanes
                y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0x128, 0xF, 0xF, false));
            } else {
                if constexpr (PL >= 2)
                    y += __shfl_xor(y, TC);
                if constexpr (PL >= 4)
                    y += __shfl_xor(y, 2 * TC);
            }
            yq[q] = y;
        }
        const float y = GATED ? silu_f32(yq[0]) * yq[NP - 1] : yq[0];
        if (lane < TC) {
            const int col = bid * TC + lane;
            if (a.y_f32)
                ((float *)Yp)[col] = y;
            else
                ((uint16_t *)Yp)[col] = f32_to_bf16_rne(y);
            if constexpr (PAIR == 2) {
                if (a.y_f32)
                    ((float *)a.Y2)[col] = yq[1];
                else
                    ((uint16_t *)a.Y2)[col] = f32_to_bf16_rne(yq[1]);
            }
        }
    }
}

} // namespace

GemvPlan plan_gemv_with(int N, int K, int gpw, int pl, int ao)
{
    GemvPlan p{};
    const int G = K / kGroup;
    const int tc = pl == 3 ? 5 : pl > 0 ? 16 / pl : 0;
    const int ng = gpw * pl;
    p.gpw = gpw;
    p.pl = pl;
    p.ao = ao;
    p.waves = ng > 0 ? (G + ng - 1) / ng : 0;
    p.grid = tc > 0 ? N / tc : 0;
    p.lds_bytes = (size_t)gemv_x_off(p.waves, ng) + (ao ? (size_t)K * 2 : 0);
    p.ok = N >= 1 && K >= kGroup && ((pl == 2 && gpw == 2) || (pl == 4 && gpw == 3) || (pl == 3 && gpw == 4 && !ao)) && N % tc == 0 &&
           p.waves >= 1 && p.waves <= kGemvMaxWaves && p.lds_bytes <= (size_t)kGemvMaxLds;
    return p;
}

// the gated pair (pair 1) or two outputs (pair 2) at M = 1, up to 40 groups: the (2, 2)
// plan, the wave partials of both projections in LDS
GemvPlan plan_gemv_pair(int N, int K, int pair)
{
    if (K / kGroup > 40 || (pair != 1 && pair != 2))
        return GemvPlan{};
    GemvPlan p = plan_gemv_with(N, K, 2, 2, 0);
    p.pair = pair;
    p.lds_bytes = (size_t)gemv_r_off(p.waves, 4) + (size_t)p.waves * 128;
    p.ok = p.ok && p.lds_bytes <= (size_t)kGemvMaxLds;
    return p;
}

GemvPlan plan_gemv(int N, int K, int ao)
{
    // measured on MI355X at M = 1 (graph replays over rotating weights): two groups of
    // 8 columns per instruction and 4 groups per wave up to 40 groups (5 waves of 8
    // columns at K = 2560), three instructions of 4 columns x 4 groups beyond (7 waves
    // of 4 columns at K = 9728), or four of 5 columns x 3 groups where N / 5 workgroups
    // are whole rounds of the CUs (9728 -> 2560: 512 workgroups, two per CU, 6.15 us,
    // against 640 as two or three per CU, 6.4 us)
    const int G = K / kGroup;
    if (G <= 40)
        return plan_gemv_with(N, K, 2, 2, ao);
    if (!ao && N % (5 * 256) == 0)
        return plan_gemv_with(N, K, 4, 3, ao);
    return plan_gemv_with(N, K, 3, 4, ao);
}

GemvPlan plan_gemv_multi(const int *N, int K, int count, int *wg0)
{
    if (count < 1 || count > kMaxProblemsGemv)
        return GemvPlan{};
    bool by5 = true;
    for (int q = 0; q < count; ++q)
        by5 = by5 && N[q] % (5 * 256) == 0;
    // the single-projection choice, with five columns per workgroup only where every N
    // is a whole number of rounds of the CUs
    const int G = K / kGroup;
    GemvPlan p = G <= 40 ? plan_gemv_with(N[0], K, 2, 2, 0)
                 : by5   ? plan_gemv_with(N[0], K, 4, 3, 0)
                         : plan_gemv_with(N[0], K, 3, 4, 0);
    const int tc = p.pl == 3 ? 5 : 16 / p.pl;
    int wg = 0;
    for (int q = 0; q < count; ++q) {
        p.ok = p.ok && N[q] >= 1 && N[q] % tc == 0;
        wg0[q] = wg;
        wg += N[q] / tc;
    }
    p.pair = 3;
    p.grid = wg;
    return p;
}

hipError_t launch_gemv(const GemvArgs &args, const GemvPlan &p, hipStream_t stream)
{
    if (!p.ok)
        return hipErrorInvalidValue;
    GemvArgs a = args;
    a.waves = p.waves;
    const dim3 grid(p.grid), block(64 * p.waves);
    const int v = p.pair * 1000 + p.gpw * 100 + p.pl * 10 + (p.ao ? 1 : 0);
    switch (v) {
#define W4A16_GEMV_CASE(GPW, PL, AO)                                                                           \
    case GPW * 100 + PL * 10 + AO:                                                                             \
        hipLaunchKernelGGL((gemv_kernel<GPW, PL, AO != 0>), grid, block, p.lds_bytes, stream, a);              \
        break;
    case 1000 + 2 * 100 + 2 * 10:
        hipLaunchKernelGGL((gemv_kernel<2, 2, false, 1>), grid, block, p.lds_bytes, stream, a);
        break;
    case 2000 + 2 * 100 + 2 * 10:
        hipLaunchKernelGGL((gemv_kernel<2, 2, false, 2>), grid, block, p.lds_bytes, stream, a);
        break;
    case 3000 + 2 * 100 + 2 * 10:
        hipLaunchKernelGGL((gemv_kernel<2, 2, false, 3>), grid, block, p.lds_bytes, stream, a);
        break;
    case 3000 + 3 * 100 + 4 * 10:
        hipLaunchKernelGGL((gemv_kernel<3, 4, false, 3>), grid, block, p.lds_bytes, stream, a);
        break;
    case 3000 + 4 * 100 + 3 * 10:
        hipLaunchKernelGGL((gemv_kernel<4, 3, false, 3>), grid, block, p.lds_bytes, stream, a);
        break;
        W4A16_GEMV_CASE(2, 2, 0)
        W4A16_GEMV_CASE(2, 2, 1)
        W4A16_GEMV_CASE(3, 4, 0)
        W4A16_GEMV_CASE(3, 4, 1)
        W4A16_GEMV_CASE(4, 3, 0)
#undef W4A16_GEMV_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace w4a16
