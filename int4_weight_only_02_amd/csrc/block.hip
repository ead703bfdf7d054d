// block.hip -- W4A16 linear for one draft block (2 <= M <= 16 rows) on gfx950, one or
// several projections per launch.
//
// The pages' verifier runs the target over a block of 16 draft tokens at every
// speculative step (Pith review, Assumptions & free parameters: block size 16;
// mlsanity index page, Abstract), so every projection of a decoder layer runs at
// M = 16.  There the layer streams its packed weights once and each CU must also
// read all of X (16 rows x K bf16: 82 KB at K = 2560, 311 KB at K = 9728, as much
// as or more than the CU's share of the weights).  The kernel is shaped for that:
//
//   * One workgroup per CU (or a few), each owning a balanced run of 16-column
//     tiles and all of K (or, for long K, a part of it), so partial sums cross
//     workgroups only between the parts of K (a cross-workgroup hand-off costs
//     several round trips through the memory side).
//   * K is split over the workgroup's waves; each wave pulls its K slice of X into
//     its own LDS region by DMA in whole cache lines, reads it once into registers as
//     MFMA A fragments (lane (r, h): row r, k-block h) and keeps it for every tile of
//     the workgroup.  X is therefore read once per CU, with no barrier in front of it.
//   * A gated pair (silu(gate) * up) takes gate and up tiles of the same columns in
//     one workgroup and applies the activation in its epilogue.
//   * The codes of every (tile, group) of the wave's slice are requested up front:
//     lane (c, h) loads bytes 16h .. 16h+15 of column c's group, the B operand of
//     four v_mfma_f32_16x16x32_bf16 on the exact biased codes 128 + q (every product
//     exact in fp32), P = sum x * (128 + q); the bias and the zero-point come out in
//     fp32 with the row sums S of X over the group: acc += s * (P - (128 + z) * S).
//   * Each wave needs the scale and zero word of every (tile, group) pair of its slice,
//     the same value on the four lane rows of a column.  So lane row h loads them for
//     pair 4j + h (one instruction per four pairs, not one per pair), and two lane
//     swaps hand each value to all four rows when its fold runs.  The waves' K-slice
//     accumulators are added through LDS in slice order.  All sums run in a fixed
//     order: results are deterministic.
//   * Act-order (GPTQ g_idx) reaches this kernel with X already permuted by a gather
//     launch: gathering inside it, from the X rows in LDS, measured 2 us slower (about
//     40 thousand two-byte LDS reads per workgroup).
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr uint32_t kOobB = 0xFFFFFF00u; // an offset past the end of every tensor
constexpr int kRsrcWord3B = 0x00020000; // raw (untyped) buffer loads on gfx9-class GPUs
constexpr int kBlockCUs = 256;
constexpr int kBlockLds = 160 * 1024 - 256; // the rest holds the kernel's static LDS

// bytes of LDS per K slice when X goes through LDS (up to two groups per wave): the
// slice's X (4 KB per group), later its partial sums (1 KB per tile)
__host__ __device__ constexpr int block_xl_stride(int gpw, int tmax)
{
    return gpw * 4096 > tmax * 1024 ? gpw * 4096 : tmax * 1024;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3B);
}

__device__ __forceinline__ u32x4_t ld16_b(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ bf16x8_t frag_b(uint32_t w, uint32_t mask, uint32_t bias)
{
    u32x4_t r;
    r.x = (w & mask) | bias;
    r.y = ((w >> 4) & mask) | bias;
    r.z = ((w >> 8) & mask) | bias;
    r.w = ((w >> 12) & mask) | bias;
    return __builtin_bit_cast(bf16x8_t, r);
}

// rows 4 (l / 16) .. + 3 of column 16 t + l % 16 of Y (those inside M x N), by buffer
// stores at 32-bit offsets (Y is below 2^31 bytes)
__device__ __forceinline__ void store_rows(const BlockProb &pr, const BlockArgs &a, const f32x4_t &y, int t, int l,
                                           int M, int N)
{
    const int n = t * 16 + (l & 15);
    const int r0 = 4 * (l >> 4);
    if (n >= N)
        return;
    const uint32_t esz = a.y_f32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t ry = rsrc_b(pr.Y, (uint32_t)M * (uint32_t)N * esz);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        if (r < M) {
            const uint32_t off = ((uint32_t)r * (uint32_t)N + (uint32_t)n) * esz;
            if (a.y_f32)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[i]), ry, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(y[i]), ry, off, 0, 0);
        }
    }
}

// 4 x 4 transpose across the four 16-lane rows of a wave: afterwards register j of
// row h holds what register h of row j held.  Two swap stages (rows {0,1} <-> {2,3}
// between registers j and j + 2, then rows {0,2} <-> {1,3} between j and j + 1).
__device__ __forceinline__ void transpose_rows4(u32x4_t (&v)[4])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const auto r = __builtin_amdgcn_permlane32_swap(v[j][e], v[j + 2][e], false, false);
            v[j][e] = r[0];
            v[j + 2][e] = r[1];
        }
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const auto r = __builtin_amdgcn_permlane16_swap(v[j][e], v[j + 1][e], false, false);
            v[j][e] = r[0];
            v[j + 1][e] = r[1];
        }
    }
}

// the value that lane row r (of four) holds in v, on every lane row (column by column):
// swapping rows 0 <-> 1 and 2 <-> 3 gives [v0 v0 v2 v2] and [v1 v1 v3 v3], swapping the
// halves of the one that holds row r gives row r on all four
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, int r)
{
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const uint32_t x = (r & 1) ? p[1] : p[0];
    const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (r & 2) ? q[1] : q[0];
}

// LDS DMA: 16 bytes per lane from offset voff of r into LDS at dst + 16 * lane
__device__ __forceinline__ void dma16_b(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

// GPW: the most groups a wave's K slice holds; TMAX: the most tiles a workgroup owns;
// MODE 0: one projection; 1: several projections in the launch; 2: a gated pair (pr[0]
// the gate, pr[1] the up projection, the same shape; K whole): tile slot 2u holds gate
// tile t0 + u and slot 2u + 1 the up tile of the same columns, and the workgroup
// stores silu(gate) * up (the MLP activation of the pages' target; Pith review,
// Referee Report, Summary).
//
// The arguments live in memory that every CU reads through its scalar cache, and each
// read that depends on an earlier one costs a round trip to memory (about half a
// microsecond on a cold cache).  So every argument is read at a fixed offset: one
// projection reads pr[0] directly; several find their projection with one compare per
// entry (all entries read at once), then read its fields, two round trips in all.
template <int GPW, int TMAX, int MODE>
__global__ __launch_bounds__(1024) void block_kernel(BlockArgs a)
{
    constexpr bool MULTI = MODE == 1, GATED = MODE == 2;
    static_assert(!GATED || TMAX % 2 == 0, "gated slots come in pairs");
    extern __shared__ __align__(16) unsigned char lds[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = blockDim.x >> 6;
    // the workgroup's projection, its tile group [t0, t1) (balanced over the projection's
    // ntg tile groups) and its part of K (parts of a tile group are adjacent workgroups)
    int q = 0;
    if constexpr (MULTI) {
#pragma unroll
        for (int j = 1; j < kMaxProblemsBlock; ++j)
            q += (j < a.count && (int)blockIdx.x >= a.pr[j].wg0) ? 1 : 0;
    }
    const BlockProb &pr = a.pr[MULTI ? q : 0];
    const int P = pr.parts;
    const int b = blockIdx.x - pr.wg0;
    const int tg = b / P, part = b - tg * P;
    // tg * nt < 2^31: at most 2^16 tiles of 16 columns
    const int t0 = tg * pr.nt / pr.ntg;
    const int t1 = (tg + 1) * pr.nt / pr.ntg;
    const int T = t1 - t0;            // column tiles
    const int TS = GATED ? 2 * T : T; // live tile slots
    const int G = pr.K / kGroup, N = pr.N, M = a.M;
    const int Gp = (G + P - 1) / P;
    const int ga = part * Gp, gnp = min(Gp, G - ga); // the part's groups [ga, ga + gnp)
    const int gpw = (gnp + W - 1) / W;
    // the wave's K slice, rotated by the workgroup index so that the CUs, which all
    // read the same X, do not walk its lines in step
    const int slice = (w + (int)blockIdx.x) % W;
    const int g0 = ga + slice * gpw;
    const int gn = min(gpw, ga + gnp - g0); // this wave's groups (may be <= 0)
    const int c = lane & 15, h = lane >> 4;
    const uint32_t rowb = (uint32_t)(pr.K / 2);

    const __amdgpu_buffer_rsrc_t rw = rsrc_b(pr.qw, (uint32_t)N * rowb);
    const __amdgpu_buffer_rsrc_t rs = rsrc_b(pr.scales, (uint32_t)N * (uint32_t)G * 2u);
    const __amdgpu_buffer_rsrc_t rz = rsrc_b(pr.qz, (uint32_t)(N / 8) * (uint32_t)G * 4u);
    const __amdgpu_buffer_rsrc_t rx = rsrc_b(pr.X, (uint32_t)M * (uint32_t)pr.K * 2u);
    // gated: the up projection's grid (the same shape)
    const BlockProb &pu = a.pr[GATED ? 1 : 0];
    const __amdgpu_buffer_rsrc_t rw2 = GATED ? rsrc_b(pu.qw, (uint32_t)N * rowb) : rw;
    const __amdgpu_buffer_rsrc_t rs2 = GATED ? rsrc_b(pu.scales, (uint32_t)N * (uint32_t)G * 2u) : rs;
    const __amdgpu_buffer_rsrc_t rz2 = GATED ? rsrc_b(pu.qz, (uint32_t)(N / 8) * (uint32_t)G * 4u) : rz;

    // 1. the wave's K slice of X.  The MFMAs need lane (r, h) to hold
    //    X[r][(g0 + i) * 128 + 32h + 8j .. + 8] for j = 0..3 (the 64 bytes at 64h of the
    //    group's row).
    //    Up to two groups per wave (XL): the wave pulls its slice into its own LDS region
    //    by DMA in whole 128-byte lines (the load pipeline pays per line touched, so
    //    half-used lines would cost about half as much again): instruction u of group i
    //    brings rows 4u .. 4u+3, lane (c, h) the 16-byte chunk c ^ r of row r = 4u + h
    //    into slot c, so that the sixteen lanes of a lane row, which read one chunk of
    //    rows 0..15 below, find it in sixteen different slots (no bank conflicts).  Rows
    //    past M are not read (no output row depends on them).  Only this wave reads the
    //    region, after its own wait: no barrier.
    //    Three groups per wave: load j brings the 16 bytes at 64j + 16h into registers,
    //    so that the four lanes of a row read 64 contiguous bytes per instruction, and a
    //    4 x 4 transpose across the lane rows (below) puts each chunk in place (rows past
    //    M read as 0).
    constexpr bool XL = GPW <= 2;
    u32x4_t xf[GPW][4];
    unsigned char *xsl = lds + slice * block_xl_stride(GPW, TMAX); // XL: the slice's region
    if constexpr (XL) {
#pragma unroll
        for (int i = 0; i < GPW; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * u + h;
                dma16_b(rx, xsl + i * 4096 + u * 1024,
                        (r < M && i < gn) ? (uint32_t)r * (uint32_t)pr.K * 2u + (uint32_t)(g0 + i) * 256u +
                                                16u * (uint32_t)(c ^ r)
                                          : kOobB);
            }
    } else {
#pragma unroll
        for (int i = 0; i < GPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xf[i][j] = ld16_b(rx, (c < M && i < gn) ? (uint32_t)c * (uint32_t)pr.K * 2u +
                                                              (uint32_t)(g0 + i) * 256u + 64u * j + 16u * h
                                                        : kOobB);
    }

    // 2. the scale and zero word of (column tile, group) pair 4j + h (pairs numbered
    //    tile-major) of the lane's column (gated: of each projection in turn, one buffer
    //    per instruction); then the codes of every (tile slot, group) of the slice
    constexpr int TC = GATED ? TMAX / 2 : TMAX; // column tiles
    constexpr int PB = (TC * GPW + 3) / 4;      // parameter loads per projection
    constexpr int NPB = GATED ? 2 * PB : PB;
    uint32_t sv[NPB], zv[NPB];
#pragma unroll
    for (int sp = 0; sp < (GATED ? 2 : 1); ++sp)
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int pp = 4 * j + h, u = pp / GPW, i = pp - u * GPW;
            const int n = (t0 + u) * 16 + c;
            const bool live = u < T && i < gn && n < N;
            const uint32_t g = (uint32_t)(g0 + i);
            sv[sp * PB + j] = __builtin_amdgcn_raw_buffer_load_b16(
                sp ? rs2 : rs, live ? ((uint32_t)n * (uint32_t)G + g) * 2u : kOobB, 0, 0);
            zv[sp * PB + j] = __builtin_amdgcn_raw_buffer_load_b32(
                sp ? rz2 : rz, live ? ((uint32_t)(n >> 3) * (uint32_t)G + g) * 4u : kOobB, 0, 0);
        }
    u32x4_t wv[TMAX][GPW];
#pragma unroll
    for (int tl = 0; tl < TMAX; ++tl)
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int u = GATED ? tl >> 1 : tl;
            const int n = (t0 + u) * 16 + c;
            wv[tl][i] = ld16_b((GATED && (tl & 1)) ? rw2 : rw,
                               (u < T && i < gn && n < N) ? (uint32_t)n * rowb + (uint32_t)(g0 + i) * 64u + 16u * h
                                                          : kOobB);
        }
    asm volatile("" ::: "memory");
    // every load of the wave is issued before any arithmetic on X: left to itself the
    // compiler moves the arrangement of X (below) above the code loads and waits for X
    // first, so the codes' HBM latency would start only after X had arrived
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XL) {
        // the DMA was issued before the parameter and code loads: vmcnt(that many) means
        // it has landed; then chunk 4h + j of row c sits in slot (4h + j) ^ c
        constexpr int kAfter = 2 * NPB + TMAX * GPW;
        static_assert(kAfter < 64, "vmcnt is a 6-bit counter");
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kAfter & 15) | ((kAfter >> 4) << 14));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < GPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xf[i][j] = *(const u32x4_t *)(xsl + i * 4096 + c * 256 + 16 * ((4 * h + j) ^ c));
    }

    // X in place (the fragment order of the codes), and S[r][g] = sum of row r of X over
    // group g from the matrix cores: four MFMAs of the group's X fragments against a B of
    // ones (bf16 1.0) give D[r][c] = S[r][g] for every column c, so lane (c, h) receives
    // S of rows 4h .. 4h+3, the rows its accumulators hold (every product is exact; the
    // sums run in the matrix cores' fixed order).  Per wave that is four MFMAs per group
    // in place of some seventy VALU instructions and a round trip through LDS.
    uint32_t one = 0x3F803F80u;
    asm volatile("" : "+v"(one));
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one, one, one, one});
    f32x4_t Sv[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        if constexpr (!XL)
            transpose_rows4(xf[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xf[i][j] = x_permute8(xf[i][j]);
        f32x4_t sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sv = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[i][j]), ones, sv);
        Sv[i] = sv;
    }

    // 3. per (tile, group): four MFMAs on the biased codes (P = sum x * (128 + q)), then
    //    acc += s * (P - (128 + z) * S) in fp32
    uint32_t mask = 0x000F000Fu, bias = kBiasBits;
    asm volatile("" : "+v"(mask));
    asm volatile("" : "+v"(bias));
    const int zsh = (c & 7) * 4;
    f32x4_t acc[TMAX];
#pragma unroll
    for (int tl = 0; tl < TMAX; ++tl) {
        acc[tl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (tl < TS) {
#pragma unroll
            for (int i = 0; i < GPW; ++i) {
                if (i < gn) {
                    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
                    d = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[i][0]), frag_b(wv[tl][i].x, mask, bias), d);
                    d = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[i][1]), frag_b(wv[tl][i].y, mask, bias), d);
                    d = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[i][2]), frag_b(wv[tl][i].z, mask, bias), d);
                    d = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[i][3]), frag_b(wv[tl][i].w, mask, bias), d);
                    const int pp = (GATED ? tl >> 1 : tl) * GPW + i;
                    const int pb = (GATED && (tl & 1)) ? PB : 0;
                    const uint32_t zw = row_bcast(zv[pb + (pp >> 2)], pp & 3);
                    const float zb = -(float)(kCodeBias + ((zw >> zsh) & 15u));
                    const float s = f16_bits_to_f32((uint16_t)row_bcast(sv[pb + (pp >> 2)], pp & 3));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[tl][e] = fmaf(s, fmaf(zb, Sv[i][e], d[e]), acc[tl][e]);
                }
            }
        }
    }

    // 4. the K slices of each tile added in slice order; lane (c, h) holds rows 4h .. 4h+3
    //    of column c.  Slice v's partial sums of tile tl: XL, in the slice's own region
    //    (its X is no longer read); else [W][TMAX][64] from the start of LDS
    auto slice_acc = [&](int v, int tl) -> f32x4_t * {
        return XL ? (f32x4_t *)(lds + v * block_xl_stride(GPW, TMAX) + tl * 1024)
                  : (f32x4_t *)lds + (v * TMAX + tl) * 64;
    };
#pragma unroll
    for (int tl = 0; tl < TMAX; ++tl)
        if (tl < TS)
            slice_acc(slice, tl)[lane] = acc[tl];
    __syncthreads();
    __shared__ int s_last;
    float *pb = (float *)(a.ws + pr.part_off) + (size_t)tg * P * pr.tmx * 256; // [part][tmx * 64][4]
    uint32_t *ctr = (uint32_t *)(a.ws + kOffCounters) + (size_t)(pr.tkt + tg) * kCounterStride;
    for (int e = threadIdx.x; e < T * 64; e += W * 64) {
        const int tl = e >> 6, l = e & 63;
        f32x4_t y;
        if constexpr (GATED) {
            // the gate and up sums of column tile tl (K whole), then silu(gate) * up
            f32x4_t yg = slice_acc(0, 2 * tl)[l], yu = slice_acc(0, 2 * tl + 1)[l];
            for (int v = 1; v < W; ++v) {
                const f32x4_t og = slice_acc(v, 2 * tl)[l], ou = slice_acc(v, 2 * tl + 1)[l];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    yg[i] += og[i];
                    yu[i] += ou[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                y[i] = silu_f32(yg[i]) * yu[i];
        } else {
            y = slice_acc(0, tl)[l];
            for (int v = 1; v < W; ++v) {
                const f32x4_t o = slice_acc(v, tl)[l];
                y[0] += o[0];
                y[1] += o[1];
                y[2] += o[2];
                y[3] += o[3];
            }
        }
        if (GATED || P == 1) {
            store_rows(pr, a, y, t0 + tl, l, M, N);
        } else {
            // the part's partial sums, device-coherent, for the tile group's last arriver
            float *dst = pb + ((size_t)part * pr.tmx * 64 + e) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __hip_atomic_store(dst + i, y[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (!GATED && P > 1) {
        // parts of K meet in the workspace: each part stores its partial sums, then takes
        // an arrival ticket; the last to arrive adds the P parts in part order and stores
        // Y, so the result does not depend on the arrival order
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0): this thread's stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1);
        __syncthreads();
        if (s_last) {
            for (int e = threadIdx.x; e < T * 64; e += W * 64) {
                f32x4_t y;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = __hip_atomic_load(pb + (size_t)e * 4 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int pp = 1; pp < P; ++pp) {
                    const float *src = pb + ((size_t)pp * pr.tmx * 64 + e) * 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        y[i] += __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                store_rows(pr, a, y, t0 + (e >> 6), e & 63, M, N);
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

} // namespace

static size_t block_ws_bytes(int N, int T, int P)
{
    if (P <= 1)
        return 0;
    const int nt = (N + 15) / 16;
    const int ntg = (nt + T - 1) / T;
    const int tmx = (nt + ntg - 1) / ntg;
    return (size_t)ntg * P * tmx * 1024;
}

// Measured on MI355X at M = 16 (graph replays, K = 2560 .. 9728, N = 1024 .. 19456): K
// stays whole up to 47 groups (every CU reads all of X, and the hand-off of partial
// sums between parts costs more than the X it saves); longer K is cut into parts of
// at most 32 groups (so that a part's waves, two groups each, stay within 16), and
// each CU reads a part of X.  At K = 9728, N = 2560: 3 parts of 13 waves with 2 tiles
// per workgroup, 9.8-10.1 us, against 10.6-11.0 us for 4 to 6 parts.  The tile groups
// then spread the (tile group, part) workgroups of the whole launch about once over
// the CUs, at most 5 tiles each.
static int block_parts(int K)
{
    const int G = K / kGroup;
    return G < 48 ? 1 : (G + 31) / 32;
}

// Per projection the tile-group size T and the parts of K P (block_choose, or the
// hints); one wave count for the launch: enough that each wave's share of a part
// holds about two groups.
BlockPlan plan_block(const int *N, const int *K, int count, int M, int tmax_hint, int waves_hint, int parts_hint)
{
    BlockPlan p{};
    p.count = count;
    if (M < 2 || M > 16 || count < 1 || count > kMaxProblemsBlock)
        return p;
    int tmax = 1, gpmax = 1, tkt = 0;
    size_t off = kZeroRegion;
    int wg = 0;
    long long units = 0; // (tile, part) pairs of the launch
    for (int q = 0; q < count; ++q)
        units += (long long)((N[q] + 15) / 16) * block_parts(K[q]);
    int Tl = (int)((units + kBlockCUs - 1) / kBlockCUs);
    Tl = Tl < 1 ? 1 : Tl > 5 ? 5 : Tl;
    // each projection rounds its tile groups up: take one more tile per workgroup where
    // that keeps the launch within one round of the CUs (K = 9728, N = 4096: 86 x 3
    // workgroups of 3 tiles would leave two for a second round; 64 x 3 of 4 tiles do not)
    for (;;) {
        long long wgs = 0;
        for (int q = 0; q < count; ++q) {
            const int G = K[q] / kGroup, P = block_parts(K[q]);
            wgs += (long long)(((N[q] + 15) / 16 + Tl - 1) / Tl) * (P > G ? G : P);
        }
        if (wgs <= kBlockCUs || Tl >= 5)
            break;
        ++Tl;
    }
    for (int q = 0; q < count; ++q) {
        int T = Tl, P = block_parts(K[q]);
        if (tmax_hint > 0)
            T = tmax_hint;
        if (parts_hint > 0)
            P = parts_hint;
        const int G = K[q] / kGroup;
        P = P > G ? G : P;
        const int nt = (N[q] + 15) / 16;
        const int ntg = (nt + T - 1) / T;
        const int tmx = (nt + ntg - 1) / ntg;
        p.parts[q] = P;
        p.ntg[q] = ntg;
        p.tmx[q] = tmx;
        p.wg0[q] = wg;
        wg += ntg * P;
        tmax = tmx > tmax ? tmx : tmax;
        const int Gp = (G + P - 1) / P;
        gpmax = Gp > gpmax ? Gp : gpmax;
        p.tkt[q] = tkt;
        p.part_off[q] = off;
        if (P > 1) {
            tkt += ntg;
            off += block_ws_bytes(N[q], T, P);
        }
    }
    if (tkt > kMaxCounters)
        return p;
    p.ws_bytes = off == kZeroRegion ? 0 : off;
    p.grid = wg;
    int W = (gpmax + 1) / 2;
    if (waves_hint > 0)
        W = waves_hint;
    W = W < 1 ? 1 : W > 16 ? 16 : W;
    int gpw = (gpmax + W - 1) / W;
    p.tmax = tmax <= 1 ? 1 : tmax <= 2 ? 2 : tmax <= 5 ? 5 : 0;
    // register budget: three groups per wave at most with up to two tiles, else two
    const int gcap = p.tmax <= 2 ? 3 : 2;
    while (gpw > gcap && W < 16) {
        ++W;
        gpw = (gpmax + W - 1) / W;
    }
    p.gpw = gpw <= 1 ? 1 : gpw <= 2 ? 2 : gpw <= gcap ? 3 : 0;
    if (p.gpw == 0 || p.tmax == 0)
        return p;
    p.waves = W;
    // LDS: up to two groups per wave, X goes through LDS (one region per K slice, later
    // its slice accumulators); else the slice accumulators [W][TMAX][64] of 16 B
    p.lds_bytes = p.gpw <= 2 ? (size_t)W * block_xl_stride(p.gpw, p.tmax) : (size_t)W * p.tmax * 64 * 16;
    p.ok = p.lds_bytes <= (size_t)kBlockLds;
    return p;
}

// A gated pair (gate and up of the same shape, 2 <= M <= 16) in one launch: column
// tiles spread over the CUs about once (up to 3 per workgroup, i.e. 6 tile slots), K
// whole (up to 47 groups), up to two groups per wave.  !ok otherwise.
BlockPlan plan_block_gated(int N, int K, int M)
{
    BlockPlan p{};
    const int G = K / kGroup;
    if (M < 2 || M > 16 || block_parts(K) != 1 || G < 1)
        return p;
    const int nt = (N + 15) / 16;
    int T = (nt + kBlockCUs - 1) / kBlockCUs;
    T = T < 1 ? 1 : T;
    if (T > 3)
        return p;
    const int ntg = (nt + T - 1) / T;
    const int tmx = (nt + ntg - 1) / ntg;
    p.count = 1;
    p.gated = 1;
    p.parts[0] = 1;
    p.ntg[0] = ntg;
    p.tmx[0] = tmx;
    p.grid = ntg;
    p.tmax = 2 * tmx;
    int W = (G + 1) / 2;
    W = W < 1 ? 1 : W > 16 ? 16 : W;
    const int gpw = (G + W - 1) / W;
    if (gpw > 2)
        return p;
    p.gpw = gpw;
    p.waves = W;
    p.lds_bytes = (size_t)W * block_xl_stride(p.gpw, p.tmax);
    p.ok = p.lds_bytes <= (size_t)kBlockLds;
    return p;
}

// every block kernel may use up to kBlockLds bytes of dynamic LDS (beyond the 64 KB
// default); raised once per device
static hipError_t allow_block_lds(int)
{
    const void *fns[] = {
        (const void *)block_kernel<1, 1, 0>, (const void *)block_kernel<1, 2, 0>, (const void *)block_kernel<1, 5, 0>,
        (const void *)block_kernel<2, 1, 0>, (const void *)block_kernel<2, 2, 0>, (const void *)block_kernel<2, 5, 0>,
        (const void *)block_kernel<3, 1, 0>, (const void *)block_kernel<3, 2, 0>, (const void *)block_kernel<1, 1, 1>,
        (const void *)block_kernel<1, 2, 1>, (const void *)block_kernel<1, 5, 1>, (const void *)block_kernel<2, 1, 1>,
        (const void *)block_kernel<2, 2, 1>, (const void *)block_kernel<2, 5, 1>, (const void *)block_kernel<3, 1, 1>,
        (const void *)block_kernel<3, 2, 1>, (const void *)block_kernel<1, 2, 2>, (const void *)block_kernel<1, 4, 2>,
        (const void *)block_kernel<1, 6, 2>, (const void *)block_kernel<2, 2, 2>, (const void *)block_kernel<2, 4, 2>,
        (const void *)block_kernel<2, 6, 2>};
    for (const void *f : fns) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kBlockLds);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_block(const BlockArgs &args, const BlockPlan &p, hipStream_t stream)
{
    if (!p.ok)
        return hipErrorInvalidValue;
    BlockArgs a = args;
    a.count = p.count;
    for (int q = 0; q < p.count; ++q) {
        a.pr[q].wg0 = p.wg0[q];
        a.pr[q].nt = (a.pr[q].N + 15) / 16;
        a.pr[q].ntg = p.ntg[q];
        a.pr[q].parts = p.parts[q];
        a.pr[q].tmx = p.tmx[q];
        a.pr[q].tkt = p.tkt[q];
        a.pr[q].part_off = p.part_off[q];
    }
    const hipError_t e = once_per_device(kOnceBlock, allow_block_lds);
    if (e != hipSuccess)
        return e;
    const dim3 grid(p.grid), block(64 * p.waves);
    const int mode = p.gated ? 2 : p.count > 1 ? 1 : 0;
    switch (p.gpw * 1000 + p.tmax * 100 + mode) {
#define W4A16_BLOCK_CASE(GP, TM, MO)                                                                           \
    case GP * 1000 + TM * 100 + MO:                                                                            \
        hipLaunchKernelGGL((block_kernel<GP, TM, MO>), grid, block, p.lds_bytes, stream, a);                   \
        break;
        W4A16_BLOCK_CASE(1, 1, 0)
        W4A16_BLOCK_CASE(1, 2, 0)
        W4A16_BLOCK_CASE(1, 5, 0)
        W4A16_BLOCK_CASE(2, 1, 0)
        W4A16_BLOCK_CASE(2, 2, 0)
        W4A16_BLOCK_CASE(2, 5, 0)
        W4A16_BLOCK_CASE(3, 1, 0)
        W4A16_BLOCK_CASE(3, 2, 0)
        W4A16_BLOCK_CASE(1, 1, 1)
        W4A16_BLOCK_CASE(1, 2, 1)
        W4A16_BLOCK_CASE(1, 5, 1)
        W4A16_BLOCK_CASE(2, 1, 1)
        W4A16_BLOCK_CASE(2, 2, 1)
        W4A16_BLOCK_CASE(2, 5, 1)
        W4A16_BLOCK_CASE(3, 1, 1)
        W4A16_BLOCK_CASE(3, 2, 1)
        W4A16_BLOCK_CASE(1, 2, 2)
        W4A16_BLOCK_CASE(1, 4, 2)
        W4A16_BLOCK_CASE(1, 6, 2)
        W4A16_BLOCK_CASE(2, 2, 2)
        W4A16_BLOCK_CASE(2, 4, 2)
        W4A16_BLOCK_CASE(2, 6, 2)
#undef W4A16_BLOCK_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

size_t block_linear_ws(int M, int N, int K)
{
    const BlockPlan p = plan_block(&N, &K, 1, M);
    return p.ok ? p.ws_bytes : 0;
}

} // namespace w4a16
