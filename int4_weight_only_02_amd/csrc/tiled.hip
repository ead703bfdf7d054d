// tiled.hip -- W4A16 linear for large M (prefill) on gfx950: LDS-tiled fp16 MFMA.
//
// At M in the thousands the layer is bound by the matrix cores, and what limits a
// kernel that keeps the codes exact is the per-group fp32 fold it then needs
// (about six VALU instructions per MFMA).  This path instead feeds the matrix cores
// fp16 operands and accumulates all of K in fp32 directly:
//   * prep_kernel scales every row of X by a power of two 2^-e (chosen so the row's
//     largest magnitude lands in [2^14, 2^15)) and stores it as fp16.  bf16 has 8
//     significant bits and fp16 11, so the conversion is exact for every value
//     within 2^29 of the row maximum; only values far below it lose bits.  The eight
//     activations of each 16-byte chunk are stored in the order the code fragments
//     use (k0 k4 k1 k5 k2 k6 k3 k7);
//   * the weights are dequantized in registers, per packed word: the fp16 bias trick
//     gives 1024 + q exactly (0x6400 | q), one packed fp16 add of -(1024 + z) gives
//     q - z exactly, and one packed fp16 multiply by s rounds (q - z) * s once to
//     fp16 (relative error at most 2^-11 per weight);
//   * a workgroup of 8 waves (two per SIMD) computes a 256 x 256 tile of Y; each wave
//     owns 128 x 64 (8 x 4 tiles of v_mfma_f32_16x16x32_f16, accumulators in AGPRs).  K advances
//     one group (128) at a time through two LDS buffers filled by LDS DMA
//     (buffer_load ... lds) one group ahead: the X tile [256 rows x 16 chunks], its
//     16-byte slots XOR-swizzled by row (conflict-free fragment reads), and the
//     packed words [256 columns x 64 B];
//   * the epilogue multiplies each row by 2^e and stores bf16 (RNE) or fp32.  When
//     the tiles alone would leave most CUs idle in the last round, K is split into
//     slices: each slice stores its fp32 partial sums and reduce_kernel adds them in
//     slice order (deterministic), scales the row and stores Y;
//   * gated pair (the MLP's silu(X Wg^T) * (X Wu^T); Pith review, Referee Report,
//     Summary: the target's MLP): a tile covers 128 output columns, and each wave's
//     four column tiles are two of gate and the same two of up, so the epilogue forms
//     silu(gate) * up from the wave's own accumulators and neither projection's
//     output is ever stored.
// With X ~ N(0, 1) the rounding of the weights contributes about 3e-4 * rms(Y) (rms),
// a few percent of the 1e-2 * rms(Y) bound at the largest shapes.
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

constexpr int BM = 256, BN = 256, kThreads = 512;
constexpr int kXBytes = BM * kGroup * 2; // 65536: X tile of one group (fp16)
constexpr int kWBytes = BN * 64;         // 16384: packed words of one group
constexpr int kBufBytes = kXBytes + kWBytes;
constexpr int kLdsBytes = 2 * kBufBytes; // 163840
constexpr uint32_t kOob = 0xFFFFFF00u;   // an offset past the end of every tensor
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kF16Bias = 0x64006400u; // fp16 1024 in both halves
constexpr int kSc1 = 16;                   // buffer cache-policy bit sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane from global memory (offset off of r) into LDS at dst + 16 * lane;
// dst must be the same for the whole wave
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// XOR swizzle of the 16-byte chunks of X-tile row r.  A fragment read has lane l at row
// l % 16 and chunk 4 (l / 16) + j; spreading rows 0..7 over the even swizzles and rows
// 8..15 over the odd ones keeps every pass of the 128-bit LDS read conflict-free (it
// measured about 1.5x faster than the swizzle r % 16 on gfx950).
__device__ __forceinline__ int xswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); } // vmcnt(0)

// One row per workgroup: X[m] * 2^-e as fp16 (chunks permuted to the fragment order),
// and 2^e into rowscale[m].  A row of up to kPrepHeld * 256 chunks of 8 (K <= 16384) is
// read once, into registers, all loads in flight together; longer rows are read twice.
constexpr int kPrepHeld = 8;

__device__ __forceinline__ float absmax8(const u32x4_t &v)
{
    return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))), fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))),
                 fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))), fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
}

// eight activations times 2^-e, as fp16 in the fragment order k0 k4 k1 k5 k2 k6 k3 k7
__device__ __forceinline__ u32x4_t scale8(const u32x4_t &v, float down)
{
    const float f0 = bf16_lo(v.x) * down, f1 = bf16_hi(v.x) * down;
    const float f2 = bf16_lo(v.y) * down, f3 = bf16_hi(v.y) * down;
    const float f4 = bf16_lo(v.z) * down, f5 = bf16_hi(v.z) * down;
    const float f6 = bf16_lo(v.w) * down, f7 = bf16_hi(v.w) * down;
    const f16x8_t o = {(_Float16)f0, (_Float16)f4, (_Float16)f1, (_Float16)f5,
                       (_Float16)f2, (_Float16)f6, (_Float16)f3, (_Float16)f7};
    return __builtin_bit_cast(u32x4_t, o);
}

__global__ __launch_bounds__(256) void prep_kernel(const uint16_t *X, int K, uint16_t *Xh, float *rowscale)
{
    __shared__ float wmax[4];
    const int m = blockIdx.x, tid = threadIdx.x;
    const u32x4_t *xr = (const u32x4_t *)(X + (size_t)m * K);
    u32x4_t *hr = (u32x4_t *)(Xh + (size_t)m * K);
    const int nc = K / 8;
    const bool held = nc <= kPrepHeld * 256; // uniform

    u32x4_t v[kPrepHeld];
    const int rounds = (nc + 255) / 256; // uniform: rounds past it are skipped
    float mx = 0.f;
    if (held) {
#pragma unroll
        for (int i = 0; i < kPrepHeld; ++i)
            if (i < rounds)
                v[i] = tid + i * 256 < nc ? xr[tid + i * 256] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kPrepHeld; ++i)
            if (i < rounds)
                mx = fmaxf(mx, absmax8(v[i]));
    } else {
        for (int c = tid; c < nc; c += 256)
            mx = fmaxf(mx, absmax8(xr[c]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0)
        wmax[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

    // floor(log2(max)) = E - 127 for a normal max; the scaled maximum lands in
    // [2^14, 2^15).  e is clamped so that 2^e and 2^-e are normal floats.
    const int E = (int)((__float_as_uint(mx) >> 23) & 0xFFu);
    int e = mx > 0.f ? E - 141 : 0;
    e = e < -126 ? -126 : e > 113 ? 113 : e;
    const float down = __uint_as_float((uint32_t)(127 - e) << 23); // 2^-e
    if (tid == 0)
        rowscale[m] = __uint_as_float((uint32_t)(127 + e) << 23); // 2^e

    if (held) {
#pragma unroll
        for (int i = 0; i < kPrepHeld; ++i)
            if (i < rounds && tid + i * 256 < nc)
                hr[tid + i * 256] = scale8(v[i], down);
    } else {
        for (int c = tid; c < nc; c += 256)
            hr[c] = scale8(xr[c], down);
    }
}

__device__ __forceinline__ f16x2_t as_h2(uint32_t u) { return __builtin_bit_cast(f16x2_t, u); }

// one packed word (codes k0..k7 of a column) -> fp16 fragment (k0 k4 k1 k5 k2 k6 k3 k7)
// of (q - z) * s: (1024 + q) exact, minus (1024 + z) exact, times s rounded once
__device__ __forceinline__ f16x8_t dequant_word(uint32_t w, uint32_t mask, uint32_t bias, f16x2_t zn, f16x2_t s2)
{
    const f16x2_t d0 = as_h2((w & mask) | bias) + zn;
    const f16x2_t d1 = as_h2(((w >> 4) & mask) | bias) + zn;
    const f16x2_t d2 = as_h2(((w >> 8) & mask) | bias) + zn;
    const f16x2_t d3 = as_h2(((w >> 12) & mask) | bias) + zn;
    const f16x2_t r0 = d0 * s2, r1 = d1 * s2, r2 = d2 * s2, r3 = d3 * s2;
    return f16x8_t{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

// A workgroup computes a sequence of tile-groups (tile t, group g; tiles n-fastest)
// through one software pipeline that also runs across tile boundaries (the next
// tile's first group is fetched while the current tile's last group computes).
//   split plan  (STREAM false): one tile, one K slice [ks * gper, ...) per workgroup;
//               with ksplit > 1 the slice's fp32 partial sums go to the workspace and
//               reduce_kernel finishes Y;
//   stream plan (STREAM true, at least one tile per CU): workgroup b first takes whole
//               tiles, one per round (all rounds but the last one or two), then owns
//               segment s of the remaining tiles' tile-groups; segments differ by at
//               most one tile-group and hold at least G, so a tile is either whole in
//               one segment or split in two parts at one segment boundary.  Both parts
//               store their fp32 sums in the workspace and take a ticket; the second
//               to arrive adds the other part (a + b = b + a in fp32, so the result
//               does not depend on the arrival order), scales and stores Y, and
//               returns the ticket to zero.
template <bool STREAM, bool GATED>
__global__ __launch_bounds__(kThreads) void tiled_kernel(TiledArgs a, TiledPlan p)
{
    static_assert(!(STREAM && GATED), "the gated pair runs whole tiles");
    constexpr int BNO = GATED ? BN / 2 : BN; // output columns per tile
    extern __shared__ __align__(16) unsigned char smem[]; // all of the 160 KB: no static LDS

    const int M = a.M, N = a.N, K = a.K, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3; // 2 x 4 waves of 128 x 64
    const int h = lane >> 4, col = lane & 15;

    // runs are dealt out so that each XCD (blocks b, b + 8, ...) takes a contiguous
    // stretch of tiles in n-fastest order: its CUs share X rows in their L2
    const int ntiles = p.tiles_m * p.tiles_n;
    const int b = blockIdx.x;
    // lo, hi: this workgroup's range of K-split or stream-segment tile-groups; dpr: the
    // whole tiles it takes first (stream plan), tile k * grid + pos in round k
    int lo, hi, seg, dpr = 0;
    if constexpr (STREAM) {
        seg = (p.grid & 7) == 0 ? (b & 7) * (p.grid >> 3) + (b >> 3) : b;
        dpr = p.dp_rounds;
        const long long U = (long long)(ntiles - dpr * p.grid) * G;
        lo = (int)(U * seg / p.grid);
        hi = (int)(U * (seg + 1) / p.grid);
    } else {
        // K slices are the outermost index: unit u = slice * ntiles + tile
        const int nunits = ntiles * p.ksplit;
        int u = (b & 7) * (nunits / 8) + (b >> 3);
        if ((nunits & 7) != 0)
            u = b; // uneven split: plain order
        const int ks = u / ntiles, t = u - ks * ntiles;
        const int g0 = ks * p.gper, g1 = G < g0 + p.gper ? G : g0 + p.gper;
        lo = t * G + g0;
        hi = t * G + g1;
        seg = ks;
    }
    const int total = dpr * G + (hi - lo);
    const int sk0 = dpr * p.grid * G; // first tile-group of the stream segments
    // the i-th tile-group of this workgroup: tile t, group g
    auto unit = [&](int i, int &t, int &g) {
        if constexpr (!STREAM) {
            t = lo / G; // one tile
            g = lo - t * G + i;
        } else if (i < dpr * G) {
            const int k = i / G;
            t = k * p.grid + seg;
            g = i - k * G;
        } else {
            const int u = sk0 + lo + (i - dpr * G);
            t = u / G;
            g = u - t * G;
        }
    };

    const uint16_t *xh = (const uint16_t *)(a.ws + p.off_xh);
    const float *rowscale = (const float *)(a.ws + p.off_rs);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xh, (uint32_t)((size_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.qw, (uint32_t)((size_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, (uint32_t)((size_t)N * G * 2));
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.qz, (uint32_t)((size_t)(N / 8) * G * 4));
    // gated: the up projection's grid (column slots 32 .. 63 of each quarter of the tile)
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(GATED ? a.qw2 : a.qw, (uint32_t)((size_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(GATED ? a.scales2 : a.scales, (uint32_t)((size_t)N * G * 2));
    const __amdgpu_buffer_rsrc_t rz2 = make_rsrc(GATED ? a.qz2 : a.qz, (uint32_t)((size_t)(N / 8) * G * 4));
    // the output column of column slot cl (0 .. 255) of a tile at n0, and of the lane's
    // column tile nt; gated: quarter cl / 64 holds 32 columns of gate, then the same 32
    // of up
    auto slot_col = [&](int n0, int cl) { return GATED ? n0 + (cl >> 6) * 32 + (cl & 31) : n0 + cl; };
    auto lane_col = [&](int n0, int nt) {
        return GATED ? n0 + wn * 32 + (nt & 1) * 16 + col : n0 + wn * 64 + nt * 16 + col;
    };

    // Per-lane offsets of group 0 of the tile being fetched; group g adds g * 256 bytes
    // (X), g * 64 (words), 2g (scales), 4g (zero words) as the scalar offset.  Rows past
    // M and columns past N start at kOob: with the scalar offset added the address may
    // wrap to somewhere inside the tensor, which is harmless (those rows and columns
    // are never stored).
    uint32_t xoff[8], woff[2], soff[4], zoff[4];
    auto set_tile = [&](int t) {
        const int tm = t / p.tiles_n, tn = t - tm * p.tiles_n;
        const int m0 = tm * BM, n0 = tn * BNO;
        // the lane index through an opaque copy: the per-lane terms below are recomputed
        // at each tile instead of being hoisted out of the loop and kept live throughout
        // (which pushes the stream plan's instance past the register file)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = (wave * 8 + i) * 64 + ln; // X slot: row s/16, swizzled chunk s%16
            const int row = s >> 4, c = (s & 15) ^ xswz(row);
            xoff[i] = m0 + row < M ? ((uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)(c * 8)) * 2u : kOob;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int s = (wave * 2 + i) * 64 + ln; // word slot: column s/4, swizzled quarter s%4
            const int cl = s >> 2, q = (s & 3) ^ ((cl >> 2) & 3);
            const int n = slot_col(n0, cl);
            woff[i] = n < N ? (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(q * 16) : kOob;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int n = lane_col(n0, nt);
            soff[nt] = n < N ? (uint32_t)(n * G) * 2u : kOob;
            zoff[nt] = n < N ? (uint32_t)((n >> 3) * G) * 4u : kOob;
        }
    };
    // DMA of group g into buffer bi: X 8 x 1 KB per wave, words 2 x 1 KB per wave
    auto issue = [&](int g, int bi) {
        unsigned char *base = smem + bi * kBufBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dma16(rx, base + (wave * 8 + i) * 1024, xoff[i], (uint32_t)g * (kGroup * 2));
        // a word instruction covers 16 column slots, all of one projection
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(GATED && (((wave * 2 + i) >> 1) & 1) ? rw2 : rw, base + kXBytes + (wave * 2 + i) * 1024, woff[i],
                  (uint32_t)g * 64u);
    };
    // per-lane scale and zero word of the wave's 4 column tiles for group g
    uint32_t sc_raw[4], zw_raw[4];
    auto load_params = [&](int g) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const bool up = GATED && nt >= 2;
            sc_raw[nt] = __builtin_amdgcn_raw_buffer_load_b16(up ? rs2 : rs, soff[nt], (uint32_t)g * 2u, 0);
            zw_raw[nt] = __builtin_amdgcn_raw_buffer_load_b32(up ? rz2 : rz, zoff[nt], (uint32_t)g * 4u, 0);
        }
    };

    // dequantization constants pinned in VGPRs (one v_and_or_b32 per code pair)
    uint32_t kmask = 0x000F000Fu, kbias = kF16Bias;
    asm volatile("" : "+v"(kmask));
    asm volatile("" : "+v"(kbias));

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Y of the tile: 2^e_m * acc, stored as bf16 (RNE, the hardware conversion) or fp32.
    // A lane holds 4 rows of one column per 16 x 16 tile; a 4 x 4 transpose within each
    // quad of lanes (two exchanges with lanes j ^ 1 and j ^ 2) leaves lane j with row
    // 4h + j of 4 consecutive columns, stored as one 8-byte (bf16) or 16-byte (fp32)
    // run: a quarter of the store instructions.  The row scales are requested before
    // the first store, so waiting for them waits for no store (the memory counter the
    // wait uses also counts stores).
    auto store_y = [&](int m0, int n0) {
        const int j = col & 3, cq = col & ~3; // lane in its quad, the quad's first column
        const bool odd = (j & 1) != 0, hi2 = (j & 2) != 0;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(rowscale, (uint32_t)((size_t)M * sizeof(float)));
        float rsj[8]; // the scale of row 4h + j of each row tile (rows past M read 0)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            rsj[mt] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)(m0 + wm * 128 + mt * 16 + 4 * h + j) * 4u, 0, 0));
        auto quad_t = [&](const f32x4_t &v) {
            // exchange with lane j ^ 1: the elements whose bit 0 differs from j's
            const float r0 = __shfl_xor(odd ? v[0] : v[1], 1), r1 = __shfl_xor(odd ? v[2] : v[3], 1);
            const f32x4_t t = odd ? f32x4_t{r0, v[1], r1, v[3]} : f32x4_t{v[0], r0, v[2], r1};
            // exchange with lane j ^ 2: the elements whose bit 1 differs from j's
            const float q0 = __shfl_xor(hi2 ? t[0] : t[2], 2), q1 = __shfl_xor(hi2 ? t[1] : t[3], 2);
            return hi2 ? f32x4_t{q0, q1, t[2], t[3]} : f32x4_t{t[0], t[1], q0, q1};
        };
        // gated: column tiles 0, 1 (gate) pair with 2, 3 (up) of the same columns
        constexpr int NT = GATED ? 2 : 4;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int row = m0 + wm * 128 + mt * 16 + 4 * h + j;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float sc = rsj[mt];
                const f32x4_t w = quad_t(acc[mt][nt]);
                f32x4_t y = {w[0] * sc, w[1] * sc, w[2] * sc, w[3] * sc};
                if constexpr (GATED) {
                    const f32x4_t u = quad_t(acc[mt][nt + 2]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        y[r] = silu_f32(y[r]) * (u[r] * sc);
                }
                const int cn = lane_col(n0, nt) - col + cq; // N % 8 == 0: 4 columns all in or all out
                if (row < M && cn < N) {
                    const size_t off = (size_t)row * N + cn;
                    if (a.y_f32) {
                        *(f32x4_t *)((float *)a.Y + off) = y;
                    } else {
                        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
                        *(bf16x4_t *)((__bf16 *)a.Y + off) = bf16x4_t{(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
                    }
                }
            }
        }
    };

    // The end of a run of tile t (groups gs .. ge-1), origin (m0, n0), whose last group
    // computed from LDS buffer bi.  Every thread of the workgroup calls it (the barriers
    // inside are uniform).
    auto finish = [&](int m0, int n0, int gs, int ge, int bi) {
        if (!STREAM && !GATED && p.ksplit > 1) {
            // fp32 partial sums of this K slice; reduce_kernel finishes the rows
            float *part = (float *)(a.ws + p.off_part) + (size_t)seg * M * N;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int cn = n0 + wn * 64 + nt * 16 + col;
                    if (cn >= N)
                        continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = m0 + wm * 128 + mt * 16 + 4 * h + r;
                        if (row < M)
                            part[(size_t)row * N + cn] = acc[mt][nt][r];
                    }
                }
            return;
        }
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(a.ws + p.off_part, (uint32_t)((size_t)(p.grid - 1) * 2 * BM * BN * sizeof(float)));
        // A tile split at a segment boundary: the boundary's pair of regions, one per
        // part ([part][row tile, column tile][thread][4 rows], so each store instruction
        // covers 1 KB), stored and loaded with the sc1 cache policy (the
        // instructions of relaxed device-scope atomics: coherent across the XCDs' L2s).
        // (One call site of store_y: a second inlined copy makes the register
        // allocator spill.)
        const bool split = STREAM && !(gs == 0 && ge == G); // only stream segments split tiles
        const int slot = gs == 0 ? seg : seg - 1; // boundary seg + 1 or seg, minus one
        const int mine = gs == 0 ? 0 : 1;
        const uint32_t other = ((uint32_t)(slot * 2 + 1 - mine) * (BM * BN) + (uint32_t)tid * 4u) * 4u;
        uint32_t *tk = (uint32_t *)(a.ws + kOffCounters) + (size_t)slot * kCounterStride;
        if constexpr (STREAM) {
            if (split) {
                const uint32_t own = ((uint32_t)(slot * 2 + mine) * (BM * BN) + (uint32_t)tid * 4u) * 4u;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[mt][nt]), rp,
                                                               own + (uint32_t)((mt * 4 + nt) * kThreads * 16), 0, kSc1);
                wait_vmem(); // the stores (and anything in flight) have completed
                __syncthreads();
                // the arrival order passes through the first word of buffer bi: every wave
                // is done reading it, and the next DMA into it follows the loop's barrier
                int *flag = (int *)(smem + bi * kBufBytes);
                if (tid == 0)
                    *flag = (int)__hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                if (*flag == 0)
                    return; // the other part finishes the tile (uniform over the workgroup)
                // the other part's sums into acc, 16 bytes per column tile, the next row
                // tile's loads in flight while one adds: all before the first store, so
                // no wait for them waits for a store
                f32x4_t ob[2][4];
                auto load_other = [&](int mt, f32x4_t (&o)[4]) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        o[nt] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                rp, other + (uint32_t)((mt * 4 + nt) * kThreads * 16), 0, kSc1));
                };
                load_other(0, ob[0]);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    if (mt + 1 < 8)
                        load_other(mt + 1, ob[(mt + 1) & 1]);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] += ob[mt & 1][nt];
                }
            }
        } else {
            (void)bi; // the split plan finishes after its loop, with no buffer in use
        }
        store_y(m0, n0);
        if (split && tid == 0)
            __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    int t, g;
    unit(0, t, g);
    int gs = g;
    set_tile(t);
    int m0 = (t / p.tiles_n) * BM, n0 = (t % p.tiles_n) * BNO;
    issue(g, 0);
    load_params(g);
    wait_vmem();
    __syncthreads();

    for (int i = 0; i < total; ++i) {
        const int bi = i & 1;
        const unsigned char *base = smem + bi * kBufBytes;
        f16x2_t s2[4], zn[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int zsh = (lane_col(n0, nt) & 7) * 4;
            s2[nt] = as_h2((sc_raw[nt] & 0xFFFFu) * 0x00010001u);
            zn[nt] = as_h2((0xE400u | ((zw_raw[nt] >> zsh) & 15u)) * 0x00010001u); // -(1024 + z)
        }
        // the next tile-group, possibly of another tile: fetched while this one computes
        int tn = t, gn = g;
        if (i + 1 < total) {
            unit(i + 1, tn, gn);
            if (tn != t)
                set_tile(tn);
            issue(gn, bi ^ 1);
            load_params(gn);
        }

        // the 4 words (k-steps 0..3) of each of the lane's 4 columns
        u32x4_t wv[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int cl = wn * 64 + nt * 16 + col;
            wv[nt] = *(const u32x4_t *)(base + kXBytes + (cl * 4 + (h ^ ((cl >> 2) & 3))) * 16);
        }
        // A fragments of k-step j (chunk 4h + j of lane group h) for the 8 row tiles; the
        // next k-step's are read while this one computes.  B is dequantized one column
        // tile at a time, between its 8 MFMAs.
        auto read_a = [&](int j, f16x8_t (&af)[8]) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const int row = wm * 128 + mt * 16 + col;
                af[mt] = *(const f16x8_t *)(base + (row * 16 + ((4 * h + j) ^ xswz(row))) * 16);
            }
        };
        f16x8_t afa[8], afb[8];
        read_a(0, afa);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x8_t(&cur)[8] = (j & 1) ? afb : afa;
            f16x8_t(&nxt)[8] = (j & 1) ? afa : afb;
            if (j < 3)
                read_a(j + 1, nxt);
            auto word = [&](int nt) { return j == 0 ? wv[nt].x : j == 1 ? wv[nt].y : j == 2 ? wv[nt].z : wv[nt].w; };
            // B of column tile nt + 1 is dequantized while the MFMAs of tile nt run
            f16x8_t bcur = dequant_word(word(0), kmask, kbias, zn[0], s2[0]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                f16x8_t bnext = bcur;
                if (nt < 3)
                    bnext = dequant_word(word(nt + 1), kmask, kbias, zn[nt + 1], s2[nt + 1]);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur[mt], bcur, acc[mt][nt], 0, 0, 0);
                bcur = bnext;
            }
        }

        if (STREAM && (i + 1 == total || tn != t)) {
            finish(m0, n0, gs, g + 1, bi);
#pragma unroll
            for (int x = 0; x < 8; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y)
                    acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        wait_vmem(); // the next group's DMA and parameters have landed
        __syncthreads();
        if (tn != t) {
            t = tn;
            gs = gn;
            m0 = (t / p.tiles_n) * BM;
            n0 = (t % p.tiles_n) * BNO;
        }
        g = gn;
    }
    if constexpr (!STREAM)
        finish(m0, n0, gs, gs + total, 0); // the one tile (or K slice) of this workgroup
}

// Y[m, 4c .. 4c+3] = 2^e_m * sum over slices s (in order) of part[s][m][4c ..]; N % 8 == 0
__global__ __launch_bounds__(256) void reduce_kernel(const float *part, const float *rowscale, int M, int N, int ksplit,
                                                     void *Y, int y_f32)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x; // 4 outputs each
    const long long total = (long long)M * N / 4;
    if (i >= total)
        return;
    const int m = (int)(i * 4 / N);
    const size_t stride = (size_t)M * N;
    f32x4_t s = *(const f32x4_t *)(part + i * 4);
    for (int k = 1; k < ksplit; ++k) {
        const f32x4_t v = *(const f32x4_t *)(part + (size_t)k * stride + i * 4);
        s[0] += v[0];
        s[1] += v[1];
        s[2] += v[2];
        s[3] += v[3];
    }
    const float sc = rowscale[m];
    if (y_f32) {
        *(f32x4_t *)((float *)Y + i * 4) = f32x4_t{s[0] * sc, s[1] * sc, s[2] * sc, s[3] * sc};
    } else {
        const uint32_t lo = f32_to_bf16_rne(s[0] * sc) | ((uint32_t)f32_to_bf16_rne(s[1] * sc) << 16);
        const uint32_t hi = f32_to_bf16_rne(s[2] * sc) | ((uint32_t)f32_to_bf16_rne(s[3] * sc) << 16);
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
        *(u32x2_t *)((uint16_t *)Y + i * 4) = u32x2_t{lo, hi};
    }
}

size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

} // namespace

TiledPlan plan_tiled(int M, int N, int K)
{
    TiledPlan p{};
    p.G = K / kGroup;
    p.tiles_m = (M + BM - 1) / BM;
    p.tiles_n = (N + BN - 1) / BN;
    const long long ntiles = (long long)p.tiles_m * p.tiles_n;
    const int kCUs = 256;
    p.off_xh = kZeroRegion;
    p.off_rs = round_up(p.off_xh + (size_t)M * K * 2, 256);
    p.off_part = round_up(p.off_rs + (size_t)M * sizeof(float), 256);
    // Estimated time of each plan: rounds * groups per round (one tile-group ~ 3.5 us on
    // a CU), plus the traffic of the partial sums (~5 TB/s) for K slices; the stream
    // plan (at least one tile per CU) spreads the tile-groups evenly over the CUs at
    // about 10% more per tile-group (split tiles meet in memory; measured on MI355X)
    double best = 1e30;
    p.stream = 0;
    p.dp_rounds = 0;
    p.ksplit = 1;
    for (int ks = 1; ks <= 4 && ks <= p.G; ++ks) {
        const int gper = (p.G + ks - 1) / ks;
        const double rounds = (double)((ntiles * ks + kCUs - 1) / kCUs);
        double t = rounds * gper * 3.5e-6;
        if (ks > 1)
            t += (double)(ks * 4 + 2) * M * N / 5e12;
        if (t < best * 0.97) { // prefer fewer slices unless clearly faster
            best = t;
            p.ksplit = ks;
        }
    }
    if (ntiles >= kCUs && (double)ntiles * p.G / kCUs * 3.5e-6 * 1.1 < best) {
        // one segment of tile-groups per CU, balanced to one tile-group, after whole
        // tiles in all rounds but the last two (tile k * grid + pos, so that the tiles in
        // flight at a time are neighbours that share X rows in L2); the segments (at
        // least G each) split at most one tile at each inner boundary: a pair of fp32
        // regions and an arrival counter per boundary
        static_assert(kCUs - 1 <= kMaxCounters, "one arrival counter per inner boundary");
        p.stream = 1;
        p.grid = kCUs;
        p.dp_rounds = (int)(ntiles / kCUs) - 1;
        p.ksplit = 1;
        p.gper = p.G;
        p.ws_bytes = p.off_part + (size_t)(p.grid - 1) * 2 * BM * BN * sizeof(float);
        p.ok = true;
        return p;
    }
    p.gper = (p.G + p.ksplit - 1) / p.ksplit;
    p.ksplit = (p.G + p.gper - 1) / p.gper; // no empty slices
    p.grid = (int)(ntiles * p.ksplit);
    p.ws_bytes = p.off_part + (p.ksplit > 1 ? (size_t)p.ksplit * M * N * sizeof(float) : 0);
    p.ok = true;
    return p;
}

// The gated pair (gate and up of the same N x K shape): tiles of 256 rows x 128 output
// columns, whole K, no split; ok when the tiles alone fill at least one round of the
// CUs (otherwise the two projections run as separate calls).
TiledPlan plan_tiled_gated(int M, int N, int K)
{
    TiledPlan p = plan_tiled(M, N, K);
    p.tiles_n = (N + BN / 2 - 1) / (BN / 2);
    p.stream = 0;
    p.dp_rounds = 0;
    p.ksplit = 1;
    p.gper = p.G;
    p.grid = p.tiles_m * p.tiles_n;
    p.gated = 1;
    p.ws_bytes = p.off_part;
    p.ok = p.grid >= 256;
    return p;
}

hipError_t launch_tiled(const TiledArgs &a, const TiledPlan &p, hipStream_t stream)
{
    if (p.gated && (!a.qw2 || !a.scales2 || !a.qz2 || p.stream || p.ksplit != 1))
        return hipErrorInvalidValue;
    // every tile kernel uses all 160 KB of LDS: allowed once per device
    hipError_t e = once_per_device(kOnceTiled, [](int) -> hipError_t {
        const void *fns[] = {(const void *)tiled_kernel<false, false>, (const void *)tiled_kernel<true, false>,
                             (const void *)tiled_kernel<false, true>};
        for (const void *f : fns) {
            const hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
            if (r != hipSuccess)
                return r;
        }
        return hipSuccess;
    });
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(prep_kernel, dim3(a.M), dim3(256), 0, stream, a.X, a.K, (uint16_t *)(a.ws + p.off_xh),
                       (float *)(a.ws + p.off_rs));
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (p.gated)
        hipLaunchKernelGGL((tiled_kernel<false, true>), dim3(p.grid), dim3(kThreads), kLdsBytes, stream, a, p);
    else if (p.stream)
        hipLaunchKernelGGL((tiled_kernel<true, false>), dim3(p.grid), dim3(kThreads), kLdsBytes, stream, a, p);
    else
        hipLaunchKernelGGL((tiled_kernel<false, false>), dim3(p.grid), dim3(kThreads), kLdsBytes, stream, a, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.ksplit == 1)
        return e;
    const long long quads = (long long)a.M * a.N / 4;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream,
                       (const float *)(a.ws + p.off_part), (const float *)(a.ws + p.off_rs), a.M, a.N, p.ksplit, a.Y,
                       a.y_f32);
    return hipGetLastError();
}

} // namespace w4a16
