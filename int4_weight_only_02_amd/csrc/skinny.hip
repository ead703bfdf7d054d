// skinny.hip -- W4A16 linear for small M (decode, draft-block verification) on gfx950,
// and the fused lm_head greedy-verify epilogue.
//
// At M <= 16 per m-block the layer is bound by HBM: every packed weight byte is
// read once and used for at most 16 rows.  The kernel streams the packed words
// with 128-bit buffer loads straight into MFMA B fragments (no LDS staging of
// weights):
//   * a wave owns a 16-column tile (or a K slice of one); lane l holds column l%16
//     and, per group of 128 codes, one 16-byte load = 32 codes = the B operand of
//     four v_mfma_f32_16x16x32_bf16 (lane group l/16 covers codes 32*(l/16) .. +31);
//   * the activations X[m-block][K] are staged once per workgroup in LDS, permuted
//     to the fragment order and shared by all its waves;
//   * per group, eight MFMAs accumulate P = sum x * (q - z) in fp32: four with the
//     exact biased codes 128 + q and four with the column constant -(128 + z) (also
//     exact in bf16: at most 8 significant bits), in two independent chains, so the
//     bias and the zero-point cancel inside the accumulators.  The group is then
//     scaled in fp32: acc += s * P.  The matrix cores are otherwise idle in this
//     memory-bound kernel, so the zero-point costs no VALU work beyond building
//     its fragment;
//   * when K is a multiple of 512, the scales and zero words of four groups arrive
//     in one 8-byte and one 16-byte load: 1.5 memory instructions per 1 KB of codes.
// Every workgroup owns whole output columns, so no partial sum crosses a workgroup:
//   split mode   (few tiles: decode, the 7 projections of a decoder layer) -- a
//                workgroup takes tw tiles and splits K over sk waves per tile; each
//                wave requests its first three batches before X is staged; the sk
//                partial accumulators are summed through LDS in a fixed order;
//   stream mode  (many tiles: the 151936-column lm_head) -- persistent workgroups,
//                each wave walks its own sequence of whole tiles with the next
//                batch of loads always in flight, across tile boundaries.
// Results are deterministic (fixed summation order everywhere).
//
// lm_head mode (the pages' greedy verification of a draft block: Pith review,
// Assumptions & free parameters, first assumption; blocks of 16 tokens) keeps the
// fp32 logits, folds each finished column into a per-row (value, column) key,
// reduces the keys with 64-bit atomic max (ties -> lowest column), and the last
// workgroup turns them into argmax ids and the accepted-prefix length.
#include <cstdio>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

constexpr int kMaxWaves = 8;           // up to 512 threads per workgroup (256 VGPRs per lane)
constexpr int kStreamWaves = 8;
constexpr int kB = 4;                  // groups per register batch
constexpr int kCUs = 256;
constexpr size_t kLdsBudget = 160 * 1024 - 4096;
constexpr uint32_t kOob = 0xFFFFFF00u; // an offset past the end of every tensor
constexpr int kSplitDirect = 0, kSplitLds = 1, kStream = 2, kSplitPriv = 3, kSplitChunk = 4, kSplitPrivDma = 5;
constexpr int kMaxTickets = kMaxCounters; // arrival counters of chunked tiles

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

// Cross-workgroup hand-off (lm_head keys and the finishing ticket).  They move
// through device-scope atomics, which the gfx950 memory path keeps coherent across
// the XCDs' L2s.  The only ordering needed is that a workgroup's device-scope
// atomics have completed before it takes its ticket: s_waitcnt vmcnt(0) (vmcnt
// counts stores and no-return atomics on gfx9).  Agent-scope fences would instead
// write back and invalidate a whole L2.
__device__ __forceinline__ void wait_device_writes()
{
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0), expcnt and lgkmcnt unconstrained
}

// Buffer resource word 3 for raw (untyped) loads on gfx9-class GPUs.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// The lane's view of the packed grid for one 16-column tile: byte offsets of the
// lane's column.  Group g of the lane's codes sits at wo + 64 g, its scale at
// so + 2 g and its zero word at zo + 4 g.  A load past the end of a tensor (or at
// kOob) returns 0 instead of faulting; groups past the lane's range read finite
// neighbouring data or 0 and are masked in compute_batch.
struct LaneGrid {
    uint32_t wo, so, zo;
    int zsh;
};

__device__ __forceinline__ LaneGrid lane_grid(int tile, int col, int h, int N, int K, int G, bool live)
{
    LaneGrid L;
    int n = tile * 16 + col;
    n = n < N ? n : N - 1;
    L.wo = live ? (uint32_t)n * (uint32_t)(K / 2) + 16u * (uint32_t)h : kOob;
    L.so = live ? (uint32_t)n * (uint32_t)(2 * G) : kOob;
    L.zo = live ? (uint32_t)(n >> 3) * (uint32_t)(4 * G) : kOob;
    L.zsh = (n & 7) * 4;
    return L;
}

// kB consecutive groups of one lane's column: 16 bytes of codes, the fp16 scale and
// the zero word for each
struct Batch {
    u32x4_t w[kB];
    uint32_t s[kB];
    uint32_t z[kB];
};

// The scales and zero words of groups at byte offsets so, zo (kOob: none).  ALIGNED
// (G and the first group multiples of 4): one 8-byte and one 16-byte load.
template <bool ALIGNED>
__device__ __forceinline__ void load_params(uint32_t (&sc)[kB], uint32_t (&zw)[kB], __amdgpu_buffer_rsrc_t rs,
                                            __amdgpu_buffer_rsrc_t rz, uint32_t so, uint32_t zo)
{
    if constexpr (ALIGNED) {
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
        const u32x2_t sv = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0));
        const u32x4_t zv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rz, zo, 0, 0));
        sc[0] = sv.x & 0xFFFFu;
        sc[1] = sv.x >> 16;
        sc[2] = sv.y & 0xFFFFu;
        sc[3] = sv.y >> 16;
        zw[0] = zv.x;
        zw[1] = zv.y;
        zw[2] = zv.z;
        zw[3] = zv.w;
    } else {
        // the four zero words are consecutive (4-byte aligned): one 16-byte load, each
        // word range-checked on its own
        const u32x4_t zv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rz, zo, 0, 0));
#pragma unroll
        for (int i = 0; i < kB; ++i)
            sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, so + 2u * i, 0, 0);
        zw[0] = zv.x;
        zw[1] = zv.y;
        zw[2] = zv.z;
        zw[3] = zv.w;
    }
}

// Load groups gs .. gs+kB-1 (unconditionally: a batch starting at or past gend
// loads from kOob and costs no memory traffic)
template <bool ALIGNED>
__device__ __forceinline__ void load_batch(Batch &b, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t rz, const LaneGrid &L, int gs, int gend)
{
    const bool in = gs < gend;
    const uint32_t wo = in ? L.wo + 64u * (uint32_t)gs : kOob;
#pragma unroll
    for (int i = 0; i < kB; ++i)
        b.w[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 64u * i, 0, 0));
    load_params<ALIGNED>(b.s, b.z, rs, rz, in ? L.so + 2u * (uint32_t)gs : kOob, in ? L.zo + 4u * (uint32_t)gs : kOob);
}

// 8 codes -> MFMA fragment, with the mask and the bias held in registers so that
// each pair costs one v_and_or_b32 (plus a shift for the pairs 1..3)
__device__ __forceinline__ bf16x8_t codes_to_frag_r(uint32_t w, uint32_t mask, uint32_t bias)
{
    u32x4_t r;
    r.x = (w & mask) | bias;
    r.y = ((w >> 4) & mask) | bias;
    r.z = ((w >> 8) & mask) | bias;
    r.w = ((w >> 12) & mask) | bias;
    return __builtin_bit_cast(bf16x8_t, r);
}

// Per group, for this lane's column and the rows 4h .. 4h+3 (D layout):
//   P = sum_k x * (128 + q)        four MFMAs on the exact biased codes (fp32 sums)
//   acc += s * (P - (128 + z) * S)  S = sum_k x over the group, from LDS
// which is s * sum_k x * (q - z).  Groups at or past gend get s = 0 (their data is
// finite, so they add exactly 0).  xlane points at the lane's X row in the staged
// chunk, sl at S of rows 4h .. 4h+3 of its first group.  NR = the accumulator rows
// that can hold real output (1 for M = 1, 2 for M = 2).
template <int NR>
__device__ __forceinline__ void compute_batch(const Batch &b, f32x4_t &acc, const u32x4_t *xlane,
                                              const float *sl, int gs, int gend, int Mb, int zsh,
                                              uint32_t mask, uint32_t bias)
{
    // the X fragments and S of group i + 1 are read from LDS while group i computes
    u32x4_t xf[2][4];
    f32x4_t sv[2];
    auto fetch = [&](int i, int buf) {
        const int g = gs + i;
        const int gl = g < gend ? g : gend - 1;
        const u32x4_t *xg = xlane + gl * 16 * Mb;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xf[buf][j] = xg[j * Mb];
        sv[buf] = *(const f32x4_t *)(sl + gl * 16);
    };
    fetch(0, 0);
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        const int cur = i & 1;
        if (i + 1 < kB)
            fetch(i + 1, cur ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        const int g = gs + i;
        f32x4_t pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t wj = j == 0 ? b.w[i].x : j == 1 ? b.w[i].y : j == 2 ? b.w[i].z : b.w[i].w;
            pq = mfma16x16x32(__builtin_bit_cast(bf16x8_t, xf[cur][j]), codes_to_frag_r(wj, mask, bias), pq);
        }
        const float zc = (float)(kCodeBias + ((b.z[i] >> zsh) & 15u));
        const float s = g < gend ? f16_bits_to_f32((uint16_t)b.s[i]) : 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            acc[r] = fmaf(s, fmaf(-zc, sv[cur][r], pq[r]), acc[r]);
    }
}

// Direct variant of the split mode, for shapes where every workgroup needs many
// X rows and has few tiles to share them (M = 16 with one tile per workgroup): each
// wave reads only its K slice of X, straight from global memory (L2), together with
// its weights, so all of it is in flight at once instead of passing through a
// staging round.  A BatchX holds kB groups of the lane's column and the lane's X
// fragments for them (row m0 + xrow, codes 32h .. 32h+31 of each group).
struct BatchX {
    u32x4_t w[kB];
    u32x4_t x[kB][4];
    uint32_t s[kB];
    uint32_t z[kB];
};

// xo = byte offset of the lane's X fragment for group 0 (row * 2K + 64 h)
template <bool ALIGNED>
__device__ __forceinline__ void load_batch_x(BatchX &b, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs,
                                             __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rx,
                                             const LaneGrid &L, uint32_t xo, int gs, int gend)
{
    const bool in = gs < gend;
    const uint32_t wo = in ? L.wo + 64u * (uint32_t)gs : kOob;
    const uint32_t xg = in ? xo + 256u * (uint32_t)gs : kOob;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        b.w[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, wo + 64u * i, 0, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b.x[i][j] =
                __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xg + 256u * i + 16u * j, 0, 0));
    }
    load_params<ALIGNED>(b.s, b.z, rs, rz, in ? L.so + 2u * (uint32_t)gs : kOob, in ? L.zo + 4u * (uint32_t)gs : kOob);
}

// compute_batch with the X fragments taken from the batch (permuted in registers)
template <int NR>
__device__ __forceinline__ void compute_batch_x(const BatchX &b, f32x4_t &acc, int gs, int gend, int zsh,
                                                uint32_t mask, uint32_t bias)
{
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        const int g = gs + i;
        const uint32_t zb = (((b.z[i] >> zsh) & 15u) | 0xC300u) * 0x00010001u;
        const bf16x8_t zfrag = __builtin_bit_cast(bf16x8_t, u32x4_t{zb, zb, zb, zb});
        f32x4_t pq = {0.f, 0.f, 0.f, 0.f}, pz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, x_permute8(b.x[i][j]));
            const uint32_t wj = j == 0 ? b.w[i].x : j == 1 ? b.w[i].y : j == 2 ? b.w[i].z : b.w[i].w;
            pq = mfma16x16x32(xa, codes_to_frag_r(wj, mask, bias), pq);
            pz = mfma16x16x32(xa, zfrag, pz);
        }
        const float s = g < gend ? f16_bits_to_f32((uint16_t)b.s[i]) : 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            acc[r] = fmaf(s, pq[r] + pz[r], acc[r]);
    }
}

// 16 bytes per lane from global memory (offset voff of r) into LDS at dst + 16 * lane
// (dst the same for the whole wave): LDS DMA, no registers involved
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N): all but the N most recent vector memory loads of the wave have
// completed (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt, lgkmcnt unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm_below()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// vector memory loads per register batch (codes, scales, zero words), as written in
// load_batch / load_params: the waits for the X DMA below count on this
template <bool ALIGNED>
constexpr int batch_loads() { return ALIGNED ? kB + 2 : 2 * kB + 1; }

// compute_batch for the chunked mode: the X fragments come from LDS in natural order
// (as the DMA left them; permuted in registers) and the zero-point is folded by a
// second MFMA chain on the column constant -(128 + z), as in compute_batch_x.
// xlane points at the lane's X row in the first staged group (group gbase).
template <int NR>
__device__ __forceinline__ void compute_batch_lx(const Batch &b, f32x4_t &acc, const u32x4_t *xlane, int gs,
                                                 int gend, int gbase, int Mb, int zsh, uint32_t mask, uint32_t bias)
{
    u32x4_t xf[2][4];
    auto fetch = [&](int i, int buf) {
        const int g = gs + i;
        const int gl = (g < gend ? g : gend - 1) - gbase;
        const u32x4_t *xg = xlane + gl * 16 * Mb;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xf[buf][j] = xg[j * Mb];
    };
    fetch(0, 0);
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        const int cur = i & 1;
        if (i + 1 < kB)
            fetch(i + 1, cur ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        const int g = gs + i;
        const uint32_t zb = (((b.z[i] >> zsh) & 15u) | 0xC300u) * 0x00010001u;
        const bf16x8_t zfrag = __builtin_bit_cast(bf16x8_t, u32x4_t{zb, zb, zb, zb});
        f32x4_t pq = {0.f, 0.f, 0.f, 0.f}, pz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, x_permute8(xf[cur][j]));
            const uint32_t wj = j == 0 ? b.w[i].x : j == 1 ? b.w[i].y : j == 2 ? b.w[i].z : b.w[i].w;
            pq = mfma16x16x32(xa, codes_to_frag_r(wj, mask, bias), pq);
            pz = mfma16x16x32(xa, zfrag, pz);
        }
        const float s = g < gend ? f16_bits_to_f32((uint16_t)b.s[i]) : 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            acc[r] = fmaf(s, pq[r] + pz[r], acc[r]);
    }
}

// Staging of X[m0 .. m0+Mb)[all groups] into LDS, in fragment order.  LDS slot i
// holds chunk kc = i / Mb (group kc/16, c = kc%16) of row m = i % Mb, so consecutive
// threads write consecutive 16-byte slots (no bank conflicts); the quotient comes from
// a multiply by ceil(2^32 / Mb).  Alongside each slot goes the sum of its 8
// activations (part[i]), from which group_sums builds S.  A round is kStageU slots per
// thread; the first round is issued before the weight loads, so that waiting for X
// does not wait for the weights (loads complete in order).
constexpr int kStageU = 4;

struct XRound {
    u32x4_t v[kStageU];
};

struct XStage {
    __amdgpu_buffer_rsrc_t rx;
    uint32_t base;             // byte offset of X[m0][0]
    unsigned long long magic;  // ceil(2^32 / Mb)
    int Mb, K, total;
};

__device__ __forceinline__ void stage_issue(XRound &xr, const XStage &st, int i0, int tid, int nthreads)
{
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
        const int i = i0 + u * nthreads + tid;
        const int kc = (int)(((unsigned long long)(unsigned)i * st.magic) >> 32);
        const int m = i - kc * st.Mb;
        const uint32_t off = i < st.total ? st.base + (uint32_t)(m * st.K + kc * 8) * 2u : kOob;
        xr.v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(st.rx, off, 0, 0));
    }
}

__device__ __forceinline__ void stage_commit(const XRound &xr, const XStage &st, u32x4_t *xs, float *part, int i0,
                                             int tid, int nthreads)
{
    // the loaded registers are used unconditionally (only the LDS writes are
    // predicated), so no path leaves these loads pending behind the weight loads
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
        const int i = i0 + u * nthreads + tid;
        const u32x4_t pv = x_permute8(xr.v[u]);
        const float ps = sum8_bf16(xr.v[u]);
        if (i < st.total) {
            xs[i] = pv;
            part[i] = ps;
        }
    }
}

// Rounds after the first (only when X exceeds one round: several rows with a long
// K).  They are issued after the weight loads, so they wait for those too; the
// closing vmcnt(0) makes that explicit, so that the single-round path, which skips
// this, keeps its weight loads in flight into the compute loop.
__device__ __forceinline__ void stage_rest(const XStage &st, u32x4_t *xs, float *part, int tid, int nthreads)
{
    if (st.total <= kStageU * nthreads)
        return;
    for (int i0 = kStageU * nthreads; i0 < st.total; i0 += kStageU * nthreads) {
        XRound xr;
        stage_issue(xr, st, i0, tid, nthreads);
        stage_commit(xr, st, xs, part, i0, tid, nthreads);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0)
}

// S[g][r] = sum of the 128 activations of row min(r, Mb - 1) in group g: the 16 slot
// sums of the group, c ascending (a fixed order).  Rows >= Mb repeat row Mb - 1, whose
// activations the lanes of those rows also read.  Caller synchronizes around it.
__device__ __forceinline__ void group_sums(const float *part, float *S, int Mb, int ng, int tid, int nthreads)
{
    for (int e = tid; e < ng * Mb; e += nthreads) {
        const int g = e / Mb, m = e - g * Mb;
        const float *pp = part + g * 16 * Mb + m;
        float v[16];
#pragma unroll
        for (int c = 0; c < 16; ++c)
            v[c] = pp[c * Mb];
        __builtin_amdgcn_sched_barrier(0); // all 16 reads in flight before the sum
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            t += v[c];
        S[g * 16 + m] = t;
        if (m == Mb - 1)
            for (int r = Mb; r < 16; ++r)
                S[g * 16 + r] = t;
    }
}

// The work of one workgroup on one projection.  MODE: kSplitDirect, kSplitLds,
// kSplitPriv, kSplitPrivDma, kSplitChunk or kStream (see the plan).  The workgroup takes items first, first +
// stride, ... (split mode) or tile groups first, first + stride, ... (stream mode).
template <int NR, int MODE, bool ALIGNED, bool GATED = false>
__device__ __forceinline__ void skinny_body(const SkinnyArgs &a, const SkinnyPlan &p, int first, int stride,
                                            unsigned char *smem, unsigned long long (*kred)[16], int &s_flag)
{
    constexpr bool STREAM = MODE == kStream;

    const int M = a.M, N = a.N, K = a.K, G = a.G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: scalar loop control
    const int h = lane >> 4, col = lane & 15;
    const int nthreads = blockDim.x, nwaves = nthreads >> 6;
    const int mrows = M < 16 ? M : 16;

    // LDS: staged X [group][chunk c][row] (16 B each), the slot sums, S [group][16 rows]
    // -- shared by the workgroup, or (kSplitPriv) one such region per wave holding
    // p.chunk groups of its own K slice -- then the K-slice partial sums
    // [wave][64 lanes][4]
    const int nslot = p.chunk * 16 * mrows;
    const size_t region = (size_t)nslot * 20 + (size_t)p.chunk * 64;
    constexpr bool PRIV = MODE == kSplitPriv || MODE == kSplitPrivDma;
    unsigned char *xbase = PRIV ? smem + (size_t)wave * region : smem;
    u32x4_t *xs = (u32x4_t *)xbase;
    float *part = (float *)(xbase + (size_t)nslot * 16);
    float *S = part + nslot;
    // kSplitChunk: the raw X of the item's K chunk (DMA slots, whole 1 KB rounds), then
    // the K-slice partial sums
    const size_t xchunk = (size_t)((p.cg * 16 * mrows + 63) & ~63) * 16;
    float *red = (float *)(smem + (PRIV                  ? (size_t)nwaves * region
                                   : MODE == kSplitChunk ? xchunk
                                                         : region));
    uint32_t *ticket = (uint32_t *)(a.ws + kOffTicket);
    unsigned long long *keys = (unsigned long long *)(a.ws + kOffKeys);

    // gated pairs: the waves of odd tile slots stream the up projection
    const bool upw = !STREAM && GATED && ((wave % p.tw) & 1);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(upw ? a.qw2 : a.qw, (uint32_t)((size_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(upw ? a.scales2 : a.scales, (uint32_t)((size_t)N * G * 2));
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(upw ? a.qz2 : a.qz, (uint32_t)((size_t)(N / 8) * G * 4));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, (uint32_t)((size_t)M * K * 2));
    auto x_stage = [&](int m0, int Mb) {
        XStage st;
        st.rx = rx;
        st.base = (uint32_t)m0 * (uint32_t)K * 2u;
        st.magic = ((1ull << 32) + (unsigned)Mb - 1) / (unsigned)Mb;
        st.Mb = Mb;
        st.K = K;
        st.total = Mb * G * 16;
        return st;
    };
    // code-to-bf16 constants, pinned in VGPRs (see codes_to_frag_r)
    uint32_t kmask = 0x000F000Fu, kbias = kBiasBits;
    asm volatile("" : "+v"(kmask));
    asm volatile("" : "+v"(kbias));

    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
    int cur_mb = -1;

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
                kred[wave][4 * h + r] = best[r];
        }
        __syncthreads();
        if (tid < 16 && mb * 16 + tid < M) {
            unsigned long long k = kred[0][tid];
            for (int v = 1; v < nwaves; ++v)
                k = max_u64(k, kred[v][tid]);
            if (k)
                __hip_atomic_fetch_max(&keys[mb * 16 + tid], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r)
            best[r] = 0ull;
    };

    // finished tile: store the rows < Mb of column n, or fold them into the argmax keys
    auto finish_tile = [&](const f32x4_t &acc, int m0, int Mb, int n) {
        if (n >= N)
            return;
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
    };

    if constexpr (STREAM) {
        // ---- stream mode: X of the m-block is staged once (all of K); workgroup b owns
        // the tiles [b nt / grid, (b + 1) nt / grid) (every CU the same bytes, within a
        // tile), and wave w walks tiles t0 + w, t0 + w + nwaves, ... of that run.
        const int t0 = (int)((long long)first * p.nt / stride);
        const int t1 = (int)((long long)(first + 1) * p.nt / stride);
        const int jn = (t1 - t0 + nwaves - 1) / nwaves; // tile rounds of the workgroup
        for (int mb = 0; mb < p.mblocks; ++mb) {
            const int m0 = mb * 16;
            const int Mb = M - m0 < 16 ? M - m0 : 16;
            const int xrow = col < Mb ? col : Mb - 1; // rows >= Mb feed outputs that are never stored
            const u32x4_t *xlane = xs + (4 * h) * Mb + xrow;
            const float *sl = S + 4 * h;
            if (a.lmhead && cur_mb >= 0)
                flush_best(cur_mb);
            cur_mb = mb;

            int tgA = 0, gA = 0;
            int tileA = t0 + tgA * nwaves + wave;
            bool liveA = tgA < jn && tileA < t1;
            LaneGrid LA = lane_grid(tileA, col, h, N, K, G, liveA);
            // X first, then the first weight batch: both in flight together
            const XStage st = x_stage(m0, Mb);
            XRound xr;
            stage_issue(xr, st, 0, tid, nthreads);
            Batch bA, bB;
            load_batch<ALIGNED>(bA, rw, rs, rz, LA, gA, G);
            __syncthreads(); // the previous m-block's reads of X are done
            stage_commit(xr, st, xs, part, 0, tid, nthreads);
            stage_rest(st, xs, part, tid, nthreads);
            __syncthreads();
            group_sums(part, S, Mb, G, tid, nthreads);
            __syncthreads();

            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            while (true) {
                // phase A: prefetch the batch after A into bB, compute A
                int tgB = tgA, gB = gA + kB;
                if (gB >= G) {
                    tgB += 1;
                    gB = 0;
                }
                const int tileB = t0 + tgB * nwaves + wave;
                const bool liveB = tgB < jn && tileB < t1;
                const LaneGrid LB = lane_grid(tileB, col, h, N, K, G, liveB);
                load_batch<ALIGNED>(bB, rw, rs, rz, LB, gB, G);
                __builtin_amdgcn_sched_barrier(0);
                compute_batch<NR>(bA, acc, xlane, sl, gA, G, Mb, LA.zsh, kmask, kbias);
                __builtin_amdgcn_sched_barrier(0);
                if (gA + kB >= G) {
                    if (liveA)
                        finish_tile(acc, m0, Mb, tileA * 16 + col);
                    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                if (tgB >= jn)
                    break;
                // phase B: prefetch the batch after B into bA, compute B
                int tgC = tgB, gC = gB + kB;
                if (gC >= G) {
                    tgC += 1;
                    gC = 0;
                }
                const int tileC = t0 + tgC * nwaves + wave;
                const bool liveC = tgC < jn && tileC < t1;
                const LaneGrid LC = lane_grid(tileC, col, h, N, K, G, liveC);
                load_batch<ALIGNED>(bA, rw, rs, rz, LC, gC, G);
                __builtin_amdgcn_sched_barrier(0);
                compute_batch<NR>(bB, acc, xlane, sl, gB, G, Mb, LB.zsh, kmask, kbias);
                __builtin_amdgcn_sched_barrier(0);
                if (gB + kB >= G) {
                    if (liveB)
                        finish_tile(acc, m0, Mb, tileB * 16 + col);
                    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                if (tgC >= jn)
                    break;
                tgA = tgC;
                gA = gC;
                tileA = tileC;
                liveA = liveC;
                LA = LC;
            }
        }
    } else {
        // ---- split mode: item = (m-block, group of tw tiles); wave = (tile slot, K slice)
        const int tslot = wave % p.tw, ks = wave / p.tw;
        for (int it = first; it < p.items; it += stride) {
            // kSplitChunk: item = (tile group, K chunk), the chunk index fastest
            const int chunk = MODE == kSplitChunk ? it % p.C : 0;
            const int rest = MODE == kSplitChunk ? it / p.C : it;
            const int mb = rest / p.ntg, tg = rest - mb * p.ntg;
            const int m0 = mb * 16;
            const int Mb = M - m0 < 16 ? M - m0 : 16;
            const int xrow = col < Mb ? col : Mb - 1;
            const int tile = tg * p.tw + tslot;
            const int ptile = GATED ? tile >> 1 : tile; // the tile in the wave's own projection
            const bool live = ptile * 16 < N;
            const LaneGrid L = lane_grid(ptile, col, h, N, K, G, live);
            if (a.lmhead && mb != cur_mb) {
                if (cur_mb >= 0)
                    flush_best(cur_mb);
                cur_mb = mb;
            }
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (PRIV) {
                // each wave stages only its own K slice of X (few rows), in its own LDS
                // region: the loads, the commit, the row sums and the compute of one wave
                // need no workgroup barrier (LDS operations of a wave complete in order)
                const int g0 = ks * p.per;
                const int g1 = G < g0 + p.per ? G : g0 + p.per;
                const int ng = g1 > g0 ? g1 - g0 : 0; // slices past K are empty
                if constexpr (MODE == kSplitPrivDma) {
                    // X by LDS DMA and the zero-point folded by MFMA (no row sums): the
                    // shorter chain wins for 2..4 rows and for slices of one batch; one row
                    // over many groups keeps the register staging and the row-sum fold,
                    // which leaves the matrix cores half the work in the compute tail.
                    // The previous item's LDS reads and loads are done before the region and
                    // the batch registers are reused.
                    wait_vm_below<0>();
                    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
                    const int total = ng * 16 * Mb;
                    const uint32_t xb = ((uint32_t)m0 * (uint32_t)K + (uint32_t)(g0 < G ? g0 : 0) * kGroup) * 2u;
                    const unsigned long long magic = 0xFFFFFFFFull / (uint32_t)Mb + 1ull; // ceil(2^32 / Mb)
                    for (int i = 0; i * 64 < total; ++i) {
                        // slot q = (group, chunk c) * Mb + row, as in the register staging
                        const int q = i * 64 + lane;
                        const int kc = (int)(((unsigned long long)(uint32_t)q * magic) >> 32);
                        const int m = q - kc * Mb;
                        dma16(rx, xbase + (size_t)i * 1024, q < total ? xb + (uint32_t)(m * K + kc * 8) * 2u : kOob);
                    }
                    asm volatile("" ::: "memory"); // the weight loads stay behind the DMA
                    Batch b0, b1, b2;
                    load_batch<ALIGNED>(b0, rw, rs, rz, L, g0, g1);
                    load_batch<ALIGNED>(b1, rw, rs, rz, L, g0 + kB, g1);
                    load_batch<ALIGNED>(b2, rw, rs, rz, L, g0 + 2 * kB, g1);
                    asm volatile("" ::: "memory"); // ... and ahead of the wait
                    wait_vm_below<3 * batch_loads<ALIGNED>()>(); // this wave's X has landed
                    const u32x4_t *xlane = xs + (4 * h) * Mb + xrow;
                    for (int g = g0; g < g1; g += 3 * kB) {
                        __builtin_amdgcn_sched_barrier(0);
                        compute_batch_lx<NR>(b0, acc, xlane, g, g1, g0, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b0, rw, rs, rz, L, g + 3 * kB, g1);
                        __builtin_amdgcn_sched_barrier(0);
                        if (g + kB < g1)
                            compute_batch_lx<NR>(b1, acc, xlane, g + kB, g1, g0, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b1, rw, rs, rz, L, g + 4 * kB, g1);
                        __builtin_amdgcn_sched_barrier(0);
                        if (g + 2 * kB < g1)
                            compute_batch_lx<NR>(b2, acc, xlane, g + 2 * kB, g1, g0, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b2, rw, rs, rz, L, g + 5 * kB, g1);
                    }
                } else {
                    XStage st = x_stage(m0, Mb);
                    st.base += (uint32_t)(g0 < G ? g0 * kGroup : 0) * 2u;
                    st.total = Mb * ng * 16;
                    XRound xr;
                    stage_issue(xr, st, 0, lane, 64);
                    Batch b0, b1, b2;
                    load_batch<ALIGNED>(b0, rw, rs, rz, L, g0, g1);
                    load_batch<ALIGNED>(b1, rw, rs, rz, L, g0 + kB, g1);
                    load_batch<ALIGNED>(b2, rw, rs, rz, L, g0 + 2 * kB, g1);
                    stage_commit(xr, st, xs, part, 0, lane, 64);
                    stage_rest(st, xs, part, lane, 64);
                    group_sums(part, S, Mb, ng, lane, 64);
                    // compute_batch indexes by absolute group: shift the bases by g0
                    const u32x4_t *xlane = xs + (4 * h) * Mb + xrow - (size_t)g0 * 16 * Mb;
                    const float *sl = S + 4 * h - (size_t)g0 * 16;
                    for (int g = g0; g < g1; g += 3 * kB) {
                        __builtin_amdgcn_sched_barrier(0);
                        compute_batch<NR>(b0, acc, xlane, sl, g, g1, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b0, rw, rs, rz, L, g + 3 * kB, g1);
                        __builtin_amdgcn_sched_barrier(0);
                        if (g + kB < g1)
                            compute_batch<NR>(b1, acc, xlane, sl, g + kB, g1, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b1, rw, rs, rz, L, g + 4 * kB, g1);
                        __builtin_amdgcn_sched_barrier(0);
                        if (g + 2 * kB < g1)
                            compute_batch<NR>(b2, acc, xlane, sl, g + 2 * kB, g1, Mb, L.zsh, kmask, kbias);
                        __builtin_amdgcn_sched_barrier(0);
                        load_batch<ALIGNED>(b2, rw, rs, rz, L, g + 5 * kB, g1);
                    }
                }
            } else if constexpr (MODE == kSplitChunk) {
                // X of the chunk's groups [ga, gb) arrives in LDS by DMA, all of it in
                // flight together with the first three weight batches of each wave; the
                // waves' K slices of the chunk are [s0, s1)
                const int ga = chunk * p.cg;
                const int gb = G < ga + p.cg ? G : ga + p.cg;
                const int s0 = ga + ks * p.per;
                const int s1 = gb < s0 + p.per ? gb : s0 + p.per; // s1 <= s0: empty slice
                if (it != first)
                    __syncthreads(); // the previous item's reads of X are done
                // the previous item's last (unused) batch loads have landed: nothing older
                // than the DMA is pending, so the batch registers need no wait below
                wait_vm_below<0>();
                const int total = (gb - ga) * 16 * Mb;
                const uint32_t xb = ((uint32_t)m0 * (uint32_t)K + (uint32_t)ga * kGroup) * 2u;
                const unsigned long long magic = 0xFFFFFFFFull / (uint32_t)Mb + 1ull; // ceil(2^32 / Mb)
                for (int i = wave; i * 64 < total; i += nwaves) {
                    // slot q = (group, chunk c) * Mb + row, as in the register staging
                    const int q = i * 64 + lane;
                    const int kc = (int)(((unsigned long long)(uint32_t)q * magic) >> 32);
                    const int m = q - kc * Mb;
                    dma16(rx, smem + (size_t)i * 1024, q < total ? xb + (uint32_t)(m * K + kc * 8) * 2u : kOob);
                }
                asm volatile("" ::: "memory"); // the weight loads stay behind the DMA
                Batch b0, b1, b2;
                load_batch<ALIGNED>(b0, rw, rs, rz, L, s0, s1);
                load_batch<ALIGNED>(b1, rw, rs, rz, L, s0 + kB, s1);
                load_batch<ALIGNED>(b2, rw, rs, rz, L, s0 + 2 * kB, s1);
                asm volatile("" ::: "memory"); // ... and ahead of the wait
                wait_vm_below<3 * batch_loads<ALIGNED>()>(); // this wave's DMA has landed
                __syncthreads();                              // and every other wave's
                const u32x4_t *xlane = xs + (4 * h) * Mb + xrow;
                for (int g = s0; g < s1; g += 3 * kB) {
                    __builtin_amdgcn_sched_barrier(0);
                    compute_batch_lx<NR>(b0, acc, xlane, g, s1, ga, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b0, rw, rs, rz, L, g + 3 * kB, s1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + kB < s1)
                        compute_batch_lx<NR>(b1, acc, xlane, g + kB, s1, ga, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b1, rw, rs, rz, L, g + 4 * kB, s1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + 2 * kB < s1)
                        compute_batch_lx<NR>(b2, acc, xlane, g + 2 * kB, s1, ga, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b2, rw, rs, rz, L, g + 5 * kB, s1);
                }
            } else if constexpr (MODE == kSplitLds) {
                // slices of p.per groups (a multiple of kB): batches stay 4-aligned
                const int g0 = ks * p.per;
                const int g1 = G < g0 + p.per ? G : g0 + p.per;
                // X first, then three register batches (up to 3 * kB groups of the slice),
                // all in flight together; X is committed to LDS as soon as it lands
                const XStage st = x_stage(m0, Mb);
                XRound xr;
                stage_issue(xr, st, 0, tid, nthreads);
                Batch b0, b1, b2;
                load_batch<ALIGNED>(b0, rw, rs, rz, L, g0, g1);
                load_batch<ALIGNED>(b1, rw, rs, rz, L, g0 + kB, g1);
                load_batch<ALIGNED>(b2, rw, rs, rz, L, g0 + 2 * kB, g1);
                if (it != first)
                    __syncthreads(); // the previous item's reads of X are done
                stage_commit(xr, st, xs, part, 0, tid, nthreads);
                stage_rest(st, xs, part, tid, nthreads);
                __syncthreads();
                group_sums(part, S, Mb, G, tid, nthreads);
                __syncthreads();
                const u32x4_t *xlane = xs + (4 * h) * Mb + xrow;
                const float *sl = S + 4 * h;
                // rotate the three batches; loads stay unconditional (a batch past the
                // slice reads kOob), only fully masked computes are skipped (uniform
                // branches)
                for (int g = g0; g < g1; g += 3 * kB) {
                    __builtin_amdgcn_sched_barrier(0);
                    compute_batch<NR>(b0, acc, xlane, sl, g, g1, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b0, rw, rs, rz, L, g + 3 * kB, g1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + kB < g1)
                        compute_batch<NR>(b1, acc, xlane, sl, g + kB, g1, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b1, rw, rs, rz, L, g + 4 * kB, g1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + 2 * kB < g1)
                        compute_batch<NR>(b2, acc, xlane, sl, g + 2 * kB, g1, Mb, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch<ALIGNED>(b2, rw, rs, rz, L, g + 5 * kB, g1);
                }
            } else {
                const int g0 = ks * p.per;
                const int g1 = G < g0 + p.per ? G : g0 + p.per;
                const uint32_t xo = (uint32_t)(m0 + xrow) * (uint32_t)(2 * K) + 64u * (uint32_t)h;
                // two register batches (weights, scales, zeros and X fragments): batch b+1 is
                // in flight while batch b computes
                BatchX b0, b1;
                load_batch_x<ALIGNED>(b0, rw, rs, rz, rx, L, xo, g0, g1);
                load_batch_x<ALIGNED>(b1, rw, rs, rz, rx, L, xo, g0 + kB, g1);
                for (int g = g0; g < g1; g += 2 * kB) {
                    __builtin_amdgcn_sched_barrier(0);
                    compute_batch_x<NR>(b0, acc, g, g1, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch_x<ALIGNED>(b0, rw, rs, rz, rx, L, xo, g + 2 * kB, g1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (g + kB < g1)
                        compute_batch_x<NR>(b1, acc, g + kB, g1, L.zsh, kmask, kbias);
                    __builtin_amdgcn_sched_barrier(0);
                    load_batch_x<ALIGNED>(b1, rw, rs, rz, rx, L, xo, g + 3 * kB, g1);
                }
            }
            if (p.sk > 1) {
                // sum the K slices of each tile through LDS, slice 0 first, in slice order
                *(f32x4_t *)(red + ((size_t)wave * 64 + lane) * 4) = acc;
                __syncthreads();
                if (ks == 0) {
                    for (int s = 1; s < p.sk; ++s) {
                        const f32x4_t o = *(const f32x4_t *)(red + ((size_t)(s * p.tw + tslot) * 64 + lane) * 4);
                        acc[0] += o[0];
                        acc[1] += o[1];
                        acc[2] += o[2];
                        acc[3] += o[3];
                    }
                }
                __syncthreads();
            }
            if (MODE == kSplitChunk && p.C > 1) {
                // K chunks of one tile group meet in the workspace: each workgroup stores
                // its fp32 partial sums [chunk][row][column] (device-coherent stores), then
                // takes an arrival ticket; the last to arrive adds the C partials in chunk
                // order (its own from registers) and finishes the tiles, so the result
                // does not depend on the arrival order
                // (gated: over the 2N columns of the pair, gate and up tiles alternating)
                float *pbuf = (float *)(a.ws + p.part_off);
                uint32_t *tk = (uint32_t *)(a.ws + kOffCounters) + (size_t)(p.tkt + rest) * kCounterStride;
                const int Nv = GATED ? 2 * N : N;
                const int n = tile * 16 + col;
                if (ks == 0 && live && n < Nv) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * h + r < Mb)
                            __hip_atomic_store(pbuf + ((size_t)chunk * M + m0 + 4 * h + r) * Nv + n, acc[r],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                wait_device_writes();
                __syncthreads();
                if (tid == 0) {
                    const uint32_t old = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    s_flag = old == (uint32_t)(p.C - 1) ? 1 : 0;
                }
                __syncthreads();
                if (!s_flag)
                    continue; // uniform over the workgroup
                if (ks == 0 && live && n < Nv) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (4 * h + r >= Mb)
                            continue;
                        float t = 0.f;
                        for (int cc = 0; cc < p.C; ++cc)
                            t += cc == chunk ? acc[r]
                                             : __hip_atomic_load(pbuf + ((size_t)cc * M + m0 + 4 * h + r) * Nv + n,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        acc[r] = t;
                    }
                }
                if (tid == 0)
                    __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if constexpr (GATED) {
                // the gate tile's sums (even slot) meet the up tile's (the next slot)
                // through LDS: Y = silu(gate) * up.  Every wave of the workgroup passes
                // both barriers (the branch is uniform).
                if (ks == 0 && !(tslot & 1))
                    *(f32x4_t *)(red + ((size_t)tslot * 64 + lane) * 4) = acc;
                __syncthreads();
                if (ks == 0 && (tslot & 1) && live) {
                    const f32x4_t gv = *(const f32x4_t *)(red + ((size_t)(tslot - 1) * 64 + lane) * 4);
                    f32x4_t y;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        y[r] = silu_f32(gv[r]) * acc[r];
                    finish_tile(y, m0, Mb, ptile * 16 + col);
                }
                __syncthreads(); // before the next item reuses the exchange region
            } else if (ks == 0 && live) {
                finish_tile(acc, m0, Mb, tile * 16 + col);
            }
        }
    }

    if (a.lmhead) {
        if (cur_mb >= 0)
            flush_best(cur_mb);
        wait_device_writes();
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_flag = (old == (uint32_t)(gridDim.x - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (s_flag && tid < 64) {
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

template <int NR, int MODE, bool ALIGNED, bool GATED = false>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyArgs a, SkinnyPlan p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ unsigned long long kred[kMaxWaves][16];
    __shared__ int s_flag;
    skinny_body<NR, MODE, ALIGNED, GATED>(a, p, blockIdx.x, gridDim.x, smem, kred, s_flag);
}

// Several projections (same M) in one launch: workgroup b works on item
// b - begin[q] of projection q, with that projection's own plan (all plans use the
// same number of waves).  Consecutive projections overlap: no launch gap, and the
// tail of one is filled by the next.
template <int NR, bool ALIGNED>
__global__ __launch_bounds__(512) void skinny_multi_kernel(SkinnyMulti mp)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ unsigned long long kred[kMaxWaves][16];
    __shared__ int s_flag;
    const int b = blockIdx.x;
    int q = 0;
    for (int i = 1; i < mp.count; ++i)
        if (b >= mp.begin[i])
            q = i;
    const SkinnyArgs a = mp.args[q];
    const SkinnyPlan p = mp.plan[q];
    const int it = b - mp.begin[q];
    if (p.xlds == 3)
        skinny_body<NR, kSplitChunk, ALIGNED>(a, p, it, 1 << 30, smem, kred, s_flag);
    else if (p.xlds == 2 && p.xdma)
        skinny_body<NR, kSplitPrivDma, ALIGNED>(a, p, it, 1 << 30, smem, kred, s_flag);
    else if (p.xlds == 2)
        skinny_body<NR, kSplitPriv, ALIGNED>(a, p, it, 1 << 30, smem, kred, s_flag);
    else if (p.xlds == 1)
        skinny_body<NR, kSplitLds, ALIGNED>(a, p, it, 1 << 30, smem, kred, s_flag);
    else
        skinny_body<NR, kSplitDirect, ALIGNED>(a, p, it, 1 << 30, smem, kred, s_flag);
}

// LDS per staged group: 16 slots of 16 B and their 4-byte sums per row, and S (16 rows)
size_t lds_per_group(int M)
{
    const int mrows = M < 16 ? M : 16;
    return (size_t)mrows * 16 * (16 + 4) + 16 * 4;
}

// LDS of a plan: X (shared, per wave, or one chunk) and the K-slice partial sums of
// every wave the workgroup launches with (p.waves; waves past tw * sk stay idle)
size_t lds_for(const SkinnyPlan &p, int M)
{
    const size_t red = (p.sk > 1 || p.pair) ? (size_t)p.waves * 1024 : 0;
    if (p.xlds == 3) {
        const int mrows = M < 16 ? M : 16;
        return (size_t)((p.cg * 16 * mrows + 63) & ~63) * 16 + red;
    }
    const size_t xs = (size_t)p.chunk * lds_per_group(M);
    return (p.xlds == 2 ? xs * p.waves : xs) + red;
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Chunked split mode: tw tiles per workgroup share X, whose K range is cut into C
// chunks of cg groups (one workgroup per tile group and chunk).  Fills p.tw, sk, per,
// cg, C, ntg, items, grid; with fixed, sk = kMaxWaves / tw (slices past the chunk stay
// empty).  Returns false when the chunk does not fit in LDS or there are too many
// arrival counters.
bool plan_chunk(SkinnyPlan &p, int M, size_t lds_limit, int tw, int cg, bool fixed)
{
    const int mrows = M < 16 ? M : 16;
    const int G = p.G;
    const int ntg = (p.nt + tw - 1) / tw;
    if (cg <= 0 || cg >= G)
        cg = G;
    else
        cg = round_up(cg, kB);
    if (cg >= G)
        cg = G;
    const int C = (G + cg - 1) / cg;
    // a launch of several projections gives each its own share of the counters
    if (C > 1 && (long long)p.mblocks * ntg > (fixed ? kMaxTickets / kMaxProblems : kMaxTickets))
        return false;
    // K slices of the chunk over the remaining waves: whole batches each
    int sk = kMaxWaves / tw;
    if (!fixed) {
        const int batches = (cg + kB - 1) / kB;
        sk = sk > batches ? batches : sk;
        sk = sk < 1 ? 1 : sk;
    }
    p.per = round_up((cg + sk - 1) / sk, kB);
    if (!fixed)
        sk = (cg + p.per - 1) / p.per;
    p.tw = tw;
    p.sk = sk;
    p.cg = cg;
    p.C = C;
    p.ntg = ntg;
    p.items = p.mblocks * ntg * C;
    p.grid = p.items;
    p.xlds = 3;
    p.chunk = 0;
    p.tkt = 0;
    p.part_off = kZeroRegion;
    p.waves = fixed ? kMaxWaves : tw * sk;
    return lds_for(p, M) <= lds_limit && mrows > 0;
}

// The chunked mode's choice for one m-block of 5..16 rows (measured on MI355X at
// M = 5, 8, 16 and K = 2560 .. 9728): when every tile can have its own workgroup
// (at most one tile per CU), one tile per workgroup with X of all of K in LDS, or,
// when that does not fit, two tiles per workgroup and chunks of 32 groups.  With
// more tiles than CUs the workgroup-shared staging of the other split modes wins.
bool choose_chunk(SkinnyPlan &p, int M, size_t lds_limit, bool fixed, int tw_hint)
{
    int tw = 0;
    SkinnyPlan c = p;
    if (p.mblocks != 1 || M <= 4 || (tw_hint <= 0 && p.nt > kCUs))
        return false;
    tw = tw_hint > 0 ? tw_hint : 1;
    if (plan_chunk(c, M, lds_limit, tw, 0, fixed)) {
        p = c;
        return true;
    }
    c = p;
    if (plan_chunk(c, M, lds_limit, tw > 2 ? tw : 2, 32, fixed)) {
        p = c;
        return true;
    }
    return false;
}

} // namespace

SkinnyPlan plan_skinny(int M, int N, int K, int lmhead, size_t lds_limit)
{
    SkinnyPlan p{};
    if (lds_limit == 0 || lds_limit > kLdsBudget)
        lds_limit = kLdsBudget;
    p.G = K / kGroup;
    p.mblocks = (M + 15) / 16;
    p.nt = (N + 15) / 16;
    const int mrows = M < 16 ? M : 16;
    const size_t per_group = lds_per_group(M);
    const long long tiles = (long long)p.nt * p.mblocks;
    if (tiles >= 16LL * kCUs && (size_t)p.G * per_group <= lds_limit) {
        // many tiles (a vocabulary-sized lm_head): persistent workgroups, whole tiles per wave
        p.stream = 1;
        p.xlds = 1;
        p.sk = 1;
        p.tw = kStreamWaves;
        p.chunk = p.G;
        p.per = p.G;
        p.ntg = (p.nt + p.tw - 1) / p.tw;
        p.items = p.mblocks * p.ntg;
        const size_t lds = lds_for(p, M);
        int per_cu = (int)(lds_limit / (lds ? lds : 1));
        per_cu = per_cu < 1 ? 1 : per_cu > 2 ? 2 : per_cu;
        p.grid = p.ntg < kCUs * per_cu ? p.ntg : kCUs * per_cu;
    } else {
        // few tiles: each workgroup takes tw tiles and splits K over sk waves per tile;
        // tw is the smallest count that keeps the grid within one workgroup per CU,
        // sk gives each wave at least one batch of groups
        p.stream = 0;
        int tw = (int)((tiles + kCUs - 1) / kCUs);
        tw = tw < 1 ? 1 : tw > kMaxWaves ? kMaxWaves : tw;
        const int batches = (p.G + kB - 1) / kB;
        int sk = kMaxWaves / tw;
        sk = sk > batches ? batches : sk;
        sk = sk < 1 ? 1 : sk;
        const size_t red = sk > 1 ? (size_t)tw * sk * 1024 : 0;
        // whole batches per slice; drop the slices that rounding left empty
        p.per = round_up((p.G + sk - 1) / sk, kB);
        sk = (p.G + p.per - 1) / p.per;
        // X in LDS: per wave (its own slice) for up to 4 rows, else shared by the
        // workgroup when all of K fits and staging it is cheap next to the weights the
        // workgroup streams (several tiles sharing each staged row); else from L2
        const bool priv = mrows <= 4 && (size_t)tw * sk * p.per * per_group + red <= lds_limit;
        const bool fits = (size_t)p.G * per_group + red <= lds_limit;
        p.xlds = priv ? 2 : (fits && (mrows <= 4 || tw >= 2)) ? 1 : 0;
        p.chunk = p.xlds == 2 ? p.per : p.xlds == 1 ? p.G : 0;
        p.xdma = priv && (M >= 2 || p.per <= kB); // measured on MI355X at M = 1..4
        p.tw = tw;
        p.sk = sk;
        p.ntg = (p.nt + tw - 1) / tw;
        p.items = p.mblocks * p.ntg;
        p.grid = p.items;
        if (!lmhead)
            choose_chunk(p, M, lds_limit, false, 0);
    }
    p.waves = p.tw * p.sk;
    p.lds_bytes = lds_for(p, M);
    // lm_head: the zero region (argmax keys, ticket); chunked: counters and partial sums
    p.ws_bytes = lmhead ? kZeroRegion
                 : (p.xlds == 3 && p.C > 1) ? kZeroRegion + (size_t)p.C * M * N * 4
                                             : 0;
    return p;
}

// Split-mode plan with exactly kMaxWaves waves (for projections sharing one launch):
// tw from the caller (tw_hint, balancing the launch) or the smallest power of two that
// keeps the projection within one workgroup per CU; sk = kMaxWaves / tw (waves and
// slices past K stay empty).
SkinnyPlan plan_skinny_fixed(int M, int N, int K, size_t lds_limit, int tw_hint, bool pair)
{
    SkinnyPlan p{};
    p.pair = pair ? 1 : 0;
    if (lds_limit == 0 || lds_limit > kLdsBudget)
        lds_limit = kLdsBudget;
    p.G = K / kGroup;
    p.mblocks = (M + 15) / 16;
    p.nt = (N + 15) / 16;
    const int mrows = M < 16 ? M : 16;
    const size_t per_group = lds_per_group(M);
    const long long tiles = (long long)p.nt * p.mblocks;
    int tw = 1;
    while (tw < kMaxWaves && (long long)tw * kCUs < tiles)
        tw *= 2;
    if (tw_hint > 0)
        tw = tw_hint < kMaxWaves ? tw_hint : kMaxWaves;
    const int sk = kMaxWaves / tw;
    const size_t red = (sk > 1 || pair) ? (size_t)kMaxWaves * 1024 : 0;
    p.stream = 0;
    p.tw = tw;
    p.sk = sk;
    p.per = round_up((p.G + sk - 1) / sk, kB);
    const bool priv = mrows <= 4 && (size_t)kMaxWaves * p.per * per_group + red <= lds_limit;
    const bool fits = (size_t)p.G * per_group + red <= lds_limit;
    p.xlds = priv ? 2 : (fits && (mrows <= 4 || tw >= 2)) ? 1 : 0;
    p.chunk = p.xlds == 2 ? p.per : p.xlds == 1 ? p.G : 0;
    p.xdma = priv && (M >= 2 || p.per <= kB);
    p.ntg = (p.nt + tw - 1) / tw;
    p.items = p.mblocks * p.ntg;
    p.grid = p.items;
    p.waves = kMaxWaves;
    choose_chunk(p, M, lds_limit, true, tw_hint);
    p.lds_bytes = lds_for(p, M);
    p.ws_bytes = (p.xlds == 3 && p.C > 1) ? kZeroRegion + (size_t)p.C * M * N * 4 : 0;
    return p;
}

// Gated gate/up pair: the 2N / 16 tiles of both projections, alternating, in the
// fixed-wave split plan with an even tw (each pair in one workgroup), sized so the
// launch fits one workgroup per CU.
SkinnyPlan plan_skinny_pair(int M, int N, int K, size_t lds_limit)
{
    const long long tiles = 2LL * ((N + 15) / 16) * ((M + 15) / 16);
    int tw = (int)((tiles + kCUs - 1) / kCUs);
    tw = (tw + 1) & ~1;
    tw = tw < 2 ? 2 : tw > kMaxWaves ? kMaxWaves : tw;
    return plan_skinny_fixed(M, 2 * N, K, lds_limit, tw, true);
}

namespace {

template <int MODE, bool ALIGNED, bool GATED>
void launch_variant(int nr, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const SkinnyArgs &a,
                    const SkinnyPlan &p)
{
    if (nr == 1)
        hipLaunchKernelGGL((skinny_kernel<1, MODE, ALIGNED, GATED>), grid, block, lds, stream, a, p);
    else if (nr == 2)
        hipLaunchKernelGGL((skinny_kernel<2, MODE, ALIGNED, GATED>), grid, block, lds, stream, a, p);
    else
        hipLaunchKernelGGL((skinny_kernel<4, MODE, ALIGNED, GATED>), grid, block, lds, stream, a, p);
}

template <int MODE, bool ALIGNED, bool GATED = false>
void allow_lds(size_t bytes)
{
    (void)hipFuncSetAttribute((const void *)skinny_kernel<1, MODE, ALIGNED, GATED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipFuncSetAttribute((const void *)skinny_kernel<2, MODE, ALIGNED, GATED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipFuncSetAttribute((const void *)skinny_kernel<4, MODE, ALIGNED, GATED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int MODE, bool GATED = false>
void launch_mode(bool aligned, int nr, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                 const SkinnyArgs &a, const SkinnyPlan &p)
{
    if (aligned)
        launch_variant<MODE, true, GATED>(nr, grid, block, lds, stream, a, p);
    else
        launch_variant<MODE, false, GATED>(nr, grid, block, lds, stream, a, p);
}

template <bool ALIGNED>
void allow_lds_multi(size_t bytes)
{
    (void)hipFuncSetAttribute((const void *)skinny_multi_kernel<1, ALIGNED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipFuncSetAttribute((const void *)skinny_multi_kernel<2, ALIGNED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    (void)hipFuncSetAttribute((const void *)skinny_multi_kernel<4, ALIGNED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// LDS per workgroup: whatever the device allows, up to the budget the plans assume;
// looked up, and the kernels' limits raised to it, once per device
size_t g_lds_limit[kMaxDevices];

hipError_t init_lds_limit(int dev)
{
    int v = 0;
    const hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess)
        return e;
    const size_t lim = (size_t)v > 4096 ? (size_t)v - 4096 : 0; // room for the static LDS
    const size_t lds_limit = lim < kLdsBudget ? lim : kLdsBudget;
    if (lds_limit > 64 * 1024) {
        allow_lds<kSplitLds, false>(lds_limit);
        allow_lds<kSplitLds, true>(lds_limit);
        allow_lds<kStream, false>(lds_limit);
        allow_lds<kStream, true>(lds_limit);
        allow_lds<kSplitPriv, false>(lds_limit);
        allow_lds<kSplitPriv, true>(lds_limit);
        allow_lds<kSplitPrivDma, false>(lds_limit);
        allow_lds<kSplitPrivDma, true>(lds_limit);
        allow_lds<kSplitChunk, false>(lds_limit);
        allow_lds<kSplitChunk, true>(lds_limit);
        allow_lds<kSplitLds, false, true>(lds_limit);
        allow_lds<kSplitLds, true, true>(lds_limit);
        allow_lds<kSplitPriv, false, true>(lds_limit);
        allow_lds<kSplitPriv, true, true>(lds_limit);
        allow_lds<kSplitPrivDma, false, true>(lds_limit);
        allow_lds<kSplitPrivDma, true, true>(lds_limit);
        allow_lds<kSplitChunk, false, true>(lds_limit);
        allow_lds<kSplitChunk, true, true>(lds_limit);
        allow_lds_multi<false>(lds_limit);
        allow_lds_multi<true>(lds_limit);
    }
    g_lds_limit[dev] = lds_limit;
    return hipSuccess;
}

hipError_t device_lds_limit(size_t *limit)
{
    const hipError_t e = once_per_device(kOnceSkinny, init_lds_limit);
    if (e != hipSuccess)
        return e;
    int dev = 0;
    const hipError_t d = current_device(&dev);
    if (d != hipSuccess)
        return d;
    *limit = g_lds_limit[dev];
    return hipSuccess;
}

} // namespace

void balance_multi(const int *N, const int *K, int count, int M, int *tw)
{
    // the same amount of packed weights per workgroup for every projection, sized so
    // that the launch fits one workgroup per CU: tw = ceil(work per CU / groups per tile)
    const long long mb = (M + 15) / 16;
    long long work = 0;
    for (int q = 0; q < count; ++q)
        work += (long long)((N[q] + 15) / 16) * mb * (K[q] / kGroup);
    for (int q = 0; q < count; ++q) {
        const long long g = K[q] / kGroup > 0 ? K[q] / kGroup : 1;
        long long t = (work + (long long)kCUs * g - 1) / ((long long)kCUs * g);
        tw[q] = (int)(t < 1 ? 1 : t > kMaxWaves ? kMaxWaves : t);
    }
}

size_t skinny_chunk_ws_bound(int M, int N, int K)
{
    // a chunked plan splits K only when X of all of K does not fit in LDS, and then
    // into chunks of 32 groups (any tiles-per-workgroup choice)
    const int G = K / kGroup;
    if (M <= 4 || M > 16 || G <= 32)
        return 0;
    const size_t all = (size_t)((G * 16 * M + 63) & ~63) * 16 + (size_t)kMaxWaves * 1024;
    if (all <= kLdsBudget)
        return 0;
    return kZeroRegion + (size_t)((G + 31) / 32) * M * N * 4;
}

size_t skinny_multi_scratch(SkinnyMulti &mp, int M)
{
    int tkt = 0;
    size_t off = kZeroRegion;
    for (int q = 0; q < mp.count; ++q) {
        SkinnyPlan &p = mp.plan[q];
        if (p.xlds != 3 || p.C <= 1)
            continue;
        p.tkt = tkt;
        p.part_off = off;
        tkt += p.mblocks * p.ntg;
        off += (size_t)p.C * M * mp.args[q].N * 4;
    }
    return off == kZeroRegion ? 0 : off;
}

hipError_t launch_skinny_multi(SkinnyMulti &mp, int M, size_t ws_bytes, hipStream_t stream)
{
    size_t lds_limit = 0;
    hipError_t e = device_lds_limit(&lds_limit);
    if (e != hipSuccess)
        return e;
    size_t lds = 0;
    bool aligned = true;
    int grid = 0;
    bool replanned = false;
    for (int q = 0; q < mp.count; ++q) {
        if (mp.plan[q].lds_bytes > lds_limit) {
            mp.plan[q] = plan_skinny_fixed(M, mp.args[q].N, mp.args[q].K, lds_limit, mp.plan[q].tw);
            replanned = true;
        }
        if (mp.plan[q].lds_bytes > lds_limit)
            return hipErrorInvalidValue;
        lds = mp.plan[q].lds_bytes > lds ? mp.plan[q].lds_bytes : lds;
        aligned = aligned && (mp.args[q].G % 4) == 0 && (mp.plan[q].per % 4) == 0;
        mp.begin[q] = grid;
        grid += mp.plan[q].grid;
    }
    mp.begin[mp.count] = grid;
    if (replanned && skinny_multi_scratch(mp, M) > ws_bytes)
        return hipErrorInvalidValue;
    if (grid == 0)
        return hipSuccess;
    const dim3 block(64 * kMaxWaves), g(grid);
    const int nr = M == 1 ? 1 : M == 2 ? 2 : 4;
    if (aligned) {
        if (nr == 1)
            hipLaunchKernelGGL((skinny_multi_kernel<1, true>), g, block, lds, stream, mp);
        else if (nr == 2)
            hipLaunchKernelGGL((skinny_multi_kernel<2, true>), g, block, lds, stream, mp);
        else
            hipLaunchKernelGGL((skinny_multi_kernel<4, true>), g, block, lds, stream, mp);
    } else {
        if (nr == 1)
            hipLaunchKernelGGL((skinny_multi_kernel<1, false>), g, block, lds, stream, mp);
        else if (nr == 2)
            hipLaunchKernelGGL((skinny_multi_kernel<2, false>), g, block, lds, stream, mp);
        else
            hipLaunchKernelGGL((skinny_multi_kernel<4, false>), g, block, lds, stream, mp);
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &plan, hipStream_t stream)
{
    size_t lds_limit = 0;
    const hipError_t le = device_lds_limit(&lds_limit);
    if (le != hipSuccess)
        return le;
    const SkinnyPlan p = plan.lds_bytes <= lds_limit ? plan
                         : a.gated               ? plan_skinny_pair(a.M, a.N, a.K, lds_limit)
                                                 : plan_skinny(a.M, a.N, a.K, a.lmhead, lds_limit);
    if (p.lds_bytes > lds_limit)
        return hipErrorInvalidValue;
    const dim3 block(64 * p.waves), grid(p.grid);
    const int nr = a.M == 1 ? 1 : a.M == 2 ? 2 : 4;
    // 4-group scale/zero loads need G and every slice start to be multiples of 4
    const bool aligned = (a.G % 4) == 0 && (p.per % 4) == 0;
    if (a.gated) {
        // a pair plan is never in stream mode
        if (p.stream || !p.pair || (p.tw & 1))
            return hipErrorInvalidValue;
        if (p.xlds == 3)
            launch_mode<kSplitChunk, true>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
        else if (p.xlds == 2 && p.xdma)
            launch_mode<kSplitPrivDma, true>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
        else if (p.xlds == 2)
            launch_mode<kSplitPriv, true>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
        else if (p.xlds == 1)
            launch_mode<kSplitLds, true>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
        else
            launch_mode<kSplitDirect, true>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
        return hipGetLastError();
    }
    if (p.stream)
        launch_mode<kStream>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    else if (p.xlds == 3)
        launch_mode<kSplitChunk>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    else if (p.xlds == 2 && p.xdma)
        launch_mode<kSplitPrivDma>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    else if (p.xlds == 2)
        launch_mode<kSplitPriv>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    else if (p.xlds == 1)
        launch_mode<kSplitLds>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    else
        launch_mode<kSplitDirect>(aligned, nr, grid, block, p.lds_bytes, stream, a, p);
    return hipGetLastError();
}

} // namespace w4a16
