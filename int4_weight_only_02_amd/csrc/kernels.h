// kernels.h -- host-side interface between the C ABI (api.hip) and the gfx950
// kernels (pack.hip, skinny.hip, tiled.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// ---------------------------------------------------------------- host set-up (host.hip)
constexpr int kMaxDevices = 64;
enum { kOnceSkinny = 0, kOnceTiled = 1, kOnceBlock = 2, kOnceSlots = 3 };
// the device current on the calling thread (below kMaxDevices)
hipError_t current_device(int *dev);
// init(dev) runs at most once per (slot, device), under a lock; every caller gets its status
hipError_t once_per_device(int slot, hipError_t (*init)(int dev));

constexpr int kMaxProblemsBlock = 8; // projections per block launch

// Workspace layout shared by every call.  The first kZeroRegion bytes hold
// counters that must read zero when a call starts (the caller zero-fills the
// workspace once; every call returns them to zero before it completes); scratch
// that needs no initial value starts at kZeroRegion, so calls of any shape and
// path can share one workspace.
constexpr size_t kOffTicket = 0;          // u32: workgroups finished (lm_head)
constexpr size_t kOffKeys = 256;          // u64[64]: per-row argmax keys (lm_head)
constexpr size_t kOffCounters = 1024;     // arrival counters (small-M parts of K, prefill tile hand-offs)
constexpr size_t kZeroRegion = 65536;
// Every arrival counter sits alone in a 128-byte line: device-scope atomics on one line
// complete one at a time (about 33 ns each on MI355X), so counters packed into a few
// lines would queue every arrival of a launch behind each other.
constexpr int kCounterStride = 32; // u32 per counter
constexpr int kMaxCounters = (int)((kZeroRegion - kOffCounters) / (4 * kCounterStride));

// ---------------------------------------------------------------- pack
hipError_t launch_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int G,
                       uint32_t *qweight, uint32_t *qzeros, hipStream_t stream);
hipError_t launch_pack_zeros(const uint8_t *zeros, int N, int G, uint32_t *qzeros, hipStream_t stream);

// ---------------------------------------------------------------- GPTQ act-order
// perm (host) from g_idx (host): false unless every group holds exactly `group` columns
bool actorder_perm_host(const int32_t *g_idx, int K, int group, int32_t *perm);
// codes gathered by perm and packed, zeros packed as by launch_pack (device)
hipError_t launch_pack_perm(const uint8_t *codes, const uint8_t *zeros, const int32_t *perm, int N, int K, int G,
                            uint32_t *qweight, uint32_t *qzeros, hipStream_t stream);
// dst[r][j] = src[r][perm[j]] for 1- or 2-byte elements (device), K % 8 == 0
hipError_t launch_gather_k(const void *src, const int32_t *perm, int rows, int K, int elem_bytes, void *dst,
                           hipStream_t stream);

// ---------------------------------------------------------------- sliding-window attention
struct SwaArgs {
    const uint16_t *Q, *K, *Vt; // bf16: [M][Hq][128], [T][Hkv][128], [Hkv][128][t_stride]
    int M, T, Hq, Hkv, window;
    int block;                  // 1: every key of the block is seen (bidirectional within it)
    int t_stride;               // row length of V^T (>= T, a multiple of 8)
    float scale;                // 1 / sqrt(128)
    void *O;                    // [M][Hq][128], bf16 or fp32
    int o_f32;
    int j_lo;                   // first key any query sees
    float *ml, *part;           // workspace: per (chunk, head, query) (max, sum) and O~
};
struct SwaPlan {
    int j_lo, chunks;
    size_t ml_off, part_off, ws_bytes;
};
SwaPlan plan_swa(int M, int T, int Hq, int Hkv, int window);
hipError_t launch_swa(SwaArgs a, const SwaPlan &p, unsigned char *ws, hipStream_t stream);

// ---------------------------------------------------------------- re-quantization
hipError_t launch_quantize(const uint16_t *W, const uint16_t *scales, const uint32_t *qzeros, int N, int K,
                           uint32_t *qweight, hipStream_t stream);

// ---------------------------------------------------------------- skinny (small M)
// Every workgroup owns whole 16-column tiles (no partial sums cross workgroups).
//   split mode  (stream == 0): item = (16-row m-block, group of tw tiles); a
//               workgroup of tw * sk waves takes one item at a time, each tile's K
//               split over sk waves and summed through LDS in slice order;
//   stream mode (stream == 1): persistent workgroups of tw waves; each wave takes
//               whole tiles (tile groups blockIdx.x, +grid, ...) over all of K.
// With xlds, X of the m-block is staged in LDS in chunks of `chunk` groups (all of
// K when it fits; stream mode requires that); without it (split mode only) each
// wave reads its K slice of X from global memory and chunk is 0.
struct SkinnyPlan {
    int mblocks;   // ceil(M / 16)
    int nt;        // ceil(N / 16) column tiles
    int G;         // K / 128
    int waves;     // waves per workgroup = tw * sk
    int tw, sk;    // tiles per item, K slices per tile
    int chunk;     // groups of X staged in LDS at once (all of K; xlds == 2: one slice)
    int per;       // groups per K slice (split mode; a multiple of 4)
    int ntg;       // tile groups per m-block = ceil(nt / tw)
    int items;     // mblocks * ntg
    int grid;      // workgroups
    int stream;    // 1: stream mode
    int xlds;      // 1: X staged in LDS by the workgroup; 2: each wave stages its own slice;
                   // 3: chunked (X of one K chunk in LDS by DMA, chunks meet in the workspace)
    int xdma;      // xlds 2: X arrives by LDS DMA and the zero-point is folded by MFMA
    int C, cg;     // xlds 3: K chunks per tile group, groups per chunk (a multiple of 4 if C > 1)
    int tkt;       // xlds 3, C > 1: first arrival counter (u32 at kOffCounters) of this projection
    size_t part_off; // xlds 3, C > 1: workspace offset of the fp32 partial sums [C][M][N]
    int pair;      // gated pairs: tile slot 2i holds a gate tile, 2i + 1 the up tile of the same columns (tw even)
    size_t lds_bytes;
    size_t ws_bytes; // lm_head: the zero region (argmax keys, ticket); linear: the partials (xlds 3) or 0
};

struct SkinnyArgs {
    const uint16_t *X;
    const uint32_t *qw;
    const uint16_t *scales;
    const uint32_t *qz;
    int M, N, K, G;
    void *Y;           // may be null (lm_head without logits)
    int y_f32;
    unsigned char *ws; // workspace base
    int lmhead;
    const int32_t *draft;
    int32_t *argmax_out;
    int32_t *accept_out;
    // gated (plan.pair): qw/scales/qz are the gate projection, these the up projection
    // of the same N columns; Y = silu(gate) * up
    const uint32_t *qw2;
    const uint16_t *scales2;
    const uint32_t *qz2;
    int gated;
};

SkinnyPlan plan_skinny(int M, int N, int K, int lmhead, size_t lds_limit = 0);
hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &p, hipStream_t stream);

// several linear projections with the same M in one launch (split mode, 8 waves each)
constexpr int kMaxProblems = 8;
struct SkinnyMulti {
    int count;
    int begin[kMaxProblems + 1]; // first workgroup of each projection; begin[count] = grid
    SkinnyArgs args[kMaxProblems];
    SkinnyPlan plan[kMaxProblems];
};
SkinnyPlan plan_skinny_fixed(int M, int N, int K, size_t lds_limit = 0, int tw_hint = 0, bool pair = false);
// gated gate/up pair of N columns each (N % 16 == 0): 2N/16 tiles, an even tw
SkinnyPlan plan_skinny_pair(int M, int N, int K, size_t lds_limit = 0);
// tiles per workgroup that spread the projections of one launch evenly over the CUs
void balance_multi(const int *N, const int *K, int count, int M, int *tw);
// upper bound of the partial-sum scratch any chunked plan of this shape needs
size_t skinny_chunk_ws_bound(int M, int N, int K);
// gives every chunked projection its own arrival counters and partial-sum region;
// returns the workspace bytes the launch needs (0: none)
size_t skinny_multi_scratch(SkinnyMulti &mp, int M);
hipError_t launch_skinny_multi(SkinnyMulti &mp, int M, size_t ws_bytes, hipStream_t stream);

// ---------------------------------------------------------------- gemv (M = 1)
// Workgroup b owns the TC = 16 / pl columns from b TC and all of K; its waves split K,
// wave w taking the gpw * pl groups from w gpw pl.
constexpr int kMaxProblemsGemv = 8; // projections per multi launch (pair 3)
struct GemvPlan {
    int gpw, pl, ao;  // code loads per lane, group parts per instruction, act-order
    int pair;         // 1: the gated pair (silu(gate) * up); 2: two outputs; qw2 / scales2 / qz2 the second grid;
                      // 3: several projections of one X (GemvArgs::pr), each its own workgroups
    int waves, grid;  // waves per workgroup (each NG = gpw * pl groups), N / (16 / pl)
    size_t lds_bytes;
    bool ok;          // false: the shape needs another path
};
struct GemvArgs {
    const uint16_t *X;
    const int32_t *perm; // act-order only: X'[k] = X[perm[k]]
    const uint32_t *qw;
    const uint16_t *scales;
    const uint32_t *qz;
    const uint32_t *qw2;     // pairs only: the second (up) projection's grid
    const uint16_t *scales2;
    const uint32_t *qz2;
    void *Y2;                // two outputs: the second projection's
    int N, K, G;
    void *Y;
    int y_f32;
    int waves; // copied from the plan by launch_gemv
    // pair 3: projection q owns workgroups wg0 .. of the launch (pr[0].wg0 = 0); every
    // projection reads the same X and has the same K
    struct Prob {
        const uint32_t *qw;
        const uint16_t *scales;
        const uint32_t *qz;
        void *Y;
        int N, wg0;
    } pr[kMaxProblemsGemv];
    int count;
};
GemvPlan plan_gemv(int N, int K, int ao);
// pair 3: count projections of the same K (and X); wg0[q] receives projection q's first
// workgroup.  !ok unless every N fits the plan's columns per workgroup
GemvPlan plan_gemv_multi(const int *N, int K, int count, int *wg0);
GemvPlan plan_gemv_pair(int N, int K, int pair); // pair 1: gated, 2: two outputs
GemvPlan plan_gemv_with(int N, int K, int gpw, int pl, int ao);
hipError_t launch_gemv(const GemvArgs &a, const GemvPlan &p, hipStream_t stream);

// ---------------------------------------------------------------- block (2 <= M <= 16)
// One or several projections with the same M.  Projection q is cut into ntg tile
// groups (balanced runs of at most tmx 16-column tiles) and `parts` parts of K; its
// workgroups (from wg0) take (tile group, part) in that order.  Parts of one tile group
// meet in the workspace (partial sums at part_off, an arrival counter at tkt).
struct BlockProb {
    const uint16_t *X;
    const uint32_t *qw;
    const uint16_t *scales;
    const uint32_t *qz;
    void *Y;
    int N, K;
    // filled by launch_block
    int nt, wg0, ntg, parts, tmx, tkt;
    size_t part_off;
};
struct BlockArgs {
    BlockProb pr[kMaxProblemsBlock];
    int count, M, y_f32;
    unsigned char *ws;       // workspace base (partial sums, arrival counters)
};
struct BlockPlan {
    int count, gpw, tmax, waves, grid;
    int gated; // a gated pair: pr[0] the gate, pr[1] the up projection (count 1)
    int wg0[kMaxProblemsBlock], ntg[kMaxProblemsBlock], parts[kMaxProblemsBlock], tmx[kMaxProblemsBlock];
    int tkt[kMaxProblemsBlock];
    size_t part_off[kMaxProblemsBlock];
    size_t lds_bytes, ws_bytes; // ws_bytes: 0 when no projection splits K
    bool ok;
};
BlockPlan plan_block(const int *N, const int *K, int count, int M, int tmax_hint = 0, int waves_hint = 0,
                     int parts_hint = 0);
// a gated pair in one launch (silu(gate) * up); !ok where K is split or too long
BlockPlan plan_block_gated(int N, int K, int M);
hipError_t launch_block(const BlockArgs &a, const BlockPlan &p, hipStream_t stream);
// workspace of a single projection's block plan (the zero region included when K is split)
size_t block_linear_ws(int M, int N, int K);

// ---------------------------------------------------------------- tiled (large M)
struct TiledPlan {
    int G;
    int tiles_m, tiles_n;
    int stream;       // 1: one balanced segment of tile-groups per CU (at least one tile per CU)
    int grid;         // workgroups
    int dp_rounds;    // stream: rounds of whole tiles before the segments
    int ksplit;       // K slices per tile (1: the tile kernel stores Y itself)
    int gper;         // groups per K slice
    size_t off_xh;    // X as fp16, each row scaled by a power of two, [M][K]
    size_t off_rs;    // the per-row scales (fp32, M)
    size_t off_part;  // ksplit > 1: fp32 partial sums [ksplit][M][N]; stream: one pair of
                      // fp32 tile regions per inner segment boundary
    size_t ws_bytes;
    int gated;        // the gated pair in one launch (whole tiles of 128 output columns)
    bool ok;
};

struct TiledArgs {
    const uint16_t *X;
    const uint32_t *qw;
    const uint16_t *scales;
    const uint32_t *qz;
    const uint32_t *qw2; // gated plans: the up projection (qw etc.: gate)
    const uint16_t *scales2;
    const uint32_t *qz2;
    int M, N, K, G;
    void *Y;
    int y_f32;
    unsigned char *ws;
};

TiledPlan plan_tiled(int M, int N, int K);
// Y = silu(X Wg^T) * (X Wu^T) in one tile kernel (no fp32 intermediates); !ok when
// the tiles would not fill one round of the CUs
TiledPlan plan_tiled_gated(int M, int N, int K);
hipError_t launch_tiled(const TiledArgs &a, const TiledPlan &p, hipStream_t stream);

// path choice for w4a16_linear: small M streams the weights once per 16 rows
constexpr int kSkinnyMaxM = 64;

// Y[i] = silu(G[i]) * U[i] for n fp32 values (n % 4 == 0, 16-byte aligned)
hipError_t launch_silu_mul(const float *G, const float *U, long long n, void *Y, int y_f32, hipStream_t stream);

} // namespace w4a16
