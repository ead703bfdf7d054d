// kernels.h -- host-side interface between the C ABI (api.hip) and the gfx950
// kernels (pack.hip, skinny.hip, tiled.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

// Workspace layout shared by every call.  The first kZeroRegion bytes hold
// counters that must read zero when a call starts (the caller zero-fills the
// workspace once; every call returns them to zero before it completes); scratch
// that needs no initial value starts at kZeroRegion, so calls of any shape and
// path can share one workspace.
constexpr size_t kOffTicket = 0;          // u32: workgroups finished (lm_head)
constexpr size_t kOffKeys = 256;          // u64[64]: per-row argmax keys (lm_head)
constexpr size_t kOffCounters = 1024;     // u32[kMaxGrid]: split column-block arrivals
constexpr int kMaxGrid = 1024;
constexpr size_t kZeroRegion = 8192;

// ---------------------------------------------------------------- pack
hipError_t launch_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int G,
                       uint32_t *qweight, uint32_t *qzeros, hipStream_t stream);

// ---------------------------------------------------------------- skinny (small M)
// Work unit = one group (128 of K) of one 128-column block of one 16-row m-block.
// Units are ordered (m-block, column block, group) and split into `grid`
// contiguous, near-equal ranges, one per workgroup (stream-K).  A column block
// whose K range spans several workgroups is summed by the last one to finish,
// in workgroup order, from per-workgroup fp32 partials.  Its arrival counter is
// indexed by the workgroup that owns its first unit (each workgroup owns the
// first unit of at most one split column block), so grid counters suffice.
struct SkinnyPlan {
    int mblocks;   // ceil(M / 16)
    int ncb;       // ceil(N / 128)
    int G;         // K / 128
    long long units;
    int grid;      // workgroups (<= kMaxGrid)
    int chunk;     // max groups of X staged in LDS at once
    size_t lds_bytes;
    size_t off_partial, ws_bytes; // partials start at kZeroRegion
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
};

SkinnyPlan plan_skinny(int M, int N, int K, int lmhead);
hipError_t launch_skinny(const SkinnyArgs &a, const SkinnyPlan &p, hipStream_t stream);

// ---------------------------------------------------------------- tiled (large M)
struct TiledPlan {
    int G;
    int tiles_m, tiles_n;
    size_t off_gsum, ws_bytes;  // per-row group sums of X, fp32 [G][M]
};

struct TiledArgs {
    const uint16_t *X;
    const uint32_t *qw;
    const uint16_t *scales;
    const uint32_t *qz;
    int M, N, K, G;
    void *Y;
    int y_f32;
    unsigned char *ws;
};

TiledPlan plan_tiled(int M, int N, int K);
hipError_t launch_tiled(const TiledArgs &a, const TiledPlan &p, hipStream_t stream);

// path choice for w4a16_linear: small M streams the weights once per 16 rows
constexpr int kSkinnyMaxM = 64;

} // namespace w4a16
