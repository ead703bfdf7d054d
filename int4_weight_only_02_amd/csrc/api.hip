// api.hip -- the C ABI (include/w4a16.h): host-side validation, path choice and
// launches.  Nothing here allocates, frees, synchronizes or prints; every check
// runs before the first launch, so a rejected call leaves the stream untouched.
#include "w4a16.h"

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace w4a16;

namespace {

constexpr long long kLimit = 0x7FFFFF00ll; // element counts: byte offsets stay below the out-of-range offset the kernels use

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

// checks shared by the linear and lm_head calls (after the group check)
int check_dims(int M, int N, int K)
{
    if (M < 0 || N < 0 || K < kGroup || K % kGroup != 0 || N % 8 != 0)
        return W4A16_ERR_SHAPE;
    if ((long long)M * N > kLimit || (long long)N * K > kLimit || (long long)M * K > kLimit)
        return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// 2 <= M <= 16: the draft-block kernel holds each workgroup's tiles at once, so a
// launch with more (tile group, part) workgroups than CUs runs in several rounds, each
// staging X again.  There the streaming small-M kernel is faster wherever it keeps X in
// LDS (measured on MI355X, M = 2 .. 16: K = 2560, N = 24576 .. 151936, 11.5-56.5 against
// 15.0-64.8 us; K = 9728, N = 9728, M <= 6, 16.3-19.0 against 22.4-22.8 us); with X read
// from L2 it is slower (the same shape at M >= 8: 30-41 against 23 us).
bool block_first(const BlockPlan &bp, int M, int N, int K)
{
    if (bp.grid <= 256)
        return true;
    const int xlds = plan_skinny(M, N, K, 0).xlds;
    return xlds != 1 && xlds != 2;
}

// covers both the single-call plan and the plan the same projection gets inside a
// batched launch, so that the sum over a batch's projections always suffices
size_t linear_ws(int M, int N, int K)
{
    if (M <= kSkinnyMaxM) {
        const size_t a = plan_skinny(M, N, K, 0).ws_bytes, b = skinny_chunk_ws_bound(M, N, K);
        const size_t c = (M >= 2 && M <= 16) ? block_linear_ws(M, N, K) : 0;
        const size_t ab = a > b ? a : b;
        return ab > c ? ab : c;
    }
    return plan_tiled(M, N, K).ws_bytes;
}

// the gathered X of an act-order call sits after the workspace of the linear call,
// and never in the zero region (a linear call that needs no workspace has base 0)
size_t actorder_x_offset(int M, int N, int K)
{
    size_t base = linear_ws(M, N, K);
    base = base > kZeroRegion ? base : kZeroRegion;
    return (base + 255) / 256 * 256;
}

// gated pair: the partial sums of the paired small-M plan, or (large M) the tiled
// call's workspace followed by the two fp32 outputs [M][N] of gate and up
size_t gated_gu_offset(int M, int N, int K)
{
    return (linear_ws(M, N, K) + 255) / 256 * 256;
}

size_t gated_ws(int M, int N, int K)
{
    if (M <= kSkinnyMaxM)
        return plan_skinny_pair(M, N, K).ws_bytes;
    const TiledPlan tp = plan_tiled_gated(M, N, K);
    if (tp.ok)
        return tp.ws_bytes;
    return gated_gu_offset(M, N, K) + 2 * (size_t)M * N * 4;
}

// ---------------------------------------------------------------- static scratch
// The scratch of w4a16_linear_static_ws: one array per device (each GPU the library
// runs on holds its own copy at its own address).  In host code `scratch` names a
// host-side stand-in, not the device memory: only the address obtained from
// hipGetSymbolAddress (kept per device below) is ever passed to a kernel.
constexpr size_t kStaticWsBytes = W4A16_STATIC_WS_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticWsBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

// the current device's scratch address; on its first use on a device, the address is
// looked up and the counter region cleared by a kernel on `stream`
int static_scratch(void **out, hipStream_t stream)
{
    int dev = -1;
    if (current_device(&dev) != hipSuccess)
        return W4A16_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return W4A16_ERR_HIP;
        hipLaunchKernelGGL(zero_words_kernel, dim3(8), dim3(256), 0, stream, (uint32_t *)p, (int)(kZeroRegion / 4));
        if (hipGetLastError() != hipSuccess)
            return W4A16_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}

} // namespace

extern "C" {

int w4a16_abi_version(void) { return 100; }

const char *w4a16_status_string(int status)
{
    switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL: return "null pointer";
    case W4A16_ERR_SHAPE: return "unsupported shape";
    case W4A16_ERR_ALIGN: return "pointer not 16-byte aligned";
    case W4A16_ERR_UNSUPPORTED: return "unsupported group size or output dtype";
    case W4A16_ERR_WORKSPACE: return "workspace too small";
    case W4A16_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

size_t w4a16_workspace_bytes(int op, int M, int N, int K, int group)
{
    if (group != kGroup || check_dims(M, N, K) != W4A16_OK)
        return 0;
    if (op == W4A16_OP_LINEAR)
        return (M == 0 || N == 0) ? 0 : linear_ws(M, N, K);
    if (op == W4A16_OP_LINEAR_ACTORDER)
        return (M == 0 || N == 0) ? 0 : actorder_x_offset(M, N, K) + (size_t)M * K * 2;
    if (op == W4A16_OP_LMHEAD)
        return (M < 1 || M > 64 || N < 1) ? 0 : plan_skinny(M, N, K, 1).ws_bytes;
    if (op == W4A16_OP_LINEAR_GATED)
        return (M == 0 || N == 0 || N % 16 != 0) ? 0 : gated_ws(M, N, K);
    return 0;
}

int w4a16_pack(const uint8_t *codes, const uint8_t *zeros, int N, int K, int group,
               uint32_t *qweight, uint32_t *qzeros, void *stream)
{
    if (group != kGroup)
        return W4A16_ERR_UNSUPPORTED;
    if (check_dims(0, N, K) != W4A16_OK)
        return W4A16_ERR_SHAPE;
    if (N == 0)
        return W4A16_OK;
    if (!codes || !zeros || !qweight || !qzeros)
        return W4A16_ERR_NULL;
    if (misaligned(codes) || misaligned(qweight))
        return W4A16_ERR_ALIGN;
    if (launch_pack(codes, zeros, N, K, K / kGroup, qweight, qzeros, (hipStream_t)stream) != hipSuccess)
        return W4A16_ERR_HIP;
    return W4A16_OK;
}

int w4a16_actorder_perm(const int32_t *g_idx, int K, int group, int32_t *perm)
{
    if (group != kGroup)
        return W4A16_ERR_UNSUPPORTED;
    if (K < group || K % group != 0 || (long long)K > kLimit)
        return W4A16_ERR_SHAPE;
    if (!g_idx || !perm)
        return W4A16_ERR_NULL;
    return actorder_perm_host(g_idx, K, group, perm) ? W4A16_OK : W4A16_ERR_SHAPE;
}

int w4a16_pack_actorder(const uint8_t *codes, const uint8_t *zeros, const int32_t *perm, int N, int K,
                        int group, uint32_t *qweight, uint32_t *qzeros, void *stream)
{
    if (group != kGroup)
        return W4A16_ERR_UNSUPPORTED;
    const int st = check_dims(0, N, K);
    if (st != W4A16_OK)
        return st;
    if (N == 0)
        return W4A16_OK;
    if (!codes || !zeros || !perm || !qweight || !qzeros)
        return W4A16_ERR_NULL;
    if (misaligned(codes) || misaligned(perm) || misaligned(qweight))
        return W4A16_ERR_ALIGN;
    const hipError_t e = launch_pack_perm(codes, zeros, perm, N, K, K / kGroup, qweight, qzeros,
                                          (hipStream_t)stream);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_linear_actorder(const void *X, const int32_t *perm, const uint32_t *qweight, const void *scales,
                          const uint32_t *qzeros, int M, int N, int K, int group, void *Y, int y_dtype,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    const int st = check_dims(M, N, K);
    if (st != W4A16_OK)
        return st;
    if (M == 0 || N == 0)
        return W4A16_OK;
    if (!X || !perm || !workspace)
        return W4A16_ERR_NULL;
    if (misaligned(X) || misaligned(perm) || misaligned(workspace))
        return W4A16_ERR_ALIGN;
    const size_t off = actorder_x_offset(M, N, K);
    if (workspace_bytes < off + (size_t)M * K * 2)
        return W4A16_ERR_WORKSPACE;
    // everything w4a16_linear checks is checked before the gather is enqueued
    if (!qweight || !scales || !qzeros || !Y)
        return W4A16_ERR_NULL;
    if (misaligned(qweight) || misaligned(scales) || misaligned(qzeros) || misaligned(Y))
        return W4A16_ERR_ALIGN;
    // M = 1 up to 40 groups: the gather runs inside the kernel's X staging (K values per
    // workgroup).  Otherwise a gather launch writes the permuted X to the workspace and
    // the plain linear reads it (for 2 <= M <= 16, a gather inside the draft-block
    // kernel, from the X rows in LDS, measured 2 us slower at 16 x 2560 -> 9728)
    const GemvPlan gp = (M == 1 && K / kGroup <= 40) ? plan_gemv(N, K, 1) : GemvPlan{};
    if (gp.ok) {
        GemvArgs a{};
        a.X = (const uint16_t *)X;
        a.perm = perm;
        a.qw = qweight;
        a.scales = (const uint16_t *)scales;
        a.qz = qzeros;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        return launch_gemv(a, gp, (hipStream_t)stream) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
    }
    void *xg = (unsigned char *)workspace + off;
    if (launch_gather_k(X, perm, M, K, 2, xg, (hipStream_t)stream) != hipSuccess)
        return W4A16_ERR_HIP;
    return w4a16_linear(xg, qweight, scales, qzeros, M, N, K, group, Y, y_dtype, workspace, off, stream);
}

static int swa_check(int M, int T, int Hq, int Hkv, int D, int window, int t_stride)
{
    if (D != 128)
        return W4A16_ERR_UNSUPPORTED;
    if (M < 1 || M > 16 || T < M || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || Hq / Hkv > 16 || window < 1 ||
        window > 65536 || t_stride < T || t_stride % 8 != 0)
        return W4A16_ERR_SHAPE;
    if ((long long)T * Hkv * D > kLimit || (long long)Hkv * D * t_stride > kLimit || (long long)M * Hq * D > kLimit)
        return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

size_t w4a16_swa_workspace_bytes(int M, int T, int Hq, int Hkv, int window)
{
    if (swa_check(M, T, Hq, Hkv, 128, window, (T + 7) / 8 * 8) != W4A16_OK)
        return 0;
    return plan_swa(M, T, Hq, Hkv, window).ws_bytes;
}

static int swa_call(const void *Q, const void *K, const void *Vt, int M, int T, int Hq, int Hkv, int D, int window,
                    int t_stride, void *O, int o_dtype, void *workspace, size_t workspace_bytes, void *stream, int block)
{
    if (o_dtype != W4A16_OUT_BF16 && o_dtype != W4A16_OUT_F32)
        return W4A16_ERR_UNSUPPORTED;
    const int st = swa_check(M, T, Hq, Hkv, D, window, t_stride);
    if (st != W4A16_OK)
        return st;
    if (!Q || !K || !Vt || !O || !workspace)
        return W4A16_ERR_NULL;
    if (misaligned(Q) || misaligned(K) || misaligned(Vt) || misaligned(O) || misaligned(workspace))
        return W4A16_ERR_ALIGN;
    const SwaPlan p = plan_swa(M, T, Hq, Hkv, window);
    if (workspace_bytes < p.ws_bytes)
        return W4A16_ERR_WORKSPACE;
    SwaArgs a{};
    a.Q = (const uint16_t *)Q;
    a.K = (const uint16_t *)K;
    a.Vt = (const uint16_t *)Vt;
    a.M = M;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.block = block;
    a.t_stride = t_stride;
    a.scale = 0.08838834764831845f; // 1 / sqrt(128)
    a.O = O;
    a.o_f32 = o_dtype == W4A16_OUT_F32;
    const hipError_t e = launch_swa(a, p, (unsigned char *)workspace, (hipStream_t)stream);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_swa_attention(const void *Q, const void *K, const void *Vt, int M, int T, int Hq, int Hkv, int D,
                        int window, int t_stride, void *O, int o_dtype, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    return swa_call(Q, K, Vt, M, T, Hq, Hkv, D, window, t_stride, O, o_dtype, workspace, workspace_bytes, stream, 0);
}

int w4a16_swa_attention_block(const void *Q, const void *K, const void *Vt, int M, int T, int Hq, int Hkv, int D,
                              int window, int t_stride, void *O, int o_dtype, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    return swa_call(Q, K, Vt, M, T, Hq, Hkv, D, window, t_stride, O, o_dtype, workspace, workspace_bytes, stream, 1);
}

int w4a16_quantize(const void *W, const void *scales, const uint32_t *qzeros, int N, int K, int group,
                   uint32_t *qweight, void *stream)
{
    if (group != kGroup)
        return W4A16_ERR_UNSUPPORTED;
    const int st = check_dims(0, N, K);
    if (st != W4A16_OK)
        return st;
    if (N == 0)
        return W4A16_OK;
    if (!W || !scales || !qzeros || !qweight)
        return W4A16_ERR_NULL;
    if (misaligned(W) || misaligned(scales) || misaligned(qzeros) || misaligned(qweight))
        return W4A16_ERR_ALIGN;
    const hipError_t e = launch_quantize((const uint16_t *)W, (const uint16_t *)scales, qzeros, N, K, qweight,
                                         (hipStream_t)stream);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_linear(const void *X, const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                 int M, int N, int K, int group, void *Y, int y_dtype,
                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    int st = check_dims(M, N, K);
    if (st != W4A16_OK)
        return st;
    if (M == 0 || N == 0)
        return W4A16_OK;
    if (!X || !qweight || !scales || !qzeros || !Y)
        return W4A16_ERR_NULL;
    if (misaligned(X) || misaligned(qweight) || misaligned(scales) || misaligned(qzeros) || misaligned(Y) ||
        misaligned(workspace))
        return W4A16_ERR_ALIGN;
    const size_t need = linear_ws(M, N, K);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return W4A16_ERR_WORKSPACE;

    hipError_t e;
    const GemvPlan gp = M == 1 ? plan_gemv(N, K, 0) : GemvPlan{};
    BlockPlan bp{};
    if (gp.ok) {
        GemvArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight;
        a.scales = (const uint16_t *)scales;
        a.qz = qzeros;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        e = launch_gemv(a, gp, (hipStream_t)stream);
    } else if (M >= 2 && M <= 16 && (bp = plan_block(&N, &K, 1, M)).ok && bp.ws_bytes <= workspace_bytes &&
               (bp.ws_bytes == 0 || workspace) && block_first(bp, M, N, K)) {
        BlockArgs a{};
        a.ws = (unsigned char *)workspace;
        a.pr[0].X = (const uint16_t *)X;
        a.pr[0].qw = qweight;
        a.pr[0].scales = (const uint16_t *)scales;
        a.pr[0].qz = qzeros;
        a.pr[0].Y = Y;
        a.pr[0].N = N;
        a.pr[0].K = K;
        a.M = M;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        e = launch_block(a, bp, (hipStream_t)stream);
    } else if (M <= kSkinnyMaxM) {
        const SkinnyPlan p = plan_skinny(M, N, K, 0);
        SkinnyArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight;
        a.scales = (const uint16_t *)scales;
        a.qz = qzeros;
        a.M = M;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        a.lmhead = 0;
        e = launch_skinny(a, p, (hipStream_t)stream);
    } else {
        const TiledPlan p = plan_tiled(M, N, K);
        TiledArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight;
        a.scales = (const uint16_t *)scales;
        a.qz = qzeros;
        a.M = M;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        e = launch_tiled(a, p, (hipStream_t)stream);
    }
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_linear_static_ws(const void *X, const uint32_t *qweight, const void *scales, const uint32_t *qzeros,
                           int M, int N, int K, int group, void *Y, int y_dtype, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    const int st = check_dims(M, N, K);
    if (st != W4A16_OK)
        return st;
    if (M == 0 || N == 0)
        return W4A16_OK;
    if (!X || !qweight || !scales || !qzeros || !Y)
        return W4A16_ERR_NULL;
    if (misaligned(X) || misaligned(qweight) || misaligned(scales) || misaligned(qzeros) || misaligned(Y))
        return W4A16_ERR_ALIGN;
    if (linear_ws(M, N, K) > kStaticWsBytes)
        return W4A16_ERR_WORKSPACE;
    void *ws = nullptr;
    const int sst = static_scratch(&ws, (hipStream_t)stream);
    if (sst != W4A16_OK)
        return sst;
    return w4a16_linear(X, qweight, scales, qzeros, M, N, K, group, Y, y_dtype, ws, kStaticWsBytes, stream);
}

int w4a16_linear_gated(const void *X, const uint32_t *qweight_gate, const void *scales_gate,
                       const uint32_t *qzeros_gate, const uint32_t *qweight_up, const void *scales_up,
                       const uint32_t *qzeros_up, int M, int N, int K, int group, void *Y, int y_dtype,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    int st = check_dims(M, N, K);
    if (st != W4A16_OK)
        return st;
    if (N % 16 != 0 || (long long)M * N * 2 > kLimit)
        return W4A16_ERR_SHAPE;
    if (M == 0 || N == 0)
        return W4A16_OK;
    if (!X || !qweight_gate || !scales_gate || !qzeros_gate || !qweight_up || !scales_up || !qzeros_up || !Y)
        return W4A16_ERR_NULL;
    if (misaligned(X) || misaligned(qweight_gate) || misaligned(scales_gate) || misaligned(qzeros_gate) ||
        misaligned(qweight_up) || misaligned(scales_up) || misaligned(qzeros_up) || misaligned(Y) ||
        misaligned(workspace))
        return W4A16_ERR_ALIGN;
    const size_t need = gated_ws(M, N, K);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return W4A16_ERR_WORKSPACE;

    hipError_t e;
    const GemvPlan gp = M == 1 ? plan_gemv_pair(N, K, 1) : GemvPlan{};
    const BlockPlan bp = plan_block_gated(N, K, M);
    if (gp.ok) {
        // M = 1 up to 40 groups: the decode kernel with the gate and up codes of the same
        // columns in each wave
        GemvArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight_gate;
        a.scales = (const uint16_t *)scales_gate;
        a.qz = qzeros_gate;
        a.qw2 = qweight_up;
        a.scales2 = (const uint16_t *)scales_up;
        a.qz2 = qzeros_up;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        e = launch_gemv(a, gp, (hipStream_t)stream);
    } else if (bp.ok) {
        // 2 <= M <= 16, K whole: the draft-block kernel with gate and up tiles of the same
        // columns in each workgroup
        BlockArgs a{};
        for (int q = 0; q < 2; ++q) {
            a.pr[q].X = (const uint16_t *)X;
            a.pr[q].qw = q ? qweight_up : qweight_gate;
            a.pr[q].scales = (const uint16_t *)(q ? scales_up : scales_gate);
            a.pr[q].qz = q ? qzeros_up : qzeros_gate;
            a.pr[q].Y = Y;
            a.pr[q].N = N;
            a.pr[q].K = K;
        }
        a.M = M;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        e = launch_block(a, bp, (hipStream_t)stream);
    } else if (M <= kSkinnyMaxM) {
        // one launch: each workgroup holds gate and up tiles of the same columns
        const SkinnyPlan p = plan_skinny_pair(M, N, K);
        SkinnyArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight_gate;
        a.scales = (const uint16_t *)scales_gate;
        a.qz = qzeros_gate;
        a.qw2 = qweight_up;
        a.scales2 = (const uint16_t *)scales_up;
        a.qz2 = qzeros_up;
        a.gated = 1;
        a.M = M;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        a.lmhead = 0;
        e = launch_skinny(a, p, (hipStream_t)stream);
    } else if (const TiledPlan tp = plan_tiled_gated(M, N, K); tp.ok) {
        // large M: one tile kernel, each wave holding gate and up tiles of the same columns
        TiledArgs a{};
        a.X = (const uint16_t *)X;
        a.qw = qweight_gate;
        a.scales = (const uint16_t *)scales_gate;
        a.qz = qzeros_gate;
        a.qw2 = qweight_up;
        a.scales2 = (const uint16_t *)scales_up;
        a.qz2 = qzeros_up;
        a.M = M;
        a.N = N;
        a.K = K;
        a.G = K / kGroup;
        a.Y = Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        e = launch_tiled(a, tp, (hipStream_t)stream);
    } else {
        // mid M (the tiles would not fill the CUs once): the two projections in turn
        // (fp32, into the workspace, each with its own K split), then the activation
        unsigned char *ws = (unsigned char *)workspace;
        const size_t off = gated_gu_offset(M, N, K);
        float *G = (float *)(ws + off), *U = G + (size_t)M * N;
        st = w4a16_linear(X, qweight_gate, scales_gate, qzeros_gate, M, N, K, group, G, W4A16_OUT_F32, workspace,
                          off, stream);
        if (st != W4A16_OK)
            return st;
        st = w4a16_linear(X, qweight_up, scales_up, qzeros_up, M, N, K, group, U, W4A16_OUT_F32, workspace, off,
                          stream);
        if (st != W4A16_OK)
            return st;
        e = launch_silu_mul(G, U, (long long)M * N, Y, y_dtype == W4A16_OUT_F32, (hipStream_t)stream);
    }
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_linear_batch(const w4a16_problem *problems, int count, int M, int group, int y_dtype,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    if (count < 0 || count > W4A16_MAX_BATCH || M < 0)
        return W4A16_ERR_SHAPE;
    if (count > 0 && !problems)
        return W4A16_ERR_NULL;
    size_t need = 0;
    for (int q = 0; q < count; ++q) {
        const w4a16_problem &pr = problems[q];
        const int st = check_dims(M, pr.N, pr.K);
        if (st != W4A16_OK)
            return st;
        if (M == 0 || pr.N == 0)
            continue;
        if (!pr.X || !pr.qweight || !pr.scales || !pr.qzeros || !pr.Y)
            return W4A16_ERR_NULL;
        if (misaligned(pr.X) || misaligned(pr.qweight) || misaligned(pr.scales) || misaligned(pr.qzeros) ||
            misaligned(pr.Y))
            return W4A16_ERR_ALIGN;
        const size_t n = linear_ws(M, pr.N, pr.K);
        need = n > need ? n : need;
    }
    if (M == 0)
        return W4A16_OK;
    if (misaligned(workspace))
        return W4A16_ERR_ALIGN;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return W4A16_ERR_WORKSPACE;

    if (M > kSkinnyMaxM) {
        // large M: the matrix cores are busy within each projection; run them in turn
        for (int q = 0; q < count; ++q) {
            const w4a16_problem &pr = problems[q];
            const int st = w4a16_linear(pr.X, pr.qweight, pr.scales, pr.qzeros, M, pr.N, pr.K, group, pr.Y,
                                        y_dtype, workspace, workspace_bytes, stream);
            if (st != W4A16_OK)
                return st;
        }
        return W4A16_OK;
    }
    if (M >= 2 && M <= 16) {
        // one draft block: the block kernel, every projection's tiles in one launch
        int bn[W4A16_MAX_BATCH], bk[W4A16_MAX_BATCH], nb = 0;
        BlockArgs a{};
        for (int q = 0; q < count; ++q) {
            const w4a16_problem &pr = problems[q];
            if (pr.N == 0)
                continue;
            a.pr[nb].X = (const uint16_t *)pr.X;
            a.pr[nb].qw = pr.qweight;
            a.pr[nb].scales = (const uint16_t *)pr.scales;
            a.pr[nb].qz = pr.qzeros;
            a.pr[nb].Y = pr.Y;
            a.pr[nb].N = pr.N;
            a.pr[nb].K = pr.K;
            bn[nb] = pr.N;
            bk[nb] = pr.K;
            ++nb;
        }
        if (nb == 0)
            return W4A16_OK;
        const BlockPlan bp = plan_block(bn, bk, nb, M);
        if (bp.ok && bp.ws_bytes <= workspace_bytes && (bp.ws_bytes == 0 || workspace)) {
            a.ws = (unsigned char *)workspace;
            a.M = M;
            a.y_f32 = y_dtype == W4A16_OUT_F32;
            return launch_block(a, bp, (hipStream_t)stream) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
        }
    }
    if (M == 1) {
        // two projections of one shape that read the same X (gate and up): the decode
        // kernel with both grids in each wave, up to 40 groups
        int qs[2], nq = 0;
        for (int q = 0; q < count; ++q)
            if (problems[q].N != 0 && nq < 2)
                qs[nq++] = q;
        int live = 0;
        for (int q = 0; q < count; ++q)
            live += problems[q].N != 0 ? 1 : 0;
        if (live == 2) {
            const w4a16_problem &p0 = problems[qs[0]], &p1 = problems[qs[1]];
            const GemvPlan gp = (p0.X == p1.X && p0.N == p1.N && p0.K == p1.K) ? plan_gemv_pair(p0.N, p0.K, 2)
                                                                               : GemvPlan{};
            if (gp.ok) {
                GemvArgs a{};
                a.X = (const uint16_t *)p0.X;
                a.qw = p0.qweight;
                a.scales = (const uint16_t *)p0.scales;
                a.qz = p0.qzeros;
                a.qw2 = p1.qweight;
                a.scales2 = (const uint16_t *)p1.scales;
                a.qz2 = p1.qzeros;
                a.N = p0.N;
                a.K = p0.K;
                a.G = p0.K / kGroup;
                a.Y = p0.Y;
                a.Y2 = p1.Y;
                a.y_f32 = y_dtype == W4A16_OUT_F32;
                return launch_gemv(a, gp, (hipStream_t)stream) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
            }
        }
        // projections that read the same X (q, k and v): the decode kernel, each
        // projection its own run of workgroups in one launch
        GemvArgs a{};
        int gn[W4A16_MAX_BATCH], wg0[W4A16_MAX_BATCH], nm = 0;
        bool same = live >= 1 && live <= kMaxProblemsGemv;
        const w4a16_problem *first = nullptr;
        for (int q = 0; q < count && same; ++q) {
            const w4a16_problem &pr = problems[q];
            if (pr.N == 0)
                continue;
            if (!first)
                first = &pr;
            same = pr.X == first->X && pr.K == first->K;
            a.pr[nm].qw = pr.qweight;
            a.pr[nm].scales = (const uint16_t *)pr.scales;
            a.pr[nm].qz = pr.qzeros;
            a.pr[nm].Y = pr.Y;
            a.pr[nm].N = pr.N;
            gn[nm++] = pr.N;
        }
        if (same) {
            const GemvPlan gp = plan_gemv_multi(gn, first->K, nm, wg0);
            if (gp.ok) {
                for (int q = 0; q < nm; ++q)
                    a.pr[q].wg0 = wg0[q];
                a.count = nm;
                a.X = (const uint16_t *)first->X;
                a.K = first->K;
                a.G = first->K / kGroup;
                a.y_f32 = y_dtype == W4A16_OUT_F32;
                return launch_gemv(a, gp, (hipStream_t)stream) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
            }
        }
    }
    SkinnyMulti mp{};
    int bn[W4A16_MAX_BATCH], bk[W4A16_MAX_BATCH], btw[W4A16_MAX_BATCH], nb = 0;
    for (int q = 0; q < count; ++q)
        if (problems[q].N != 0) {
            bn[nb] = problems[q].N;
            bk[nb] = problems[q].K;
            ++nb;
        }
    balance_multi(bn, bk, nb, M, btw);
    int c = 0;
    for (int q = 0; q < count; ++q) {
        const w4a16_problem &pr = problems[q];
        if (pr.N == 0)
            continue;
        SkinnyArgs &a = mp.args[c];
        a.X = (const uint16_t *)pr.X;
        a.qw = pr.qweight;
        a.scales = (const uint16_t *)pr.scales;
        a.qz = pr.qzeros;
        a.M = M;
        a.N = pr.N;
        a.K = pr.K;
        a.G = pr.K / kGroup;
        a.Y = pr.Y;
        a.y_f32 = y_dtype == W4A16_OUT_F32;
        a.ws = (unsigned char *)workspace;
        a.lmhead = 0;
        mp.plan[c] = plan_skinny_fixed(M, pr.N, pr.K, 0, btw[c]);
        ++c;
    }
    mp.count = c;
    if (c == 0)
        return W4A16_OK;
    const size_t scratch = skinny_multi_scratch(mp, M);
    if (scratch > 0 && (!workspace || workspace_bytes < scratch))
        return W4A16_ERR_WORKSPACE;
    const hipError_t e = launch_skinny_multi(mp, M, workspace ? workspace_bytes : 0, (hipStream_t)stream);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

int w4a16_lmhead_verify(const void *X, const uint32_t *qweight, const void *scales,
                        const uint32_t *qzeros, int M, int N, int K, int group,
                        const int32_t *draft_ids, void *Y_or_null, int y_dtype,
                        int32_t *argmax, int32_t *accept_len,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    if (group != kGroup || (y_dtype != W4A16_OUT_BF16 && y_dtype != W4A16_OUT_F32))
        return W4A16_ERR_UNSUPPORTED;
    int st = check_dims(M, N, K);
    if (st != W4A16_OK)
        return st;
    if (M < 1 || M > 64 || N < 1)
        return W4A16_ERR_SHAPE;
    if (!X || !qweight || !scales || !qzeros || !draft_ids || !argmax || !accept_len || !workspace)
        return W4A16_ERR_NULL;
    if (misaligned(X) || misaligned(qweight) || misaligned(scales) || misaligned(qzeros) ||
        misaligned(Y_or_null) || misaligned(draft_ids) || misaligned(argmax) || misaligned(accept_len) ||
        misaligned(workspace))
        return W4A16_ERR_ALIGN;
    const SkinnyPlan p = plan_skinny(M, N, K, 1);
    if (workspace_bytes < p.ws_bytes)
        return W4A16_ERR_WORKSPACE;
    SkinnyArgs a{};
    a.X = (const uint16_t *)X;
    a.qw = qweight;
    a.scales = (const uint16_t *)scales;
    a.qz = qzeros;
    a.M = M;
    a.N = N;
    a.K = K;
    a.G = K / kGroup;
    a.Y = Y_or_null;
    a.y_f32 = y_dtype == W4A16_OUT_F32;
    a.ws = (unsigned char *)workspace;
    a.lmhead = 1;
    a.draft = draft_ids;
    a.argmax_out = argmax;
    a.accept_out = accept_len;
    return launch_skinny(a, p, (hipStream_t)stream) == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

} // extern "C"
