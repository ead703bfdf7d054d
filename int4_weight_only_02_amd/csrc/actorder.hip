// actorder.hip -- GPTQ act-order ("desc_act") support for the packed grid (gfx950).
//
// With act-order, column k of the weight belongs to group g_idx[k], so a group is a
// set of columns rather than a run of 128 (the pages' drafter is GPTQ INT4 with
// groups of 128: Pith review, Assumptions & free parameters; act-order is GPTQ's
// optional column ordering).  Permuting the K axis so that each group's columns are
// consecutive turns it back into the plain grid: the codes are gathered once when
// packing, and the activations are gathered on every call, after which the ordinary
// kernels run unchanged (a contraction does not depend on the order of k).
//   perm[j] = the j-th column in (group, column) order, so g_idx[perm[j]] = j / 128
//   codes'[n][j] = codes[n][perm[j]],   X'[m][j] = X[m][perm[j]]
#include "common.h"
#include "kernels.h"

namespace w4a16 {

namespace {

// dst[r][j .. j+7] = src[r][perm[j .. j+7]] for one 8-column block per thread:
// perm is read as two 16-byte loads, the 8 elements are gathered (rows are short
// and stay in L2) and written as one contiguous 8- or 16-byte store
template <typename T>
__global__ __launch_bounds__(256) void gather_k_kernel(const T *src, const int32_t *perm, int rows, int K, T *dst)
{
    // rows * K <= 2^31 - 256: block indices fit in 32 bits (a 32-bit division per block)
    const uint32_t KB = (uint32_t)(K / 8);
    const uint32_t blocks = (uint32_t)rows * KB;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < blocks; i += gridDim.x * 256u) {
        const int r = (int)(i / KB);
        const int j0 = (int)(i - (uint32_t)r * KB) * 8;
        const u32x4_t p0 = *(const u32x4_t *)(perm + j0);
        const u32x4_t p1 = *(const u32x4_t *)(perm + j0 + 4);
        const T *row = src + (size_t)r * K;
        const uint32_t last = (uint32_t)K - 1u; // an index past the row (not a permutation) stays in it
        T v[8] = {row[min(p0.x, last)], row[min(p0.y, last)], row[min(p0.z, last)], row[min(p0.w, last)],
                  row[min(p1.x, last)], row[min(p1.y, last)], row[min(p1.z, last)], row[min(p1.w, last)]};
        T *out = dst + (size_t)r * K + j0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            out[e] = v[e];
    }
}

// qweight[n][w] = codes[n][perm[8w + j]] in nibble j (the layout of w4a16_pack, on
// the permuted columns): one packed word per thread
__global__ __launch_bounds__(256) void pack_codes_perm_kernel(const uint8_t *codes, const int32_t *perm, int N,
                                                              int K, uint32_t *qweight)
{
    const uint32_t KW = (uint32_t)(K / 8);
    const uint32_t words = (uint32_t)N * KW; // N * K <= 2^31 - 256
    const uint32_t last = (uint32_t)K - 1u;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < words; i += gridDim.x * 256u) {
        const int n = (int)(i / KW);
        const int j0 = (int)(i - (uint32_t)n * KW) * 8;
        const u32x4_t p0 = *(const u32x4_t *)(perm + j0);
        const u32x4_t p1 = *(const u32x4_t *)(perm + j0 + 4);
        const uint8_t *row = codes + (size_t)n * K;
        const uint32_t idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            word |= (uint32_t)(row[min(idx[j], last)] & 15u) << (4 * j);
        qweight[i] = word;
    }
}

} // namespace

hipError_t launch_pack_perm(const uint8_t *codes, const uint8_t *zeros, const int32_t *perm, int N, int K, int G,
                            uint32_t *qweight, uint32_t *qzeros, hipStream_t stream)
{
    const long long words = (long long)N * (K / 8);
    long long grid = (words + 255) / 256;
    if (grid > 8192)
        grid = 8192;
    if (grid > 0) {
        hipLaunchKernelGGL(pack_codes_perm_kernel, dim3((unsigned)grid), dim3(256), 0, stream, codes, perm, N, K,
                           qweight);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return launch_pack_zeros(zeros, N, G, qzeros, stream);
}

bool actorder_perm_host(const int32_t *g_idx, int K, int group, int32_t *perm)
{
    const int G = K / group;
    // counting sort by group, stable in k: the start of each group, then placement
    int *count = new int[G + 1]();
    for (int k = 0; k < K; ++k) {
        const int g = g_idx[k];
        if (g < 0 || g >= G) {
            delete[] count;
            return false;
        }
        ++count[g + 1];
    }
    bool ok = true;
    for (int g = 0; g < G; ++g)
        ok = ok && count[g + 1] == group; // every group holds exactly `group` columns
    if (ok) {
        for (int g = 0; g < G; ++g)
            count[g + 1] += count[g];
        for (int k = 0; k < K; ++k)
            perm[count[g_idx[k]]++] = k;
    }
    delete[] count;
    return ok;
}

hipError_t launch_gather_k(const void *src, const int32_t *perm, int rows, int K, int elem_bytes, void *dst,
                           hipStream_t stream)
{
    const long long blocks8 = (long long)rows * (K / 8);
    long long grid = (blocks8 + 255) / 256;
    if (grid > 8192)
        grid = 8192;
    if (grid == 0)
        return hipSuccess;
    if (elem_bytes == 1)
        hipLaunchKernelGGL(gather_k_kernel<uint8_t>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const uint8_t *)src, perm, rows, K, (uint8_t *)dst);
    else
        hipLaunchKernelGGL(gather_k_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const uint16_t *)src, perm, rows, K, (uint16_t *)dst);
    return hipGetLastError();
}

} // namespace w4a16
