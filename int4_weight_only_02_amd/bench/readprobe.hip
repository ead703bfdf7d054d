// readprobe.hip -- measurement aid for bench.py (not part of the W4A16 ABI): a plain
// streaming read of `bytes` bytes with 16-byte loads, four per thread, 256 threads per
// workgroup, the whole buffer in flight.  Its time for the byte count of a launch is
// the ceiling a kernel that only reads those bytes reaches on the same GPU, and is
// reported beside each small-M launch.
//   int w4a16_bench_read(const void *p, size_t bytes, void *sink, void *stream)
// p: device buffer (16-byte aligned), bytes a multiple of 16; sink: 4 device bytes that
// receive a value only if the data XOR to an improbable constant (keeps the loads).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kU = 4;

__global__ __launch_bounds__(256) void read_kernel(const uint4 *p, size_t n16, uint32_t *sink)
{
    const size_t i = (size_t)blockIdx.x * 256 * kU + threadIdx.x;
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
        v[u] = i + (size_t)u * 256 < n16 ? p[i + (size_t)u * 256] : make_uint4(0, 0, 0, 0);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u)
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9E3779B9u)
        sink[0] = acc;
}

} // namespace

extern "C" int w4a16_bench_read(const void *p, size_t bytes, void *sink, void *stream)
{
    if (!p || !sink || (bytes & 15) != 0 || ((uintptr_t)p & 15) != 0)
        return 1;
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return 0;
    const size_t grid = (n16 + 256 * kU - 1) / (256 * kU);
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const uint4 *)p, n16,
                       (uint32_t *)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
