// Measurement helper (not on the product path): a plain streaming read of a
// device buffer, 16 bytes per lane per load, every load of a thread issued
// before any is used.  Timed on cold buffers beside the GEMM kernels, it
// gives the read rate a single launch of the same size can reach on this
// GPU, which the GEMM and expert-bank figures are compared against.
#include "../../include/mxfp4_probe.h"
#include "device.h"

namespace mx {

namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *p, int64_t n16,
                                                          uint32_t *sink, uint32_t match)
{
    const int64_t base = ((int64_t)blockIdx.x * U) * 256 + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int64_t k = base + (int64_t)i * 256;
        v[i] = k < n16 ? p[k] : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < U; ++i)
        acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    // `match` comes from the host, so the compiler must keep every load;
    // a thread whose XOR happens to equal it writes the 4-byte sink
    if (acc == match)
        sink[0] = acc;
}

} // namespace

} // namespace mx

extern "C" int mxfp4_probe_read(const void *buf, int64_t bytes, int loads_per_thread,
                                void *sink, void *stream)
{
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0 ||
        ((uintptr_t)sink % 4) != 0)
        return -1;
    const int64_t n16 = bytes / 16;
    const int U = loads_per_thread;
    if (U != 4 && U != 8 && U != 16)
        return -1;
    const int64_t per_wg = (int64_t)U * 256;
    const int64_t blocks = (n16 + per_wg - 1) / per_wg;
    if (blocks > 0x7FFFFFFF)
        return -1;
    const auto *p = static_cast<const mx::u32x4 *>(buf);
    auto *s = static_cast<uint32_t *>(sink);
    hipStream_t st = (hipStream_t)stream;
    if (U == 4)
        hipLaunchKernelGGL(mx::stream_read_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, p,
                           n16, s, 0x9E3779B9u);
    else if (U == 8)
        hipLaunchKernelGGL(mx::stream_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, p,
                           n16, s, 0x9E3779B9u);
    else
        hipLaunchKernelGGL(mx::stream_read_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st,
                           p, n16, s, 0x9E3779B9u);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
