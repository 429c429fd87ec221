// kvq_probe.hip -- bandwidth probe: a streaming read and a streaming copy of
// a device buffer, the measured reference the decode kernels' HBM rates are
// compared with (beside the 8 TB/s HBM3E specification).
//
// Each workgroup streams one contiguous chunk of the buffer with 16-byte
// vectors, eight loads per thread in flight (on MI355X this reads about
// 6.2 TB/s, where a grid-stride loop over the whole buffer reaches 5.3-5.9);
// the read kernel folds what it reads into one word per thread and stores it
// only when it matches a value the data never produces, so no load can be
// dropped and almost nothing is written.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr unsigned kProbeGrid = 4096;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4 *__restrict__ src,
                                                                   size_t n, uint32_t *__restrict__ sink,
                                                                   uint32_t never) {
    const size_t chunk = (n + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * chunk, end = beg + chunk < n ? beg + chunk : n;
    size_t i = beg + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
        uint4 a[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) a[u] = src[i + u * kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
    }
    for (; i < end; i += kProbeThreads) {
        const uint4 a = src[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (x == never) sink[0] = x;
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4 *__restrict__ src,
                                                                   uint4 *__restrict__ dst, size_t n) {
    const size_t chunk = (n + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * chunk, end = beg + chunk < n ? beg + chunk : n;
    size_t i = beg + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
        uint4 a[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) a[u] = src[i + u * kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) dst[i + u * kProbeThreads] = a[u];
    }
    for (; i < end; i += kProbeThreads) dst[i] = src[i];
}

}  // namespace

hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 16;
    const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>(kProbeGrid, n / kProbeThreads));
    if (mode == 0)
        hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, st,
                           static_cast<const uint4 *>(src), n, static_cast<uint32_t *>(dst),
                           0x9e3779b9u);
    else
        hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(kProbeThreads), 0, st,
                           static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace kvq
