// calib.hip -- streaming copy used to measure the achievable HBM bandwidth
// ceiling on the running GPU (the VeloxQuant-MLX "Benchmarks" page, "KV-Cache
// Kernel Roofline: What Actually Limits Decode", calibrates its roofline on
// the hardware itself instead of the spec sheet).  Each thread moves 16-byte
// vectors of one contiguous 8 KiB chunk per workgroup.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kCopyPerThread = 2;                  // 16-byte vectors per thread
constexpr int kCopyBlock = 256;

// Block b copies the contiguous vectors [b*512, (b+1)*512): each thread issues
// both loads before its stores.  (On MI355X this contiguous-chunk form beat
// grid-stride loops by ~25% in a sweep of unroll depth and grid size.)
__global__ __launch_bounds__(kCopyBlock) void calib_copy_kernel(const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int64_t n_vec)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyBlock * kCopyPerThread + threadIdx.x;
    uint4 v[kCopyPerThread];
#pragma unroll
    for (int u = 0; u < kCopyPerThread; ++u) {
        const int64_t i = base + u * kCopyBlock;
        if (i < n_vec) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyPerThread; ++u) {
        const int64_t i = base + u * kCopyBlock;
        if (i < n_vec) dst[i] = v[u];
    }
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    const int64_t per_block = kCopyBlock * kCopyPerThread;
    const int64_t blocks = (n_vec + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(calib_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kCopyBlock), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n_vec);
    return hipGetLastError();
}

}  // namespace kivi
