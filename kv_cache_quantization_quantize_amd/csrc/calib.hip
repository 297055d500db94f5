// calib.hip -- streaming copy used to measure the achievable HBM bandwidth
// ceiling on the running GPU (the VeloxQuant-MLX "Benchmarks" page, "KV-Cache
// Kernel Roofline: What Actually Limits Decode", calibrates its roofline on
// the hardware itself instead of the spec sheet).  Each thread moves 16-byte
// vectors; the grid is sized to fill every CU several times over.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void calib_copy_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t n_vec)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * stride < n_vec; i += kCopyUnroll * stride) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < n_vec; i += stride) dst[i] = src[i];
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    int64_t blocks = (n_vec + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(calib_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n_vec);
    return hipGetLastError();
}

}  // namespace kivi
