// calib.hip -- streaming kernels that measure the achievable HBM bandwidth
// on the running GPU (the VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel
// Roofline: What Actually Limits Decode", calibrates its roofline on the
// hardware itself instead of the spec sheet).  Four traffic shapes, one per
// kernel a hot-path kernel is compared with:
//   copy   read n bytes, write n bytes;
//   read   read n bytes (the decode attend's shape: it writes almost nothing);
//   write  write n bytes;
//   mix    read n bytes, write 3n/8 bytes: the 4-bit flush's shape (2 B of
//          fp16 in for 0.5 B of codes + 0.25 B of scale/zero per element).
// Workgroup b owns one contiguous chunk; every thread issues all of its
// 16-byte loads before its first store.  Each kernel uses the cache hints
// that measured fastest for its shape on MI355X (interleaved runs, 2 GiB):
// the nontemporal hint on loads and stores for copy, read and mix (each byte
// is touched once, as in the flush and the attend; plain stores made the mix
// 10% slower and plain loads the read 17% slower), plain stores for the
// write-only kernel (6.0-6.3 TB/s against 5.7-5.8 with the hint).
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

constexpr int kCalibBlock = 256;
constexpr int kCalibVecs = 4;                       // 16-byte vectors per thread per kernel
constexpr int64_t kCalibChunk = int64_t{kCalibBlock} * kCalibVecs;   // vectors per workgroup

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4u ld_nt(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(v4u* p, v4u v) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(kCalibBlock) void calib_copy_kernel(const v4u* __restrict__ src,
                                                                 v4u* __restrict__ dst, int64_t n_vec)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) v[u] = ld_nt(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) st_nt(dst + i, v[u]);
    }
}

// The loads are folded into one word that is stored only when it equals
// `never` (a value the caller picks; a chance match writes one word).
__global__ __launch_bounds__(kCalibBlock) void calib_read_kernel(const v4u* __restrict__ src, int64_t n_vec,
                                                                 uint32_t* __restrict__ sink, uint32_t never)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        v[u] = i < n_vec ? ld_nt(src + i) : v4u{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == never) sink[0] = acc;
}

__global__ __launch_bounds__(kCalibBlock) void calib_write_kernel(v4u* __restrict__ dst, int64_t n_vec,
                                                                  uint32_t pattern)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        if (i < n_vec) dst[i] = v4u{pattern, pattern ^ static_cast<uint32_t>(i), pattern, 0u};
    }
}

// Workgroup b reads source vectors [b*C, (b+1)*C) and writes destination
// vectors [b*3C/8, (b+1)*3C/8): 3 of every 8 threads store their loads'
// fold, C = kCalibChunk.
__global__ __launch_bounds__(kCalibBlock) void calib_mix_kernel(const v4u* __restrict__ src, int64_t n_vec,
                                                                v4u* __restrict__ dst)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCalibChunk + threadIdx.x;
    v4u v[kCalibVecs];
#pragma unroll
    for (int u = 0; u < kCalibVecs; ++u) {
        const int64_t i = base + u * kCalibBlock;
        v[u] = i < n_vec ? ld_nt(src + i) : v4u{0u, 0u, 0u, 0u};
    }
    v4u acc = v[0];
#pragma unroll
    for (int u = 1; u < kCalibVecs; ++u) acc ^= v[u];
    constexpr int kWriters = kCalibBlock * kCalibVecs * 3 / 8 / kCalibVecs;   // threads that store
    constexpr int kStores = kCalibVecs;                                      // vectors each
    if (threadIdx.x < kWriters) {
        const int64_t o = static_cast<int64_t>(blockIdx.x) * (kCalibChunk * 3 / 8) + threadIdx.x;
#pragma unroll
        for (int u = 0; u < kStores; ++u) {
            const int64_t j = o + u * kWriters;
            if (j < n_vec * 3 / 8) st_nt(dst + j, acc);
        }
    }
}

uint32_t grid_of(int64_t n_vec) { return static_cast<uint32_t>((n_vec + kCalibChunk - 1) / kCalibChunk); }

}  // namespace

hipError_t launch_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_copy_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), 0, stream,
                       static_cast<const v4u*>(src), static_cast<v4u*>(dst), n_vec);
    return hipGetLastError();
}

hipError_t launch_calib_read(const void* src, size_t n_bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_read_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), 0, stream,
                       static_cast<const v4u*>(src), n_vec, sink, 0x9E3779B9u);
    return hipGetLastError();
}

hipError_t launch_calib_write(void* dst, size_t n_bytes, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_write_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), 0, stream,
                       static_cast<v4u*>(dst), n_vec, 0x5A5A5A5Au);
    return hipGetLastError();
}

hipError_t launch_calib_mix(const void* src, size_t n_bytes, void* dst, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(n_bytes / 16);
    hipLaunchKernelGGL(calib_mix_kernel, dim3(grid_of(n_vec)), dim3(kCalibBlock), 0, stream,
                       static_cast<const v4u*>(src), n_vec, static_cast<v4u*>(dst));
    return hipGetLastError();
}

}  // namespace kivi
